"""Shared helpers of the GPU parity tests (comparison rules and tolerances)."""

import numpy as np
import torch

import oracle as O
import workloads as W

# Tolerances on the relative L2 error ||gpu - oracle|| / ||oracle||.
TOL = {"fp32": 1e-5, "bf16": 5e-3, "fp8": 5e-2}
# fp8 code rule: at most this fraction of the quantized codes of a forward one
# E4M3 step away from the oracle's, none further.
CODE_ONE_STEP_MAX = 1e-3
# Per-tensor guard for the activation codes alone. The gfx950 fp8 MFMA sums
# its 64 products per instruction with ~17 significant bits (probe: error up
# to 1.4e-4 of sum|p| at K = 64, against 2e-8 for the bf16 MFMA), which moves
# ~1% of the bf16 roundings of h1 and through them 0.1-0.2% of the act codes.
ACT_CODE_ONE_STEP_MAX = 5e-3


def dev():
    return torch.device("cuda:0")


def to_dev(d):
    return {k: v.to(dev()) for k, v in d.items()}


def f64(t):
    return W.to_f64(t)


def codes_np(t):
    return t.detach().to("cpu").numpy().astype(np.uint8)


def code_ordinal(c):
    c = np.asarray(c).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def code_steps(got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    return np.abs(code_ordinal(got) - code_ordinal(ref))


def check_codes(got, ref, label="", limit=CODE_ONE_STEP_MAX):
    """E4M3 code rule on one tensor: <= limit of the codes one step away, none
    two or more. Returns (number one step away, number of codes)."""
    d = code_steps(got, ref)
    n1 = int(np.count_nonzero(d == 1))
    dmax = int(d.max()) if d.size else 0
    assert dmax <= 1, f"{label}: codes differ by {dmax} steps"
    assert n1 <= limit * max(d.size, 1), f"{label}: {n1 / d.size:.3%} of codes one step away"
    return n1, d.size


def check_codes_combined(pairs):
    """The fp8 forward's code rule: over all quantized tensors together
    (normalised input, both kernels, activation), <= 0.1% of the codes one
    step away and none further. pairs: [(label, got, ref, per-tensor limit)]."""
    ones, total = 0, 0
    for label, got, ref, limit in pairs:
        n1, n = check_codes(got, ref, label, limit)
        print(f"  {label}: {n1} of {n} codes one step away", flush=True)
        ones, total = ones + n1, total + n
    assert ones <= CODE_ONE_STEP_MAX * total, f"{ones / total:.3%} of all codes one step away"
    return ones / max(total, 1)


def rel(got, ref):
    return O.rel_l2(np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64))


def assert_rel(got, ref, tol, label=""):
    e = rel(got, ref)
    assert e <= tol, f"{label}: rel_l2 {e:.3e} > {tol:.1e}"
    return e
