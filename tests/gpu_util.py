"""Shared helpers of the GPU parity tests (comparison rules and tolerances)."""

import numpy as np
import torch

import oracle as O
import workloads as W

# Tolerances on the relative L2 error ||gpu - oracle|| / ||oracle||.
TOL = {"fp32": 1e-5, "bf16": 5e-3, "fp8": 5e-2}
# fp8 code rule: at most this fraction of codes one E4M3 step away, none further.
CODE_ONE_STEP_MAX = 1e-3


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


def check_codes(got, ref, label=""):
    """E4M3 code rule: <= 0.1% of codes one step away, none two or more.
    Returns (fraction one step away, max steps)."""
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(code_ordinal(got) - code_ordinal(ref))
    frac1 = float(np.mean(d == 1)) if d.size else 0.0
    dmax = int(d.max()) if d.size else 0
    assert dmax <= 1, f"{label}: codes differ by {dmax} steps"
    assert frac1 <= CODE_ONE_STEP_MAX, f"{label}: {frac1:.3%} of codes one step away"
    return frac1, dmax


def rel(got, ref):
    return O.rel_l2(np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64))


def assert_rel(got, ref, tol, label=""):
    e = rel(got, ref)
    assert e <= tol, f"{label}: rel_l2 {e:.3e} > {tol:.1e}"
    return e
