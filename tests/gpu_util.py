"""Shared helpers of the GPU parity tests (comparison rules and tolerances)."""

import numpy as np
import torch

import oracle as O
import workloads as W
from tolerances import U_BF16

# Tolerances on the relative L2 error ||gpu - oracle|| / ||oracle||.
TOL = {"fp32": 1e-5, "bf16": 5e-3, "fp8": 5e-2}
# fp8 code rule, per quantized tensor: at most this fraction of its codes one
# E4M3 step away from the oracle's, none further.
CODE_ONE_STEP_MAX = 1e-3
# A GPU code may sit one step from the oracle's without any upstream
# difference only when the value being encoded lies this close (relative) to
# the midpoint between the two codes: the GPU evaluates the activation in fp32
# (exp2 and reciprocal, a few fp32 ulps) where the oracle works in fp64.
NEAR_TIE_REL = 2.0 ** -19
# Per-element guard: deviations beyond this many standard deviations of the
# error model fail (8 sigma: ~1e-15 per element for a normal model).
GUARD_SIGMAS = 8.0

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


# Largest |f'(x)| of each activation (the bound on how far a change of h moves
# f(h)): GELU (both forms) 1.129 near x = 1.5, SiLU 1.0998 near x = 2.4.
ACT_LIPSCHITZ = {"gelu": 1.13, "gelu_erf": 1.13, "silu": 1.1, "relu": 1.0, "linear": 1.0}


def e4m3_round_interval(codes):
    """The interval of values that round to each code: from the midpoint with
    its lower neighbour on the signed E4M3 grid to the midpoint with its upper
    neighbour (+-inf beyond +-448, where values saturate)."""
    c = np.asarray(codes).astype(np.int64)
    mag, neg = c & 0x7F, (c & 0x80) != 0
    v = O.e4m3_decode(mag)
    away = np.where(mag >= 0x7E, np.inf, O.e4m3_decode(np.minimum(mag + 1, 0x7E)))
    toward = np.where(mag == 0, -O.e4m3_decode(np.ones_like(mag)), O.e4m3_decode(np.maximum(mag - 1, 0)))
    hi_mag, lo_mag = 0.5 * (v + away), 0.5 * (v + toward)     # toward zero, then away from it
    lo = np.where(neg, -hi_mag, lo_mag)
    hi = np.where(neg, -lo_mag, hi_mag)
    return lo, hi


def act_code_flips(got_codes, ref_codes, got_h1, ref_h1, ref_act, scale, scale_ratio, activation_type):
    """Checks the activation codes of an fp8 forward against the oracle's. The
    activation is evaluated from the bf16 h1 (GEMM1 + bias1), so where h1
    itself differs (the GEMM's summation, or a normalised-input code one step
    away; for a gated pair either half) the scaled activation may move by at
    most scale x L x |dh1| (L = the activation's Lipschitz bound; gated
    f(a) b: L |da| |b| + |f(a)| |db| + L |da| |db|). Each GPU code must be the
    correct rounding of a value within that distance of the oracle's scaled
    activation (plus NEAR_TIE_REL of it and the relative difference of the
    two scales: the GPU evaluates f in fp32). Near zero the E4M3 grid is
    fine, so such a code may sit several steps away; where h1 agrees only a
    tie can move it, by one step.
    Returns (codes differing, of them one step away, of them where h1 differs,
    of them at ties where h1 agrees)."""
    got_codes, ref_codes = np.asarray(got_codes), np.asarray(ref_codes)
    diff = got_codes != ref_codes
    idx = np.nonzero(diff)
    L = ACT_LIPSCHITZ[activation_type[0]]
    dh = np.abs(np.asarray(got_h1) - np.asarray(ref_h1))
    if len(activation_type) == 2:
        f = dh.shape[1] // 2
        ra = np.asarray(ref_h1)[:, :f][idx]
        rb = np.asarray(ref_h1)[:, f:][idx]
        da, db = dh[:, :f][idx], dh[:, f:][idx]
        fa = O.act_fn(activation_type[0], ra)
        move = L * da * np.abs(rb) + np.abs(fa) * db + L * da * db
        h1_moved = (da > 0) | (db > 0)
    else:
        move = L * dh[idx]
        h1_moved = dh[idx] > 0
    v = np.asarray(ref_act)[idx] * scale
    allow = scale * move + (NEAR_TIE_REL + abs(scale_ratio - 1.0)) * np.abs(v)
    lo, hi = e4m3_round_interval(got_codes[idx])
    bad = (v + allow < lo) | (v - allow > hi) | ((got_codes[idx] & 0x7F) == 0x7F)   # 0x7F / 0xFF: NaN
    if bad.any():
        k = int(np.argmax(bad))
        at = tuple(int(i[k]) for i in idx)
        raise AssertionError(f"{int(bad.sum())} act codes not a rounding of a value the h1 difference allows, "
                             f"e.g. at {at}: code {int(got_codes[at])} (rounds [{lo[k]!r}, {hi[k]!r}]) vs oracle "
                             f"{int(ref_codes[at])}, scaled value {v[k]!r} +- {allow[k]!r}")
    steps = code_steps(got_codes[idx], ref_codes[idx])
    assert np.all((steps <= 1) | h1_moved), "a code more than one step away where h1 agrees"
    return int(diff.sum()), int(np.count_nonzero(steps == 1)), int(h1_moved.sum()), int((~h1_moved).sum())


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (8 significant bits, fp32 exponent range)."""
    _, ex = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.ldexp(1.0, np.maximum(ex - 1, -126) - 7)


def check_elementwise(got, ref, sigma_rel, label="", extra=None):
    """Per-element guard next to the rel-L2 check: |got - ref| <= one bf16 ulp
    of ref (the output rounding) + GUARD_SIGMAS * sigma_rel * rms(ref) (the
    propagated error, whose per-element standard deviation is sigma_rel times
    the tensor's rms under the error model the caller states) + extra (an
    optional per-element allowance). A mis-stored 16-byte chunk, a wrong row
    or column of a tile, moves values by about rms(ref) and fails."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    lim = bf16_ulp(ref) + GUARD_SIGMAS * sigma_rel * rms
    if extra is not None:
        lim = lim + extra
    err = np.abs(got - ref)
    bad = ~(err <= lim)
    assert not bad.any(), (f"{label}: {int(bad.sum())} elements beyond the guard, worst at "
                           f"{np.unravel_index(np.argmax(err - lim), err.shape)}: got "
                           f"{got.flat[np.argmax(err - lim)]!r} ref {ref.flat[np.argmax(err - lim)]!r}")
    return float(np.max(err / np.maximum(rms, 1e-300))) if err.size else 0.0


def rel(got, ref):
    return O.rel_l2(np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64))


def assert_rel(got, ref, tol, label=""):
    e = rel(got, ref)
    assert e <= tol, f"{label}: rel_l2 {e:.3e} > {tol:.1e}"
    return e


# Bounds on the fraction of fp8-forward elements that differ from the oracle,
# measured on MI355X with a margin: the GPU's GEMM1 sums the E4M3 products with
# the fp8 MFMA's own internal precision, so 1.08-1.24% of the bf16 roundings
# of h1 (300 to 8192 rows) land on the neighbouring value; the activation
# codes computed from those h1 values follow in 0.088-0.100% (GELU) and
# 0.15-0.16% (SwiGLU) of the codes, every one where h1 differs.
H1_DIFF_MAX = 2e-2
ACT_CODE_DIFF_MAX = 3e-3
# The fp8 MFMA's summation error relative to the sum of the magnitudes of the
# products it adds, sum_k |a_k b_k|: measured at most 1.9e-6 at K = 4096
# (GEMM1 at 2048 x 4096 -> 16384, against the exact fp64 sum of the same
# codes) and about 4.5e-6 at K = 272..512 (values near zero in the small
# parity shapes); bound about 2x the larger. Each matrix instruction's error
# scales with the largest of its 64 products, so this form holds for GEMM1's
# operands (normalised input and kernel codes, no heavy tail); with the
# activation's skewed codes as an operand (GEMM2) it reached 2.2e-5 at K = 400
# (test_fp8_gemm_summation_error measures both forms).
H1_ACC_REL = 8e-6


def check_fp8_forward(q, saved, y, o, activation_type, label=""):
    """The fp8 forward against the oracle's emulation of the same roundings:
    the four metas, the weight codes (bit-exact), the normalised-input codes
    (code rule of their own), h1 (each value within one bf16 step, fraction of
    differing values bounded), the activation codes (every one-step difference
    traced to an h1 difference or a tie, fraction bounded) and y (rel-L2 and
    the per-element guard). Returns a dict of the measured fractions."""
    for key, meta in (("x_meta", q.x), ("w1_meta", q.w1), ("w2_meta", q.w2), ("act_meta", q.act)):
        got, ref = meta.values(), o[key]
        assert abs(got["amax"] - ref["amax"]) <= 1e-5 * ref["amax"], key
        assert got["scale"] == float(np.float32(448.0) / np.float32(got["amax"])), key
    # the kernels' codes are computed from exact inputs: bit-exact
    w1q, w2q = codes_np(saved["w1q_t"]).T, codes_np(saved["w2q_t"]).T
    assert np.array_equal(w1q, o["w1q"]), "w1 codes"
    assert np.array_equal(w2q, o["w2q"]), "w2 codes"
    nx, sx = check_codes(codes_np(saved["xq"]), o["xq"], "xq")
    h1 = f64(saved["h1"])
    assert_rel(h1, o["h1"], TOL["bf16"], "h1")
    dh = np.abs(h1 - o["h1"])
    # each h1 value: its bf16 step, the GEMM's summation error (H1_ACC_REL of
    # sum |products|), and the shift of its row from normalised-input codes
    # one step away from the oracle's (|code difference| x |kernel1 column|)
    sxw = o["x_meta"]["scale_inv"] * o["w1_meta"]["scale_inv"]
    a_abs, b_abs = np.abs(O.e4m3_decode(o["xq"])), np.abs(O.e4m3_decode(o["w1q"]))
    lim = bf16_ulp(o["h1"]) + H1_ACC_REL * sxw * (a_abs @ b_abs)
    del a_abs
    xq_gpu = codes_np(saved["xq"])
    rf = np.nonzero(np.any(xq_gpu != o["xq"], axis=1))[0]
    if rf.size:
        dx = np.abs(O.e4m3_decode(xq_gpu[rf]) - O.e4m3_decode(o["xq"][rf]))
        lim[rf] += sxw * (dx @ b_abs)
    # the GPU's scales may differ from the oracle's in the last bits of the amaxes
    ratio = (q.x.values()["scale_inv"] * q.w1.values()["scale_inv"]) / sxw
    lim += 2.0 * abs(ratio - 1.0) * np.abs(o["h1"])
    far = dh > lim
    if far.any():
        for i in np.argsort((dh - lim).ravel())[-4:]:
            print(f"  h1 far: idx {np.unravel_index(i, dh.shape)} gpu {h1.flat[i]!r} oracle {o['h1'].flat[i]!r} "
                  f"diff {dh.flat[i]:.3e} lim {lim.flat[i]:.3e} ulp {bf16_ulp(o['h1'].flat[i]):.3e}", flush=True)
    assert not far.any(), (f"{int(far.sum())} h1 values beyond one bf16 step plus the summation and code-flip "
                           f"allowance, e.g. at {np.unravel_index(np.argmax(dh - lim), dh.shape)}")
    del lim, b_abs
    h1_frac = float(np.count_nonzero(dh)) / dh.size
    assert h1_frac <= H1_DIFF_MAX, f"{h1_frac:.3%} of h1 differs"
    am = q.act.values()
    nd, n1, by_h1, ties = act_code_flips(codes_np(saved["actq"]), o["actq"], h1, o["h1"], o["act"],
                                         o["act_meta"]["scale"], am["scale"] / o["act_meta"]["scale"],
                                         activation_type)
    act_frac = nd / o["actq"].size
    assert act_frac <= ACT_CODE_DIFF_MAX, f"{act_frac:.3%} of act codes differ"
    e = assert_rel(f64(y), o["y"], TOL["fp8"], "y")
    # y depends on the codes alone: a code one E4M3 step away moves its term by
    # at most 2^-3 of the value, so the propagated error has a relative
    # standard deviation of about sqrt(p * 2^-6) for a fraction p of such codes,
    # beside the output's own bf16 rounding
    p = act_frac + nx / max(sx, 1)
    check_elementwise(f64(y), o["y"], 1.5 * np.sqrt(U_BF16 ** 2 + p * 2.0 ** -6), f"{label} y")
    out = {"xq_one_step": nx / max(sx, 1), "h1_diff": h1_frac, "act_diff": act_frac, "act_one_step": n1,
           "act_by_h1": by_h1, "act_ties": ties, "y_rel_l2": e}
    print(f"  {label}: " + ", ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                    for k, v in out.items()), flush=True)
    return out
