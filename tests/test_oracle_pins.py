"""Pins of the fp64 oracle against things other than itself: invariants,
closed forms, brute force, exhaustive codec checks and library routines.

Each test is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, a swapped operand or half, an off-by-one exponent) fails it.
"""

import math
import itertools

import numpy as np
import pytest
import torch

import oracle as O
from conftest import read_golden

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- rounding

def test_bf16_round_matches_torch_cast():
    v = np.concatenate([
        RNG.standard_normal(20000) * 10.0 ** RNG.integers(-30, 30, 20000),
        RNG.standard_normal(2000) * 1e-39,            # fp32 subnormal range
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(v.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even significand (1).
    assert O.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even).
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.bf16_round(-(1.0 + 2.0 ** -8 + 2.0 ** -30)) == -(1.0 + 2.0 ** -7)


def test_fl32_matches_numpy_float32():
    v = RNG.standard_normal(1000) * 1e3
    assert np.array_equal(O.fl32(v), v.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- E4M3 codec

def test_e4m3_decode_spec_points():
    for code, val in read_golden("e4m3_points.txt"):
        got = O.e4m3_decode(np.array([int(code, 16)]))[0]
        assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got, val)
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_e4m3_decode_is_strictly_increasing_and_complete():
    vals = O.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(vals) > 0)
    assert vals[-1] == 448.0 and len(vals) == 127
    # brute force of the value set: subnormals k*2^-9 and normals (1+m/8)*2^(e-7)
    expect = sorted({k * 2.0 ** -9 for k in range(8)} |
                    {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)
                     if not (e == 15 and m == 7)})
    assert np.array_equal(vals, np.array(expect))


def test_e4m3_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes.astype(np.uint8))


def test_e4m3_midpoints_go_to_even_code():
    pos = O.e4m3_decode(np.arange(0, 0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    got = O.e4m3_encode(mids).astype(int)
    lo = np.arange(0, 0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)  # code parity == mantissa LSB parity
    assert np.array_equal(got, expect)
    # just off the midpoint goes to the nearer neighbour
    eps = (pos[1:] - pos[:-1]) * 1e-6
    assert np.array_equal(O.e4m3_encode(mids - eps).astype(int), lo)
    assert np.array_equal(O.e4m3_encode(mids + eps).astype(int), lo + 1)
    # negative side mirrors with the sign bit
    assert np.array_equal(O.e4m3_encode(-mids).astype(int), expect | 0x80)


def test_e4m3_saturates():
    v = np.array([448.0, 449.0, 464.0, 465.0, 1e6, np.inf, -449.0, -1e30])
    assert list(O.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    # between 416 and 448 rounds normally
    assert O.e4m3_encode(np.array([431.9, 432.1]))[0] == 0x7D
    assert O.e4m3_encode(np.array([432.1]))[0] == 0x7E


def test_e4m3_matches_torch_cast_in_range():
    v = (RNG.standard_normal(200000) * 2.0 ** RNG.integers(-12, 9, 200000))
    v = np.clip(v, -448, 448)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn)
    ref = t.view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v.astype(np.float32).astype(np.float64)), ref)


def test_e4m3_fp32_fast_path_matches_definition():
    pos = O.e4m3_decode(np.arange(0, 0x7F))
    m32 = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([pos, m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                        RNG.standard_normal(100000) * 2.0 ** RNG.integers(-14, 11, 100000),
                        [0.0, -0.0, 448.0, 449.0, 1e6, 1e-12, -1e-12]]).astype(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(O.e4m3_encode_fp32(v), O.e4m3_encode(v.astype(np.float64)))


def test_e4m3_encode_is_nearest_by_brute_force():
    table = O.e4m3_decode(np.arange(0, 0x7F))
    v = np.abs(RNG.standard_normal(3000)) * 2.0 ** RNG.integers(-11, 9, 3000)
    v = v[v < 448]
    got = O.e4m3_decode(O.e4m3_encode(v))
    d = np.abs(v[:, None] - table[None, :])
    best = d.min(axis=1)
    assert np.allclose(np.abs(got - v), best, rtol=0, atol=0)


# ---------------------------------------------------------------- current scaling

def test_current_scaling_closed_forms():
    m = O.current_scaling(np.array([1.0, -3.5, 2.0]))
    assert m == {"amax": 3.5, "scale": 128.0, "scale_inv": 1.0 / 128.0}
    z = O.current_scaling(np.zeros(5))
    assert z["amax"] == 0.0 and z["scale"] == 1.0 and z["scale_inv"] == 1.0
    # scale is the fp32 quotient 448/amax, correctly rounded
    t = np.array([0.3])
    assert O.current_scaling(t)["scale"] == float(np.float32(448.0) / np.float32(0.3))


def test_quantize_amax_element_maps_to_448():
    for seed in range(20):
        t = np.random.default_rng(seed).standard_normal(257) * (seed + 0.37)
        q, m = O.quantize(t)
        i = int(np.argmax(np.abs(t)))
        assert q[i] & 0x7F == 0x7E
        assert np.all(np.abs(O.e4m3_decode(q)) <= 448)
        # dequantized values are within half a step of t
        deq = O.dequantize(q, m)
        rel = np.abs(deq - t) / np.maximum(np.abs(t), 2.0 ** -6 / m["scale"])
        assert rel.max() <= 2.0 ** -4 * 1.0001


# ---------------------------------------------------------------- normalization

def _ln_brute(x, g, b, eps):
    out = []
    for row in x:
        n = len(row)
        mu = math.fsum(row) / n
        var = math.fsum((v - mu) ** 2 for v in row) / n
        out.append([(v - mu) / math.sqrt(var + eps) * gi + bi for v, gi, bi in zip(row, g, b)])
    return np.array(out)


def test_layernorm_brute_force():
    x = RNG.standard_normal((5, 24)) * 3 + 1
    g = RNG.standard_normal(24)
    b = RNG.standard_normal(24)
    y, mu, rs = O.layernorm(x, g, b, 1e-5)
    assert np.allclose(y, _ln_brute(x, g, b, 1e-5), rtol=1e-13, atol=1e-13)
    assert np.allclose(mu, x.mean(axis=1))


def test_layernorm_invariants_closed_form_variance():
    x = RNG.standard_normal((16, 128)) * RNG.uniform(0.01, 5, (16, 1)) + RNG.uniform(-3, 3, (16, 1))
    for eps in (1e-6, 1e-5, 1e-1):
        y, _, _ = O.layernorm(x, np.ones(128), np.zeros(128), eps)
        var = x.var(axis=1)
        assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
        assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_rmsnorm_invariant_and_brute_force():
    x = RNG.standard_normal((16, 64)) * 2 + 0.5
    for eps in (1e-6, 0.3):
        y, rs = O.rmsnorm(x, np.ones(64), eps)
        ms = (x * x).mean(axis=1)
        assert np.allclose((y * y).mean(axis=1), ms / (ms + eps), rtol=1e-12)
    g = RNG.standard_normal(64)
    y, _ = O.rmsnorm(x[:2], g, 1e-6)
    brute = [[v / math.sqrt(math.fsum(u * u for u in row) / 64 + 1e-6) * gi for v, gi in zip(row, g)]
             for row in x[:2]]
    assert np.allclose(y, brute, rtol=1e-13)


def test_rmsnorm_ignores_shift_layernorm_uses_it():
    x = RNG.standard_normal((4, 32))
    g, b = RNG.standard_normal(32), RNG.standard_normal(32)
    y0, _, _ = O.normalize(x, g, np.zeros(32), "layernorm", 1e-6, False)
    y1, _, _ = O.normalize(x, g, b, "layernorm", 1e-6, False)
    assert np.allclose(y1 - y0, b[None, :], atol=1e-14)
    r0, mu, _ = O.normalize(x, g, b, "rmsnorm", 1e-6, False)
    assert mu is None
    assert np.array_equal(r0, O.rmsnorm(x, g, 1e-6)[0])


def test_zero_centered_gamma_equivalence():
    x = RNG.standard_normal((8, 48))
    g, b = RNG.standard_normal(48) * 0.1, RNG.standard_normal(48)
    for nt in ("layernorm", "rmsnorm"):
        a, _, _ = O.normalize(x, g, b, nt, 1e-6, True)
        c, _, _ = O.normalize(x, 1.0 + g, b, nt, 1e-6, False)
        assert np.array_equal(a, c)


# ---------------------------------------------------------------- activations

def test_activation_golden_values():
    for name, xv, val in read_golden("act_values.txt"):
        got = float(O.act_fn(name, np.array([float(xv)]))[0])
        assert abs(got - float(val)) < 5e-15, (name, xv, got, val)


def test_activation_closed_forms_vs_math_module():
    xs = np.linspace(-6, 6, 97)
    phi = np.array([0.5 * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    assert np.allclose(O.act_fn("gelu_erf", xs), xs * phi, rtol=1e-14, atol=1e-16)
    th = np.array([math.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)) for v in xs])
    # 1 + tanh cancels for x << 0, so compare with an absolute floor of a few ulps of 1
    assert np.allclose(O.act_fn("gelu", xs), 0.5 * xs * (1 + th), rtol=1e-14, atol=1e-14)
    sig = np.array([1 / (1 + math.exp(-v)) for v in xs])
    assert np.allclose(O.act_fn("silu", xs), xs * sig, rtol=1e-14, atol=1e-16)
    assert np.array_equal(O.act_fn("relu", xs), np.where(xs > 0, xs, 0.0))


def test_activation_odd_part_identity():
    # relu, both gelus and silu all satisfy f(x) - f(-x) = x
    xs = RNG.standard_normal(500) * 4
    for name in ("relu", "gelu", "gelu_erf", "silu"):
        d = O.act_fn(name, xs) - O.act_fn(name, -xs)
        assert np.allclose(d, xs, rtol=1e-13, atol=1e-13), name


def test_gelu_variants_differ_and_limits():
    xs = np.array([-30.0, -1.0, 0.5, 30.0])
    e, t = O.act_fn("gelu_erf", xs), O.act_fn("gelu", xs)
    assert abs(e[1] - t[1]) > 1e-4
    assert abs(e[0]) < 1e-30 and abs(t[0]) < 1e-30 and e[3] == 30.0 and t[3] == 30.0


def test_gated_pair_is_first_half_activation_times_second():
    a = RNG.standard_normal((3, 5))
    b = RNG.standard_normal((3, 5))
    h = np.concatenate([a, b], axis=1)
    got = O.activation(h, ("silu", "linear"))
    assert np.allclose(got, a / (1 + np.exp(-a)) * b, rtol=1e-14)
    assert not np.allclose(got, b / (1 + np.exp(-b)) * a)
    assert np.allclose(O.activation(h, ("gelu", "linear")), O.act_fn("gelu", a) * b)


# ---------------------------------------------------------------- backward

@pytest.mark.parametrize("name", ["relu", "gelu", "gelu_erf", "silu", "linear"])
def test_act_grad_central_differences(name):
    xs = RNG.uniform(-4, 4, 400)
    xs = xs[np.abs(xs) > 1e-3]                 # away from the ReLU kink
    h = 1e-6
    fd = (O.act_fn(name, xs + h) - O.act_fn(name, xs - h)) / (2 * h)
    assert np.allclose(O.act_grad(name, xs), fd, rtol=1e-6, atol=1e-8)


def test_relu_grad_at_zero_is_zero():
    assert O.act_grad("relu", np.array([0.0]))[0] == 0.0


@pytest.mark.parametrize("pair", [("silu", "linear"), ("gelu", "linear"), ("relu", "linear"),
                                  ("gelu_erf", "linear")])
def test_gated_dact_central_differences(pair):
    rows, f = 4, 6
    x = RNG.uniform(-3, 3, (rows, 2 * f))
    x[np.abs(x) < 1e-3] = 0.5
    grad = RNG.standard_normal((rows, f))
    dx, dbias = O.dact_dbias(grad, x, pair)
    # d/dx_ij of sum(grad * activation(x)) by central differences, one entry at a time
    h = 1e-6
    fd = np.zeros_like(x)
    for i, j in itertools.product(range(rows), range(2 * f)):
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        fd[i, j] = (np.sum(grad * O.activation(xp, pair)) - np.sum(grad * O.activation(xm, pair))) / (2 * h)
    assert np.allclose(dx, fd, rtol=1e-6, atol=1e-8)
    assert np.allclose(dbias, [math.fsum(dx[:, j]) for j in range(2 * f)], rtol=1e-14)


def test_dbias_is_column_sum_brute_force():
    x = RNG.standard_normal((7, 9))
    g = RNG.standard_normal((7, 9))
    dx, db = O.dact_dbias(g, x, ("gelu",))
    assert np.allclose(db, [math.fsum(dx[i, j] for i in range(7)) for j in range(9)], rtol=1e-14)


# ---------------------------------------------------------------- GEMMs and composites

def test_dense_matches_triple_loop():
    x = RNG.standard_normal((3, 5))
    w = RNG.standard_normal((5, 4))
    b = RNG.standard_normal(4)
    brute = [[math.fsum(x[i, k] * w[k, j] for k in range(5)) + b[j] for j in range(4)] for i in range(3)]
    assert np.allclose(O.dense(x, w, b), brute, rtol=1e-14)


def test_dense_identity_kernel():
    x = RNG.standard_normal((6, 8))
    b = RNG.standard_normal(8)
    assert np.array_equal(O.dense(x, np.eye(8), b), x + b)


def _mlp(x, g, b, w1, w2, b1, b2, act, **kw):
    return O.layernorm_mlp_fwd(x, g, b, w1, w2, b1, b2, norm_type="layernorm", epsilon=1e-6,
                               activation_type=act, **kw)["y"]


def test_mlp_identity_kernels_pin_bias_before_activation():
    h = 16
    x = RNG.standard_normal((4, h))
    g, b = 1 + 0.1 * RNG.standard_normal(h), 0.1 * RNG.standard_normal(h)
    b1, b2 = RNG.standard_normal(h), RNG.standard_normal(h)
    xn, _, _ = O.layernorm(x, g, b, 1e-6)
    y = _mlp(x, g, b, np.eye(h), np.eye(h), b1, b2, ("relu",))
    assert np.allclose(y, np.maximum(xn + b1, 0) + b2, rtol=1e-14, atol=1e-14)


def test_mlp_selection_kernels_pin_operand_roles():
    # kernel1 = [I | 2I] (hidden x 2hidden), kernel2 = [[I], [-I]] (2hidden x hidden):
    # y = gelu(xn + b1[:h]) - gelu(2 xn + b1[h:]) + b2 -- any swapped operand or half changes it
    h = 8
    x = RNG.standard_normal((3, h))
    g, b = np.ones(h), np.zeros(h)
    w1 = np.concatenate([np.eye(h), 2 * np.eye(h)], axis=1)
    w2 = np.concatenate([np.eye(h), -np.eye(h)], axis=0)
    b1, b2 = RNG.standard_normal(2 * h), RNG.standard_normal(h)
    xn, _, _ = O.layernorm(x, g, b, 1e-6)
    y = _mlp(x, g, b, w1, w2, b1, b2, ("gelu",))
    expect = O.act_fn("gelu", xn + b1[:h]) - O.act_fn("gelu", 2 * xn + b1[h:]) + b2
    assert np.allclose(y, expect, rtol=1e-14, atol=1e-14)
    # gated: kernel1 = [I | 3I] gives silu(xn) * 3 xn
    w1g = np.concatenate([np.eye(h), 3 * np.eye(h)], axis=1)
    yg = _mlp(x, g, b, w1g, np.eye(h), None, None, ("silu", "linear"))
    assert np.allclose(yg, O.act_fn("silu", xn) * 3 * xn, rtol=1e-14, atol=1e-14)


def test_fp8_dense_exact_against_integer_arithmetic():
    xq = RNG.integers(0, 256, (4, 32)).astype(np.uint8)
    wq = RNG.integers(0, 256, (32, 5)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x11
    wq[(wq & 0x7F) == 0x7F] = 0x22
    xi = (O.e4m3_decode(xq) * 512).astype(np.int64)     # exact integers (multiples of 2^-9)
    wi = (O.e4m3_decode(wq) * 512).astype(np.int64)
    assert np.array_equal(xi / 512.0, O.e4m3_decode(xq))
    acc = [[sum(int(xi[i, k]) * int(wi[k, j]) for k in range(32)) for j in range(5)] for i in range(4)]
    one = {"scale_inv": 1.0}
    got = O.fp8_dense(xq, one, wq, one)
    assert np.array_equal(got * 2.0 ** 18, np.array(acc, dtype=np.float64))
    sx, sw = {"scale_inv": 0.25}, {"scale_inv": 3.0}
    assert np.array_equal(O.fp8_dense(xq, sx, wq, sw, np.ones(5)), got * 0.75 + 1.0)


def test_fp8_mlp_dataflow_properties():
    h, f = 32, 64
    x = RNG.standard_normal((6, h))
    g, b = 1 + 0.1 * RNG.standard_normal(h), 0.1 * RNG.standard_normal(h)
    w1, w2 = 0.02 * RNG.standard_normal((h, f)), 0.02 * RNG.standard_normal((f, h))
    b1, b2 = 0.02 * RNG.standard_normal(f), 0.02 * RNG.standard_normal(h)
    out = O.layernorm_mlp_fwd(x, g, b, w1, w2, b1, b2, activation_type=("gelu",),
                              quant="fp8_e4m3_current")
    # h1 is bf16-representable; every amax element lands on code 448
    assert np.array_equal(O.bf16_round(out["h1"]), out["h1"])
    for key in ("xq", "w1q", "w2q", "actq"):
        assert np.max(out[key] & 0x7F) == 0x7E
    # fp8 result stays close to the unquantized fp64 forward
    ref = O.layernorm_mlp_fwd(x, g, b, w1, w2, b1, b2, activation_type=("gelu",))["y"]
    assert O.rel_l2(out["y"], ref) < 0.1
    # row subset reproduces the same rows
    sub = O.layernorm_mlp_fwd(x, g, b, w1, w2, b1, b2, activation_type=("gelu",),
                              quant="fp8_e4m3_current", rows=np.array([4, 1]))
    assert np.array_equal(sub["y"], out["y"][[4, 1]])


def test_round_intermediates_is_close_to_exact():
    h, f = 64, 128
    x = RNG.standard_normal((8, h))
    g, b = np.ones(h), np.zeros(h)
    w1, w2 = 0.1 * RNG.standard_normal((h, f)), 0.1 * RNG.standard_normal((f, h))
    a = _mlp(x, g, b, w1, w2, None, None, ("gelu",))
    r = _mlp(x, g, b, w1, w2, None, None, ("gelu",), round_intermediates=True)
    e = O.rel_l2(r, a)
    assert 1e-4 < e < 5e-3


def test_bf16_rounding_error_of_normal_data():
    # the per-rounding budget the backward bounds are built from
    from tolerances import U_BF16
    x = RNG.standard_normal(1_000_000)
    for scale in (1.0, 0.02, 300.0):
        e = O.rel_l2(O.bf16_round(x * scale), x * scale)
        assert abs(e - U_BF16) <= 0.02 * U_BF16, (scale, e)


# ---- layernorm_dense forward: identity kernels reduce it to the (pinned) norm

@pytest.mark.parametrize("norm_type,zcg", [("layernorm", False), ("rmsnorm", True)])
def test_layernorm_dense_identity_kernel(norm_type, zcg):
    h = 16
    x = RNG.standard_normal((5, h)) * 2.0 + 0.5
    g = RNG.standard_normal(h) * 0.1 + (0.0 if zcg else 1.0)
    b = RNG.standard_normal(h) * 0.1
    bias = RNG.standard_normal(h)
    xn = O.normalize(x, g, b, norm_type, 1e-5, zcg)[0]
    out = O.layernorm_dense_fwd(x, np.eye(h), g, b, bias, norm_type=norm_type, zero_centered_gamma=zcg,
                                epsilon=1e-5)
    assert np.array_equal(out["y"], xn + bias)
    assert np.array_equal(out["xn"], xn)
    r = O.layernorm_dense_fwd(x, np.eye(h), g, b, bias, norm_type=norm_type, zero_centered_gamma=zcg,
                              epsilon=1e-5, round_intermediates=True)
    assert np.array_equal(r["y"], O.bf16_round(xn) + bias)
    assert np.array_equal(O.layernorm_dense_fwd(x, np.eye(h), g, b, None, norm_type=norm_type,
                                                zero_centered_gamma=zcg, epsilon=1e-5)["y"], xn)


def test_layernorm_dense_fp8_identity_kernel():
    # kernel = I: amax 1, so every diagonal code is 448 and the kernel's
    # scale_inv is fl32(1/448); y is then the normalised input after one E4M3
    # rounding at its own scale, plus the bias. Quantising x instead of the
    # normalised x, or dropping the bias, moves y far outside that.
    h = 32
    x = RNG.standard_normal((6, h)) * 3.0 + 1.0
    g, b = 1.0 + 0.1 * RNG.standard_normal(h), 0.1 * RNG.standard_normal(h)
    bias = RNG.standard_normal(h)
    xn = O.layernorm(x, g, b, 1e-6)[0]
    out = O.layernorm_dense_fwd(x, np.eye(h), g, b, bias, epsilon=1e-6, quant="fp8_e4m3_current")
    assert out["w_meta"]["amax"] == 1.0 and out["w_meta"]["scale"] == 448.0
    assert np.array_equal(out["wq"], np.where(np.eye(h) > 0, 0x7E, 0).astype(np.uint8))
    assert out["x_meta"]["amax"] == float(O.fl32(np.max(np.abs(xn))))
    # dec(code) * scale_inv: each value within half an E4M3 step (2^-4 relative,
    # or the subnormal step 2^-10 at the tensor's scale) of the normalised input
    deq = O.e4m3_decode(out["xq"]) * out["x_meta"]["scale_inv"]
    assert np.all(np.abs(deq - xn) <= np.maximum(2.0 ** -4 * np.abs(xn), 2.0 ** -10 * out["x_meta"]["scale_inv"])
                  * (1 + 1e-6))
    # 448 * fl32(1/448) differs from 1 by about 1e-8: the difference scales with deq alone
    assert np.all(np.abs(out["y"] - (deq + bias)) <= 1e-7 * np.abs(deq))
    assert O.rel_l2(out["y"], xn + bias) < 2.0 ** -4


def test_rel_l2():
    assert O.rel_l2([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert abs(O.rel_l2([3.0, 5.0], [3.0, 4.0]) - 0.2) < 1e-15


# ---- norm backward: finite differences of the (pinned) forward, invariants

def _norm_fwd_sum(dy, x, gamma, beta, norm_type, eps, zcg):
    y = O.normalize(x, gamma, beta, norm_type, eps, zcg)[0]
    return float(np.sum(dy * y))


@pytest.mark.parametrize("norm_type", ["layernorm", "rmsnorm"])
@pytest.mark.parametrize("zcg", [False, True])
def test_norm_bwd_central_differences(norm_type, zcg):
    rows, h, eps = 3, 8, 1e-3
    x = RNG.standard_normal((rows, h)) * 1.5 + 0.3
    gamma = RNG.standard_normal(h) * 0.3 + (0.0 if zcg else 1.0)
    beta = RNG.standard_normal(h) * 0.1
    dy = RNG.standard_normal((rows, h))
    dx, dgamma, dbeta = O.norm_bwd(dy, x, gamma, norm_type, eps, zcg)
    d = 1e-6

    def fd(arr, idx):
        ap, am = arr.copy(), arr.copy()
        ap[idx] += d
        am[idx] -= d
        return ap, am

    for i, j in itertools.product(range(rows), range(h)):
        xp, xm = fd(x, (i, j))
        g = (_norm_fwd_sum(dy, xp, gamma, beta, norm_type, eps, zcg)
             - _norm_fwd_sum(dy, xm, gamma, beta, norm_type, eps, zcg)) / (2 * d)
        assert abs(dx[i, j] - g) <= 1e-6 * max(1.0, abs(g)), (i, j, dx[i, j], g)
    for j in range(h):
        gp, gm = fd(gamma, j)
        g = (_norm_fwd_sum(dy, x, gp, beta, norm_type, eps, zcg) - _norm_fwd_sum(dy, x, gm, beta, norm_type, eps, zcg)) / (2 * d)
        assert abs(dgamma[j] - g) <= 1e-6 * max(1.0, abs(g))
        if norm_type == "layernorm":
            bp, bm = fd(beta, j)
            g = (_norm_fwd_sum(dy, x, gamma, bp, norm_type, eps, zcg)
                 - _norm_fwd_sum(dy, x, gamma, bm, norm_type, eps, zcg)) / (2 * d)
            assert abs(dbeta[j] - g) <= 1e-6 * max(1.0, abs(g))
    if norm_type == "rmsnorm":
        assert dbeta is None


def test_layernorm_bwd_dx_sums_to_zero_per_row():
    # shifting a row by a constant leaves LayerNorm unchanged, so dx has zero row sums
    x = RNG.standard_normal((5, 64)) * 2.0 + 1.0
    dx = O.norm_bwd(RNG.standard_normal((5, 64)), x, RNG.standard_normal(64), "layernorm", 1e-5)[0]
    assert np.max(np.abs(dx.sum(axis=-1))) <= 1e-12 * np.max(np.abs(dx)) * 64


def test_rmsnorm_bwd_dx_orthogonal_to_x_when_eps_is_zero():
    # with eps = 0 RMSNorm is invariant to scaling the row, so dx . x = 0
    x = RNG.standard_normal((4, 32))
    dx = O.norm_bwd(RNG.standard_normal((4, 32)), x, RNG.standard_normal(32), "rmsnorm", 0.0)[0]
    assert np.max(np.abs((dx * x).sum(axis=-1))) <= 1e-12 * np.max(np.abs(dx)) * 32


def test_norm_bwd_zero_centered_gamma_equivalence():
    x, dy, gamma = RNG.standard_normal((3, 16)), RNG.standard_normal((3, 16)), RNG.standard_normal(16) * 0.1
    for nt in ("layernorm", "rmsnorm"):
        a = O.norm_bwd(dy, x, gamma, nt, 1e-6, True)
        b = O.norm_bwd(dy, x, 1.0 + gamma, nt, 1e-6, False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- layernorm_mlp backward: finite differences of the whole (pinned) forward

@pytest.mark.parametrize("norm_type,act", [("layernorm", ("gelu",)), ("rmsnorm", ("silu", "linear")),
                                           ("layernorm", ("gelu_erf", "linear"))])
def test_mlp_bwd_central_differences(norm_type, act):
    rows, h, f = 3, 4, 5
    g2 = 2 if len(act) == 2 else 1
    x = RNG.standard_normal((rows, h))
    gamma = RNG.standard_normal(h) * 0.3 + 1.0
    beta = RNG.standard_normal(h) * 0.2 if norm_type == "layernorm" else None
    w1 = RNG.standard_normal((h, g2 * f)) * 0.5
    b1 = RNG.standard_normal(g2 * f) * 0.2
    w2 = RNG.standard_normal((f, h)) * 0.5
    b2 = RNG.standard_normal(h) * 0.2
    gy = RNG.standard_normal((rows, h))
    eps = 1e-3
    args = dict(x=x, gamma=gamma, beta=beta, kernel1=w1, kernel2=w2, bias1=b1, bias2=b2)

    def loss(**kw):
        a = dict(args)
        a.update(kw)
        y = O.layernorm_mlp_fwd(a["x"], a["gamma"], a["beta"], a["kernel1"], a["kernel2"], a["bias1"], a["bias2"],
                                norm_type=norm_type, epsilon=eps, activation_type=act)["y"]
        return float(np.sum(gy * y))

    g = O.layernorm_mlp_bwd(gy, x, gamma, beta, w1, w2, b1, b2, norm_type=norm_type, epsilon=eps,
                            activation_type=act)
    names = [("x", "dx"), ("gamma", "dgamma"), ("kernel1", "dkernel1"), ("bias1", "dbias1"),
             ("kernel2", "dkernel2"), ("bias2", "dbias2")]
    if norm_type == "layernorm":
        names.append(("beta", "dbeta"))
    d = 1e-6
    for arg, out in names:
        base = args[arg]
        for idx in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += d
            m[idx] -= d
            fd = (loss(**{arg: p}) - loss(**{arg: m})) / (2 * d)
            assert abs(g[out][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (arg, idx, g[out][idx], fd)
    if norm_type == "rmsnorm":
        assert g["dbeta"] is None


def test_mlp_bwd_round_intermediates_close_to_exact():
    # rounding xn, h1, act, dact, dh1 and dxn to bf16 moves each gradient by
    # about sqrt(k) one-rounding errors (k = the roundings on its chain): more
    # than nothing, less than the derived bound
    from tolerances import bwd_roundings, rounding_bound, U_BF16
    rows, h, f = 96, 64, 80
    for norm_type, act in (("layernorm", ("gelu",)), ("rmsnorm", ("silu", "linear"))):
        gated = len(act) == 2
        x = RNG.standard_normal((rows, h))
        gamma = 1.0 + 0.1 * RNG.standard_normal(h)
        beta = 0.1 * RNG.standard_normal(h) if norm_type == "layernorm" else None
        w1 = 0.1 * RNG.standard_normal((h, (2 if gated else 1) * f))
        w2 = 0.1 * RNG.standard_normal((f, h))
        b1 = 0.05 * RNG.standard_normal(w1.shape[1])
        gy = RNG.standard_normal((rows, h))
        kw = dict(norm_type=norm_type, epsilon=1e-6, activation_type=act)
        ex = O.layernorm_mlp_bwd(gy, x, gamma, beta, w1, w2, b1, None, **kw)
        rd = O.layernorm_mlp_bwd(gy, x, gamma, beta, w1, w2, b1, None, round_intermediates=True, **kw)
        for name, ref in ex.items():
            if ref is None:
                continue
            e = O.rel_l2(rd[name], ref)
            k = bwd_roundings(name, gated, output_rounded=False)
            if k == 0:
                assert e == 0.0, name
            else:
                assert 0.3 * U_BF16 < e <= rounding_bound(k), (name, act, e, rounding_bound(k))


def test_mlp_bwd_round_intermediates_keep_bf16_exact_values():
    # rows of +-1 with zero mean and unit variance normalise to themselves at
    # eps = 0; with dyadic kernels, biases and grad every intermediate of the
    # chain is a short dyadic fraction (exact in bf16), so rounding changes
    # nothing and both modes agree bit for bit
    h, f, rows = 8, 12, 6
    sgn = RNG.permuted(np.tile(np.array([1.0, -1.0] * (h // 2)), (rows, 1)), axis=1)
    w1 = RNG.choice([0.0, 0.25, -0.25, 0.5, -0.5], (h, f))
    w2 = RNG.choice([0.0, 0.25, -0.5, 0.5], (f, h))
    b1 = RNG.choice([0.125, -0.125], f)
    gy = RNG.choice([1.0, -1.0, 0.5, -0.5], (rows, h))
    kw = dict(norm_type="layernorm", epsilon=0.0, activation_type=("relu",))
    assert np.array_equal(O.layernorm(sgn, np.ones(h), np.zeros(h), 0.0)[0], sgn)
    ex = O.layernorm_mlp_bwd(gy, sgn, np.ones(h), np.zeros(h), w1, w2, b1, None, **kw)
    rd = O.layernorm_mlp_bwd(gy, sgn, np.ones(h), np.zeros(h), w1, w2, b1, None, round_intermediates=True, **kw)
    for name in ex:
        assert np.array_equal(ex[name], rd[name]), name
