"""Planted mistakes in the oracle (CPU only): each mutant must make at least
one pin of tests/test_oracle_pins.py fail. This shows the pins would catch a
dropped term, a wrong sign, constant or index, or a swapped half."""

import math

import numpy as np
import pytest

import oracle
import oracle.te_oracle as T
import test_oracle_pins as P


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(T, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _ln_unbiased(x, gamma, beta, epsilon, zero_centered_gamma=False):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1)
    var = ((x - mu[..., None]) ** 2).sum(axis=-1) / (x.shape[-1] - 1)
    rs = 1.0 / np.sqrt(var + epsilon)
    g = T.effective_gamma(gamma, zero_centered_gamma)
    return (x - mu[..., None]) * rs[..., None] * g + beta, mu, rs


def _ln_eps_outside(x, gamma, beta, epsilon, zero_centered_gamma=False):
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1)
    var = ((x - mu[..., None]) ** 2).mean(axis=-1)
    rs = 1.0 / (np.sqrt(var) + epsilon)
    g = T.effective_gamma(gamma, zero_centered_gamma)
    return (x - mu[..., None]) * rs[..., None] * g + beta, mu, rs


_orig_act = T.act_fn
_orig_encode = T.e4m3_encode
_orig_decode = T.e4m3_decode
_orig_grad = T.act_grad


def _act_bad_gelu_const(name, x):
    if name == "gelu":
        x = np.asarray(x, dtype=np.float64)
        return 0.5 * x * (1.0 + np.tanh(T.GELU_K0 * (x + 0.04 * x ** 3)))
    return _orig_act(name, x)


def _act_bad_silu_sign(name, x):
    if name == "silu":
        x = np.asarray(x, dtype=np.float64)
        return x / (1.0 + np.exp(x))
    return _orig_act(name, x)


def _grad_relu_one_at_zero(name, x):
    if name == "relu":
        return (np.asarray(x) >= 0.0).astype(np.float64)
    return _orig_grad(name, x)


def _grad_gelu_dropped_term(name, x):
    if name == "gelu":
        x = np.asarray(x, dtype=np.float64)
        t = np.tanh(T.GELU_K0 * (x + T.GELU_K1 * x ** 3))
        return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * T.GELU_K0
    return _orig_grad(name, x)


def _activation_swapped_halves(x, activation_type):
    x = np.asarray(x, dtype=np.float64)
    if len(activation_type) == 2:
        f = x.shape[-1] // 2
        return T.act_fn(activation_type[0], x[..., f:]) * T.act_fn(activation_type[1], x[..., :f])
    return T.act_fn(activation_type[0], x)


def _encode_ties_away(v):
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    _, ex = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    r = np.floor(a / q + 0.5) * q
    return _orig_encode(np.copysign(r, v))


def _decode_bias8(codes):
    return _orig_decode(codes) / 2.0


def _scaling_no_fp32(t):
    amax = float(np.max(np.abs(t)))
    if amax == 0.0:
        return {"amax": 0.0, "scale": 1.0, "scale_inv": 1.0}
    return {"amax": amax, "scale": 448.0 / amax, "scale_inv": amax / 448.0}


def _dense_bias_dropped(x, kernel, bias=None):
    return np.matmul(np.asarray(x, dtype=np.float64), np.asarray(kernel, dtype=np.float64))


def _mlp_bias_after_act(x, gamma, beta, kernel1, kernel2, bias1=None, bias2=None, norm_type="layernorm",
                        zero_centered_gamma=False, epsilon=1e-6, activation_type=("relu",), quant="none",
                        round_intermediates=False, rows=None):
    xn, mu, rs = T.normalize(x, gamma, beta, norm_type, epsilon, zero_centered_gamma)
    h = np.matmul(xn, kernel1)
    act = T.activation(h, activation_type)
    if bias1 is not None:
        act = act + bias1
    return {"y": T.dense(act, kernel2, bias2)}


def _dact_no_gate(grad, x, activation_type):
    grad = np.asarray(grad, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    if len(activation_type) == 1:
        dx = grad * T.act_grad(activation_type[0], x)
    else:
        f = x.shape[-1] // 2
        a, b = x[..., :f], x[..., f:]
        dx = np.concatenate([grad * T.act_grad(activation_type[0], a),
                             grad * T.act_fn(activation_type[0], a)], axis=-1)
    return dx, dx.sum(axis=0)


def _zcg_ignored(gamma, zero_centered_gamma):
    return np.asarray(gamma, dtype=np.float64)


def _bf16_truncate(a):
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)
    q = np.ldexp(1.0, np.maximum(ex - 1, -126) - 7)
    return np.where(a == 0, a, np.trunc(a / q) * q)


_orig_norm_bwd = T.norm_bwd


def _norm_bwd_dropped_mean(dy, x, gamma, norm_type, epsilon, zero_centered_gamma=False):
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    if norm_type != "layernorm":
        return _orig_norm_bwd(dy, x, gamma, norm_type, epsilon, zero_centered_gamma)
    mu = x.mean(axis=-1, keepdims=True)
    rs = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + epsilon)
    xhat = (x - mu) * rs
    dxhat = dy * T.effective_gamma(gamma, zero_centered_gamma)
    dx = rs * (dxhat - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def _norm_bwd_dgamma_from_x(dy, x, gamma, norm_type, epsilon, zero_centered_gamma=False):
    dx, _, dbeta = _orig_norm_bwd(dy, x, gamma, norm_type, epsilon, zero_centered_gamma)
    return dx, (np.asarray(dy) * np.asarray(x)).sum(axis=0), dbeta


_orig_mlp_bwd = T.layernorm_mlp_bwd


def _mlp_bwd_dkernel2_from_h(grad, x, gamma, beta, kernel1, kernel2, bias1=None, bias2=None, norm_type="layernorm",
                             zero_centered_gamma=False, epsilon=1e-6, activation_type=("relu",), h1=None,
                             round_intermediates=False):
    out = _orig_mlp_bwd(grad, x, gamma, beta, kernel1, kernel2, bias1, bias2, norm_type, zero_centered_gamma,
                        epsilon, activation_type, h1, round_intermediates)
    xn = T.normalize(x, gamma, beta, norm_type, epsilon, zero_centered_gamma)[0]
    h = T.dense(xn, kernel1, bias1)
    f = np.asarray(kernel2).shape[0]
    out["dkernel2"] = np.matmul(h[:, :f].T, np.asarray(grad, dtype=np.float64))   # pre-activation instead of act
    return out


_orig_dense_fwd = T.layernorm_dense_fwd


def _dense_fwd_quantizes_x(x, kernel, gamma, beta, bias=None, norm_type="layernorm", zero_centered_gamma=False,
                           epsilon=1e-6, quant="none", round_intermediates=False):
    if quant == "none":
        return _orig_dense_fwd(x, kernel, gamma, beta, bias, norm_type, zero_centered_gamma, epsilon, quant,
                               round_intermediates)
    xn, mu, rs = T.normalize(x, gamma, beta, norm_type, epsilon, zero_centered_gamma)
    xq, xm = T.quantize(np.asarray(x, dtype=np.float64))        # the input, not its normalised form
    wq, wm = T.quantize(kernel)
    return {"mu": mu, "rsigma": rs, "xn": xn, "xq": xq, "x_meta": xm, "wq": wq, "w_meta": wm,
            "y": T.fp8_dense(xq, xm, wq, wm, bias)}


def _dense_fwd_fp8_drops_bias(x, kernel, gamma, beta, bias=None, norm_type="layernorm", zero_centered_gamma=False,
                              epsilon=1e-6, quant="none", round_intermediates=False):
    return _orig_dense_fwd(x, kernel, gamma, beta, None if quant != "none" else bias, norm_type,
                           zero_centered_gamma, epsilon, quant, round_intermediates)


def _dense_fwd_drops_bias(x, kernel, gamma, beta, bias=None, norm_type="layernorm", zero_centered_gamma=False,
                          epsilon=1e-6, quant="none", round_intermediates=False):
    return _orig_dense_fwd(x, kernel, gamma, beta, None if quant == "none" else bias, norm_type,
                           zero_centered_gamma, epsilon, quant, round_intermediates)


def _mlp_bwd_truncating_rounds(grad, x, gamma, beta, kernel1, kernel2, bias1=None, bias2=None, norm_type="layernorm",
                               zero_centered_gamma=False, epsilon=1e-6, activation_type=("relu",), h1=None,
                               round_intermediates=False):
    # the backward's bf16 materialisations truncate instead of rounding to nearest
    saved = T.bf16_round
    T.bf16_round = _bf16_truncate
    try:
        return _orig_mlp_bwd(grad, x, gamma, beta, kernel1, kernel2, bias1, bias2, norm_type, zero_centered_gamma,
                             epsilon, activation_type, h1, round_intermediates)
    finally:
        T.bf16_round = saved


def _mlp_bwd_rounds_to_e4m3(grad, x, gamma, beta, kernel1, kernel2, bias1=None, bias2=None, norm_type="layernorm",
                            zero_centered_gamma=False, epsilon=1e-6, activation_type=("relu",), h1=None,
                            round_intermediates=False):
    # the wrong narrow format (4 significant bits) at the materialisation points
    saved = T.bf16_round
    T.bf16_round = lambda a: T.round_to_bits(a, 4, -6)
    try:
        return _orig_mlp_bwd(grad, x, gamma, beta, kernel1, kernel2, bias1, bias2, norm_type, zero_centered_gamma,
                             epsilon, activation_type, h1, round_intermediates)
    finally:
        T.bf16_round = saved


MUTANTS = [
    ("layernorm", _ln_unbiased, [P.test_layernorm_invariants_closed_form_variance, P.test_layernorm_brute_force]),
    ("layernorm", _ln_eps_outside, [P.test_layernorm_brute_force]),
    ("act_fn", _act_bad_gelu_const, [P.test_activation_golden_values]),
    ("act_fn", _act_bad_silu_sign, [P.test_activation_golden_values]),
    ("act_grad", _grad_relu_one_at_zero, [P.test_relu_grad_at_zero_is_zero]),
    ("act_grad", _grad_gelu_dropped_term, [lambda: P.test_act_grad_central_differences("gelu")]),
    ("activation", _activation_swapped_halves, [P.test_gated_pair_is_first_half_activation_times_second]),
    ("e4m3_encode", _encode_ties_away, [P.test_e4m3_midpoints_go_to_even_code]),
    ("e4m3_decode", _decode_bias8, [P.test_e4m3_decode_spec_points]),
    ("current_scaling", _scaling_no_fp32, [P.test_current_scaling_closed_forms]),
    ("dense", _dense_bias_dropped, [P.test_dense_matches_triple_loop]),
    ("layernorm_mlp_fwd", _mlp_bias_after_act, [P.test_mlp_identity_kernels_pin_bias_before_activation]),
    ("dact_dbias", _dact_no_gate, [lambda: P.test_gated_dact_central_differences(("silu", "linear"))]),
    ("effective_gamma", _zcg_ignored, [P.test_zero_centered_gamma_equivalence]),
    ("bf16_round", _bf16_truncate, [P.test_bf16_round_matches_torch_cast]),
    ("norm_bwd", _norm_bwd_dropped_mean, [P.test_layernorm_bwd_dx_sums_to_zero_per_row,
                                          lambda: P.test_norm_bwd_central_differences("layernorm", False)]),
    ("norm_bwd", _norm_bwd_dgamma_from_x, [lambda: P.test_norm_bwd_central_differences("rmsnorm", True)]),
    ("layernorm_mlp_bwd", _mlp_bwd_dkernel2_from_h,
     [lambda: P.test_mlp_bwd_central_differences("layernorm", ("gelu",))]),
    ("layernorm_dense_fwd", _dense_fwd_quantizes_x, [P.test_layernorm_dense_fp8_identity_kernel]),
    ("layernorm_dense_fwd", _dense_fwd_fp8_drops_bias, [P.test_layernorm_dense_fp8_identity_kernel]),
    ("layernorm_dense_fwd", _dense_fwd_drops_bias,
     [lambda: P.test_layernorm_dense_identity_kernel("layernorm", False)]),
    ("layernorm_mlp_bwd", _mlp_bwd_truncating_rounds, [P.test_mlp_bwd_round_intermediates_close_to_exact]),
    ("layernorm_mlp_bwd", _mlp_bwd_rounds_to_e4m3, [P.test_mlp_bwd_round_intermediates_close_to_exact]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, pins):
    _patch(monkeypatch, name, mutant)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {name} ({mutant.__name__})"


def test_pins_pass_unmutated():
    for _, _, pins in MUTANTS:
        for pin in pins:
            pin()
