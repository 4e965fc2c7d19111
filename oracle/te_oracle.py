"""fp64 CPU oracle for the fused norm -> GEMM1 -> activation -> GEMM2 path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP library.

Every function is the plain definition written out in float64 numpy, in the
order the pages describe. Sources (the three pages of the TransformerEngine
JAX documentation):
  [ACT]   "NVIDIA TransformerEngine JAX Activation"
  [MLP]   "NVIDIA TransformerEngine JAX LayerNorm MLP"
  [DENSE] "NVIDIA TransformerEngine JAX LayerNorm Dense"
The pages state what is computed only in words. Where they are silent the
plainest reading is taken (each is listed in the design notes of the repo):
biased variance, epsilon inside the square root, beta unused by RMSNorm,
zero-centred gamma meaning a scale of 1 + gamma, GELU = tanh approximation
(the erf form is separate), ReLU'(0) = 0, gated pair = act(first half) *
second half, FP8 = OCP E4M3 (max 448) with round-to-nearest-even and
saturation, per-tensor current scaling scale = 448 / amax (1 when amax = 0).

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against invariants, closed forms, brute force or library routines. The gated
half order (first half -> activation, second half -> linear) is a layout
convention and is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

E4M3_MAX = 448.0
GELU_K0 = math.sqrt(2.0 / math.pi)
GELU_K1 = 0.044715


# --------------------------------------------------------------------------
# Rounding helpers (the precisions the GPU path materialises tensors in)
# --------------------------------------------------------------------------

def fl32(a) -> np.ndarray:
    """Round to the nearest fp32 value (ties to even), returned as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bits(a, p: int, emin: int) -> np.ndarray:
    """Round each value to the nearest binary float with ``p`` significant bits
    and minimum normal exponent ``emin`` (ties to even), no overflow handling.

    A value v with 2^e <= |v| < 2^(e+1) is rounded on the grid of step
    2^(max(e, emin) - (p - 1)); this is the textbook definition of rounding to
    a p-bit floating-point format with gradual underflow.
    """
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)                      # |a| = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)
    q = np.ldexp(1.0, e - (p - 1))
    return np.where(a == 0.0, a, np.rint(a / q) * q)


def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 (8 significant bits, fp32 exponent range)."""
    return round_to_bits(a, 8, -126)


# --------------------------------------------------------------------------
# OCP E4M3 (E4M3FN) codec
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Value of each 8-bit E4M3 code: sign s, exponent field e (4 bits, bias 7),
    mantissa field m (3 bits). e = 0 gives subnormals m * 2^-9; otherwise
    (1 + m/8) * 2^(e-7); e = 15 with m = 7 is NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value; ties go to the even mantissa; values
    beyond +-448 saturate to +-448; the sign of zero is kept. Inputs must not
    be NaN."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    r = round_to_bits(a, 4, -6)              # 1 + 3 mantissa bits, min normal 2^-6
    r = np.minimum(r, E4M3_MAX)
    _, ex = np.frexp(r)
    e_unb = ex - 1
    normal = r >= 2.0 ** -6
    e_field = np.where(normal, e_unb + 7, 0)
    m_field = np.where(normal, np.rint((r / np.ldexp(1.0, e_unb) - 1.0) * 8.0),
                       np.rint(r / 2.0 ** -9))
    e_field = np.where(r == 0.0, 0, e_field)
    m_field = np.where(r == 0.0, 0, m_field)
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def e4m3_encode_fp32(v) -> np.ndarray:
    """e4m3_encode for fp32-representable inputs, via a library routine:
    saturate to +-448, then torch's round-to-nearest-even float8_e4m3fn cast.
    Used for large tensors; pinned against e4m3_encode in the tests."""
    import torch
    v = np.asarray(v, dtype=np.float32)
    c = np.clip(v, -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(np.ascontiguousarray(c)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def current_scaling(t) -> Dict[str, float]:
    """Per-tensor current scaling ([ACT] Description: the activation output is
    quantized; [DENSE] Description: the normalized output and the kernel are
    quantized before the GEMM). amax = max |t| over the whole tensor;
    scale = fl32(448 / fl32(amax)), or 1 when amax = 0; scale_inv = fl32(1/scale).
    """
    amax = float(np.max(np.abs(t))) if np.size(t) else 0.0
    amax32 = float(fl32(amax))
    scale = float(fl32(E4M3_MAX / amax32)) if amax32 > 0.0 else 1.0
    return {"amax": amax32, "scale": scale, "scale_inv": float(fl32(1.0 / scale))}


def quantize(t, meta: Optional[Dict[str, float]] = None):
    """E4M3 codes of ``t`` under current scaling: code = enc(fl32(fl32(t) * scale)).
    Returns (codes uint8, meta)."""
    if meta is None:
        meta = current_scaling(t)
    prod = fl32(fl32(t) * meta["scale"])
    return e4m3_encode_fp32(prod), meta


def dequantize(codes, meta) -> np.ndarray:
    """[ACT] Outputs: the quantized activation is returned dequantized back to
    the original precision: dec(code) * scale_inv."""
    return e4m3_decode(codes) * meta["scale_inv"]


# --------------------------------------------------------------------------
# Normalization ([MLP] Description step (1); [DENSE] Description; Inputs
# tables: gamma, beta, norm_type, zero_centered_gamma, epsilon)
# --------------------------------------------------------------------------

def effective_gamma(gamma, zero_centered_gamma: bool) -> np.ndarray:
    """With a zero-centred gamma the scale applied is 1 + gamma."""
    g = np.asarray(gamma, dtype=np.float64)
    return 1.0 + g if zero_centered_gamma else g


def layernorm(x, gamma, beta, epsilon: float, zero_centered_gamma: bool = False):
    """LayerNorm over the last (hidden) axis: mu = mean(x), var = mean((x-mu)^2)
    (biased), y = (x - mu) / sqrt(var + eps) * g + beta.
    Returns (y, mu, rsigma) with rsigma = 1 / sqrt(var + eps)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1)
    var = ((x - mu[..., None]) ** 2).mean(axis=-1)
    rsigma = 1.0 / np.sqrt(var + epsilon)
    y = (x - mu[..., None]) * rsigma[..., None] * effective_gamma(gamma, zero_centered_gamma) \
        + np.asarray(beta, dtype=np.float64)
    return y, mu, rsigma


def rmsnorm(x, gamma, epsilon: float, zero_centered_gamma: bool = False):
    """RMSNorm over the last axis: y = x / sqrt(mean(x^2) + eps) * g (no shift).
    Returns (y, rsigma)."""
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=-1)
    rsigma = 1.0 / np.sqrt(ms + epsilon)
    y = x * rsigma[..., None] * effective_gamma(gamma, zero_centered_gamma)
    return y, rsigma


def normalize(x, gamma, beta, norm_type: str, epsilon: float, zero_centered_gamma: bool):
    """Dispatch on norm_type ("layernorm" | "rmsnorm"). Returns (y, mu, rsigma);
    mu is None for RMSNorm."""
    if norm_type == "layernorm":
        return layernorm(x, gamma, beta, epsilon, zero_centered_gamma)
    if norm_type == "rmsnorm":
        y, rs = rmsnorm(x, gamma, epsilon, zero_centered_gamma)
        return y, None, rs
    raise ValueError(f"unknown norm_type {norm_type!r}")


def norm_bwd(dy, x, gamma, norm_type: str, epsilon: float, zero_centered_gamma: bool = False):
    """Gradients of the normalization ([DENSE] Description: the backward pass
    gives the gradients of every input, x, gamma and beta among them, from the
    saved forward context). With xhat the normalized input (before g and
    beta), rs = 1 / sqrt(var + eps) (LayerNorm) or 1 / sqrt(mean(x^2) + eps)
    (RMSNorm) and dxhat = dy * g:
      LayerNorm: dx = rs * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))
      RMSNorm:   dx = rs * (dxhat - xhat * mean(dxhat * xhat))
      dgamma = sum over rows of dy * xhat (also for a zero-centred gamma, whose
      scale 1 + gamma has the same derivative); dbeta = sum over rows of dy
      (LayerNorm only). The statistics are recomputed here from x.
    Returns (dx, dgamma, dbeta); dbeta is None for RMSNorm."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    g = effective_gamma(gamma, zero_centered_gamma)
    if norm_type == "layernorm":
        mu = x.mean(axis=-1, keepdims=True)
        rs = 1.0 / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + epsilon)
        xhat = (x - mu) * rs
    elif norm_type == "rmsnorm":
        rs = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + epsilon)
        xhat = x * rs
    else:
        raise ValueError(f"unknown norm_type {norm_type!r}")
    dxhat = dy * g
    inner = dxhat - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True)
    if norm_type == "layernorm":
        inner = inner - dxhat.mean(axis=-1, keepdims=True)
    dx = rs * inner
    dgamma = (dy * xhat).reshape(-1, x.shape[-1]).sum(axis=0)
    dbeta = dy.reshape(-1, x.shape[-1]).sum(axis=0) if norm_type == "layernorm" else None
    return dx, dgamma, dbeta


# --------------------------------------------------------------------------
# Activations ([ACT] Overview: GELU, SiLU, ReLU; Inputs: activation_type such
# as ("gelu",) or the gated pair ("silu", "linear"))
# --------------------------------------------------------------------------

def _erf(a):
    return np.vectorize(math.erf, otypes=[np.float64])(a)


def act_fn(name: str, x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if name == "relu":
        return np.maximum(x, 0.0)
    if name == "gelu":          # tanh approximation
        return 0.5 * x * (1.0 + np.tanh(GELU_K0 * (x + GELU_K1 * x ** 3)))
    if name == "gelu_erf":
        return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))
    if name == "silu":
        return x / (1.0 + np.exp(-x))
    if name == "linear":
        return x
    raise ValueError(f"unknown activation {name!r}")


def act_grad(name: str, x) -> np.ndarray:
    """Derivative of act_fn at x (ReLU'(0) taken as 0)."""
    x = np.asarray(x, dtype=np.float64)
    if name == "relu":
        return (x > 0.0).astype(np.float64)
    if name == "gelu":
        u = GELU_K0 * (x + GELU_K1 * x ** 3)
        t = np.tanh(u)
        return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * GELU_K0 * (1.0 + 3.0 * GELU_K1 * x * x)
    if name == "gelu_erf":
        return 0.5 * (1.0 + _erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    if name == "silu":
        s = 1.0 / (1.0 + np.exp(-x))
        return s * (1.0 + x * (1.0 - s))
    if name == "linear":
        return np.ones_like(x)
    raise ValueError(f"unknown activation {name!r}")


def activation(x, activation_type: Sequence[str]) -> np.ndarray:
    """[ACT] forward. One name: act(x). A pair (f, g): the last axis holds two
    equal halves [a | b] and the result is f(a) * g(b)."""
    x = np.asarray(x, dtype=np.float64)
    if len(activation_type) == 1:
        return act_fn(activation_type[0], x)
    if len(activation_type) == 2:
        f = x.shape[-1] // 2
        return act_fn(activation_type[0], x[..., :f]) * act_fn(activation_type[1], x[..., f:])
    raise ValueError("activation_type must have one or two entries")


def dact_dbias(grad, x, activation_type: Sequence[str]):
    """Activation backward with the bias reduction ([ACT] Description: the
    backward rule gives the activation gradient; [MLP] Description: the fused
    backward yields the activation gradient together with the bias reduction).
    dx = grad * act'(x); gated: da = grad * g(b) * f'(a), db = grad * f(a) * g'(b).
    dbias = sum of dx over all rows. Returns (dx, dbias)."""
    grad = np.asarray(grad, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    if len(activation_type) == 1:
        dx = grad * act_grad(activation_type[0], x)
    else:
        f = x.shape[-1] // 2
        a, b = x[..., :f], x[..., f:]
        fa, fb = act_fn(activation_type[0], a), act_fn(activation_type[1], b)
        da = grad * fb * act_grad(activation_type[0], a)
        db = grad * fa * act_grad(activation_type[1], b)
        dx = np.concatenate([da, db], axis=-1)
    return dx, dx.reshape(-1, dx.shape[-1]).sum(axis=0)


# --------------------------------------------------------------------------
# GEMMs and the composite forwards
# --------------------------------------------------------------------------

def dense(x, kernel, bias=None) -> np.ndarray:
    """[DENSE] Outputs: x @ kernel + bias (kernel is [in, out])."""
    y = np.matmul(np.asarray(x, dtype=np.float64), np.asarray(kernel, dtype=np.float64))
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


def fp8_dense(xq, x_meta, wq, w_meta, bias=None) -> np.ndarray:
    """GEMM of two E4M3 operands: the sum of products of decoded codes (exact
    in fp64 for these sizes), times both scale_inv, plus bias. wq is [in, out]."""
    acc = np.matmul(e4m3_decode(xq), e4m3_decode(wq))
    y = acc * x_meta["scale_inv"] * w_meta["scale_inv"]
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y


def layernorm_dense_fwd(x, kernel, gamma, beta, bias=None, norm_type="layernorm",
                        zero_centered_gamma=False, epsilon=1e-6, quant="none",
                        round_intermediates=False):
    """[DENSE] forward: normalization, then (fp8: quantize the normalized output
    and the kernel), then GEMM with optional bias.

    Returns a dict with y and, for fp8, the codes and metas of x and kernel.
    ``round_intermediates`` (diagnostic) rounds the normalized tensor to bf16
    as the bf16 path materialises it."""
    xn, mu, rs = normalize(x, gamma, beta, norm_type, epsilon, zero_centered_gamma)
    out = {"mu": mu, "rsigma": rs, "xn": xn}
    if quant == "none":
        a = bf16_round(xn) if round_intermediates else xn
        out["y"] = dense(a, kernel, bias)
        return out
    xq, xm = quantize(xn)
    wq, wm = quantize(kernel)
    out.update(xq=xq, x_meta=xm, wq=wq, w_meta=wm, y=fp8_dense(xq, xm, wq, wm, bias))
    return out


def layernorm_mlp_fwd(x, gamma, beta, kernel1, kernel2, bias1=None, bias2=None,
                      norm_type="layernorm", zero_centered_gamma=False, epsilon=1e-6,
                      activation_type=("relu",), quant="none", round_intermediates=False,
                      rows: Optional[np.ndarray] = None):
    """[MLP] forward: (1) normalization, (2) GEMM1 + bias1, (3) activation,
    (4) GEMM2 + bias2.

    quant == "none": pure fp64, no intermediate rounding (``round_intermediates``
    rounds the normalized input and the activation output to bf16, as the bf16
    path materialises them, for diagnostics).

    quant == "fp8_e4m3_current": the normalized x, both kernels and the
    activation output are quantized with per-tensor current scaling; the GEMM1
    result plus bias1 is kept as bf16 (the saved pre-activation h1) and the
    activation is evaluated from that bf16 h1.

    ``rows`` restricts the returned outputs to a subset of rows; whole-tensor
    amaxes are still taken over every row, as the method requires.
    """
    xn, mu, rs = normalize(x, gamma, beta, norm_type, epsilon, zero_centered_gamma)
    out = {"mu": mu, "rsigma": rs}
    sel = slice(None) if rows is None else rows
    if quant == "none":
        a_in = bf16_round(xn[sel]) if round_intermediates else xn[sel]
        h = dense(a_in, kernel1, bias1)
        act = activation(h, activation_type)
        if round_intermediates:
            act = bf16_round(act)
        out.update(h=h, act=act, y=dense(act, kernel2, bias2))
        return out
    xq, xm = quantize(xn)
    w1q, w1m = quantize(kernel1)
    w2q, w2m = quantize(kernel2)
    h1 = bf16_round(fp8_dense(xq, xm, w1q, w1m, bias1))
    act = activation(h1, activation_type)
    aq, am = quantize(act)
    y = fp8_dense(aq[sel], am, w2q, w2m, bias2)
    out.update(xq=xq, x_meta=xm, w1q=w1q, w1_meta=w1m, w2q=w2q, w2_meta=w2m,
               h1=h1[sel], act=act[sel], actq=aq[sel], act_meta=am, y=y)
    return out


def layernorm_mlp_bwd(grad, x, gamma, beta, kernel1, kernel2, bias1=None, bias2=None,
                      norm_type="layernorm", zero_centered_gamma=False, epsilon=1e-6,
                      activation_type=("relu",), h1=None, round_intermediates=False):
    """[MLP] Description: the backward pass gives the gradients of every
    parameter through fused backward operations (the activation gradient
    with the bias reduction); [DENSE] Description: gradients for x, kernel,
    gamma, beta and bias from the saved forward context. With xn the
    normalized input, h = xn @ kernel1 + bias1, act = activation(h) and
    grad = dL/dy:
      dkernel2 = act^T @ grad,   dbias2 = sum over rows of grad
      dact = grad @ kernel2^T,   dh, dbias1 = dact_dbias(dact, h)
      dkernel1 = xn^T @ dh,      dxn = dh @ kernel1^T
      dx, dgamma, dbeta = norm_bwd(dxn, x, ...)
    ``h1`` (optional) replaces h by the saved pre-activation.
    ``round_intermediates`` rounds the tensors a bf16 forward/backward pair
    materialises to bf16: xn, the saved pre-activation h, act, dact, dh and
    dxn.
    Returns a dict with dx, dgamma, dbeta (None for RMSNorm), dkernel1,
    dbias1, dkernel2, dbias2."""
    r = bf16_round if round_intermediates else (lambda t: t)
    grad = np.asarray(grad, dtype=np.float64)
    kernel1 = np.asarray(kernel1, dtype=np.float64)
    kernel2 = np.asarray(kernel2, dtype=np.float64)
    xn = normalize(x, gamma, beta, norm_type, epsilon, zero_centered_gamma)[0]
    h = np.asarray(h1, dtype=np.float64) if h1 is not None else r(dense(r(xn), kernel1, bias1))
    act = r(activation(h, activation_type))
    dkernel2 = np.matmul(act.T, grad)
    dbias2 = grad.sum(axis=0)
    dact = r(np.matmul(grad, kernel2.T))
    dh, dbias1 = dact_dbias(dact, h, activation_type)
    dh = r(dh)
    dkernel1 = np.matmul(r(xn).T, dh)
    dxn = r(np.matmul(dh, kernel1.T))
    dx, dgamma, dbeta = norm_bwd(dxn, x, gamma, norm_type, epsilon, zero_centered_gamma)
    return {"dx": dx, "dgamma": dgamma, "dbeta": dbeta, "dkernel1": dkernel1, "dbias1": dbias1,
            "dkernel2": dkernel2, "dbias2": dbias2}


def rel_l2(got, ref) -> float:
    """Relative L2 error ||got - ref|| / ||ref|| over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((got - ref).ravel()))
    return num / den if den > 0 else num
