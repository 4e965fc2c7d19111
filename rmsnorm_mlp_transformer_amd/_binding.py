"""ctypes binding of libtemi355x.so.

Argument marshalling only: torch tensors supply device memory and the
current stream; every step of the computation runs in the library's HIP
kernels. Importing this module fails loudly when the library has not been
built (there is no fallback path).

The ``te_*`` functions mirror the C ABI one to one (same names, same
argument order). ``layernorm_mlp``, ``layernorm_dense``, ``activation``,
``dact_dbias`` and ``layernorm`` follow the signatures and defaults of the
TransformerEngine JAX pages ("NVIDIA TransformerEngine JAX LayerNorm MLP",
"... LayerNorm Dense", "... Activation", Code Reference: Signature) and
allocate their outputs with torch.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtemi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first with "
        "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- enums
TE_SUCCESS, TE_ERR_INVALID_ARGUMENT, TE_ERR_UNSUPPORTED, TE_ERR_WORKSPACE_TOO_SMALL, TE_ERR_HIP = range(5)
TE_F32, TE_BF16, TE_E4M3 = 0, 1, 2
TE_LAYERNORM, TE_RMSNORM = 0, 1
(TE_ACT_RELU, TE_ACT_GELU, TE_ACT_GELU_ERF, TE_ACT_SILU, TE_ACT_LINEAR,
 TE_ACT_REGLU, TE_ACT_GEGLU, TE_ACT_SWIGLU, TE_ACT_GEGLU_ERF) = range(9)
TE_QUANT_NONE, TE_QUANT_FP8_E4M3_CURRENT = 0, 1

_NORM = {"layernorm": TE_LAYERNORM, "rmsnorm": TE_RMSNORM}
_ACT = {
    ("relu",): TE_ACT_RELU, ("gelu",): TE_ACT_GELU, ("gelu_erf",): TE_ACT_GELU_ERF,
    ("silu",): TE_ACT_SILU, ("linear",): TE_ACT_LINEAR,
    ("relu", "linear"): TE_ACT_REGLU, ("gelu", "linear"): TE_ACT_GEGLU,
    ("silu", "linear"): TE_ACT_SWIGLU, ("gelu_erf", "linear"): TE_ACT_GEGLU_ERF,
}
_DTYPE = {torch.float32: TE_F32, torch.bfloat16: TE_BF16, torch.uint8: TE_E4M3,
          torch.float8_e4m3fn: TE_E4M3}


class TEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"te status {status}: {message}")
        self.status = status


# ---------------------------------------------------------------- C structs
class te_fp8_meta(ctypes.Structure):
    _fields_ = [("amax", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("scale_inv", ctypes.c_void_p)]


class te_mlp_saved(ctypes.Structure):
    _fields_ = [("h1", ctypes.c_void_p), ("mu", ctypes.c_void_p), ("rsigma", ctypes.c_void_p),
                ("x_meta", te_fp8_meta), ("w1_meta", te_fp8_meta),
                ("act_meta", te_fp8_meta), ("w2_meta", te_fp8_meta),
                ("xq", ctypes.c_void_p), ("w1q_t", ctypes.c_void_p), ("w2q_t", ctypes.c_void_p),
                ("actq", ctypes.c_void_p)]


_vp, _i64, _sz, _int, _f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
_meta_p = ctypes.POINTER(te_fp8_meta)
_saved_p = ctypes.POINTER(te_mlp_saved)

_SIGS = {
    "te_layernorm_fwd": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _f, _vp, _int, _meta_p,
                                _vp, _vp, _vp, _sz, _vp]),
    "te_layernorm_fwd_workspace_size": (_sz, [_i64, _i64, _int, _int]),
    "te_layernorm_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _int,
                                _vp, _sz, _vp]),
    "te_layernorm_bwd_workspace_size": (_sz, [_i64, _i64, _int]),
    "te_act_lu": (_int, [_vp, _i64, _i64, _int, _int, _vp, _int, _meta_p, _vp, _sz, _vp]),
    "te_act_lu_workspace_size": (_sz, [_i64, _i64, _int, _int]),
    "te_dact_dbias": (_int, [_vp, _vp, _i64, _i64, _int, _int, _vp, _vp, _int, _vp, _sz, _vp]),
    "te_dact_dbias_workspace_size": (_sz, [_i64, _i64, _int]),
    "te_dact_dbias_noalloc": (_int, [_vp, _vp, _i64, _i64, _int, _int, _vp, _vp, _int, _vp]),
    "te_dact_dbias_noalloc_scratch_bytes": (_sz, []),
    "te_dact_dbias_quantize": (_int, [_vp, _vp, _i64, _i64, _int, _int, _vp, _meta_p, _vp, _int, _vp, _sz, _vp]),
    "te_dact_dbias_quantize_workspace_size": (_sz, [_i64, _i64, _int]),
    "te_layernorm_dense_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _f,
                                      _int, _vp, _int, _vp, _sz, _vp]),
    "te_layernorm_dense_fwd_workspace_size": (_sz, [_i64, _i64, _i64, _int, _int]),
    "te_layernorm_mlp_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                    _int, _f, _int, _int, _vp, _int, _saved_p, _vp, _sz, _vp]),
    "te_layernorm_mlp_fwd_workspace_size": (_sz, [_i64, _i64, _i64, _int, _int, _int]),
    "te_layernorm_mlp_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                    _int, _f, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _sz, _vp]),
    "te_layernorm_mlp_bwd_workspace_size": (_sz, [_i64, _i64, _i64, _int]),
    "te_quantize": (_int, [_vp, _i64, _int, _vp, _meta_p, _vp]),
    "te_dequantize": (_int, [_vp, _i64, _meta_p, _vp, _int, _vp]),
    "te_probe_mfma": (_int, [_int, _i64, _int, _vp, _vp, _vp]),
    "te_last_error": (ctypes.c_char_p, []),
    "te_version": (ctypes.c_char_p, []),
    "te_timing_enable": (_int, [_int]),
    "te_timing_collect": (_int, []),
    "te_timing_get": (_int, [_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_i64),
                             ctypes.POINTER(ctypes.c_double)]),
    "te_timing_reset": (None, []),
}
EXPORTED = tuple(_SIGS)

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(status: int) -> None:
    if status != TE_SUCCESS:
        raise TEError(status, _lib.te_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    # the kernels run on the current device and dereference every pointer there
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must be GPU tensors")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:   # a torch stream, or a raw hipStream_t handle (0 = null stream)
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def act_type_of(activation_type: Union[str, Sequence[str], int]) -> int:
    if isinstance(activation_type, int):
        return activation_type
    key = (activation_type,) if isinstance(activation_type, str) else tuple(activation_type)
    if key not in _ACT:
        raise ValueError(f"unsupported activation_type {activation_type!r}")
    return _ACT[key]


def is_gated(act: int) -> bool:
    return act >= TE_ACT_REGLU


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- fp8 metadata
class Fp8Meta:
    """Device storage for one tensor's amax, scale and scale_inv (fp32)."""

    def __init__(self, device="cuda"):
        self.buf = torch.zeros(4, dtype=torch.float32, device=device)

    def c(self) -> te_fp8_meta:
        p = self.buf.data_ptr()
        return te_fp8_meta(p, p + 4, p + 8)

    def values(self):
        a, s, si, _ = self.buf.tolist()
        return {"amax": a, "scale": s, "scale_inv": si}


class QuantizerSet:
    """Per-tensor E4M3 current scaling for the norm-MLP / norm-dense calls
    ("... LayerNorm MLP" and "... LayerNorm Dense", Inputs: quantizer_set).
    After a call the metas hold the amax / scale / scale_inv of the
    normalised input (x), the kernels (w1, w2 or kernel) and the
    activation output (act)."""

    recipe = TE_QUANT_FP8_E4M3_CURRENT

    def __init__(self, device="cuda"):
        self.x = Fp8Meta(device)
        self.w1 = Fp8Meta(device)
        self.act = Fp8Meta(device)
        self.w2 = Fp8Meta(device)


noop_quantizer_set = None


# ---------------------------------------------------------------- C ABI, one to one
def te_layernorm_fwd(x, gamma, beta, rows, hidden, x_dtype, norm_type, zero_centered_gamma, epsilon,
                     y, y_dtype, y_meta=None, mu=None, rsigma=None, workspace=None, workspace_bytes=0,
                     stream=None):
    _check(_lib.te_layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), rows, hidden, x_dtype, norm_type,
                                 int(zero_centered_gamma), float(epsilon), _ptr(y), y_dtype,
                                 ctypes.byref(y_meta.c()) if y_meta is not None else None,
                                 _ptr(mu), _ptr(rsigma), _ptr(workspace), workspace_bytes, _stream(stream)))


def te_layernorm_fwd_workspace_size(rows, hidden, x_dtype, y_dtype) -> int:
    return _lib.te_layernorm_fwd_workspace_size(rows, hidden, x_dtype, y_dtype)


def te_layernorm_bwd_workspace_size(rows, hidden, dtype) -> int:
    return _lib.te_layernorm_bwd_workspace_size(rows, hidden, dtype)


def te_layernorm_bwd(dy, x, mu, rsigma, gamma, rows, hidden, dtype, norm_type, zero_centered_gamma, dx, dgamma,
                     dbeta, dparam_dtype, workspace, workspace_bytes, stream=None):
    _check(_lib.te_layernorm_bwd(_ptr(dy), _ptr(x), _ptr(mu), _ptr(rsigma), _ptr(gamma), rows, hidden, dtype,
                                 norm_type, int(zero_centered_gamma), _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                                 dparam_dtype, _ptr(workspace), workspace_bytes, _stream(stream)))


def te_act_lu_workspace_size(rows, cols, act_type, y_dtype) -> int:
    return _lib.te_act_lu_workspace_size(rows, cols, act_type, y_dtype)


def te_act_lu(x, rows, cols, x_dtype, act_type, y, y_dtype, y_meta=None, workspace=None, workspace_bytes=0,
              stream=None):
    _check(_lib.te_act_lu(_ptr(x), rows, cols, x_dtype, act_type, _ptr(y), y_dtype,
                          ctypes.byref(y_meta.c()) if y_meta is not None else None, _ptr(workspace),
                          workspace_bytes, _stream(stream)))


def te_dact_dbias_workspace_size(rows, cols, act_type) -> int:
    return _lib.te_dact_dbias_workspace_size(rows, cols, act_type)


def te_dact_dbias(grad, x, rows, cols, dtype, act_type, dx, dbias, dbias_dtype, workspace,
                  workspace_bytes, stream=None):
    _check(_lib.te_dact_dbias(_ptr(grad), _ptr(x), rows, cols, dtype, act_type, _ptr(dx), _ptr(dbias),
                              dbias_dtype, _ptr(workspace), workspace_bytes, _stream(stream)))


def te_dact_dbias_noalloc(grad, x, rows, cols, dtype, act_type, dx, dbias, dbias_dtype, stream=None):
    _check(_lib.te_dact_dbias_noalloc(_ptr(grad), _ptr(x), rows, cols, dtype, act_type, _ptr(dx), _ptr(dbias),
                                      dbias_dtype, _stream(stream)))


def te_dact_dbias_quantize_workspace_size(rows, cols, act_type) -> int:
    return _lib.te_dact_dbias_quantize_workspace_size(rows, cols, act_type)


def te_dact_dbias_quantize(grad, x, rows, cols, dtype, act_type, dx_codes, dx_meta: "Fp8Meta", dbias,
                           dbias_dtype, workspace, workspace_bytes, stream=None):
    _check(_lib.te_dact_dbias_quantize(_ptr(grad), _ptr(x), rows, cols, dtype, act_type, _ptr(dx_codes),
                                       ctypes.byref(dx_meta.c()), _ptr(dbias), dbias_dtype, _ptr(workspace),
                                       workspace_bytes, _stream(stream)))


def te_layernorm_dense_fwd_workspace_size(rows, hidden, out_features, dtype, quant) -> int:
    return _lib.te_layernorm_dense_fwd_workspace_size(rows, hidden, out_features, dtype, quant)


def te_layernorm_dense_fwd(x, kernel, gamma, beta, bias, rows, hidden, out_features, dtype, norm_type,
                           zero_centered_gamma, epsilon, quant, y, y_dtype, workspace, workspace_bytes, stream=None):
    _check(_lib.te_layernorm_dense_fwd(_ptr(x), _ptr(kernel), _ptr(gamma), _ptr(beta), _ptr(bias), rows,
                                       hidden, out_features, dtype, norm_type, int(zero_centered_gamma),
                                       float(epsilon), quant, _ptr(y), y_dtype, _ptr(workspace), workspace_bytes,
                                       _stream(stream)))


def te_layernorm_mlp_fwd_workspace_size(rows, hidden, ffn, dtype, act_type, quant) -> int:
    return _lib.te_layernorm_mlp_fwd_workspace_size(rows, hidden, ffn, dtype, act_type, quant)


def make_saved(h1=None, mu=None, rsigma=None, qset: Optional[QuantizerSet] = None, xq=None,
               w1q_t=None, w2q_t=None, actq=None) -> te_mlp_saved:
    s = te_mlp_saved()
    s.h1, s.mu, s.rsigma = _ptr(h1), _ptr(mu), _ptr(rsigma)
    s.xq, s.w1q_t, s.w2q_t, s.actq = _ptr(xq), _ptr(w1q_t), _ptr(w2q_t), _ptr(actq)
    if qset is not None:
        s.x_meta, s.w1_meta, s.act_meta, s.w2_meta = qset.x.c(), qset.w1.c(), qset.act.c(), qset.w2.c()
    return s


def te_layernorm_mlp_fwd(x, gamma, beta, kernel1, bias1, kernel2, bias2, rows, hidden, ffn, dtype,
                         norm_type, zero_centered_gamma, epsilon, act_type, quant, y, y_dtype, saved=None,
                         workspace=None, workspace_bytes=0, stream=None):
    _check(_lib.te_layernorm_mlp_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(kernel1), _ptr(bias1),
                                     _ptr(kernel2), _ptr(bias2), rows, hidden, ffn, dtype, norm_type,
                                     int(zero_centered_gamma), float(epsilon), act_type, quant, _ptr(y), y_dtype,
                                     ctypes.byref(saved) if saved is not None else None,
                                     _ptr(workspace), workspace_bytes, _stream(stream)))


def te_layernorm_mlp_bwd_workspace_size(rows, hidden, ffn, act_type) -> int:
    return _lib.te_layernorm_mlp_bwd_workspace_size(rows, hidden, ffn, act_type)


def te_layernorm_mlp_bwd(grad, x, gamma, beta, kernel1, kernel2, mu, rsigma, h1, rows, hidden, ffn, dtype, norm_type,
                         zero_centered_gamma, epsilon, act_type, dx, dgamma, dbeta, dkernel1, dbias1, dkernel2, dbias2,
                         dparam_dtype, workspace, workspace_bytes, stream=None):
    _check(_lib.te_layernorm_mlp_bwd(_ptr(grad), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(kernel1), _ptr(kernel2),
                                     _ptr(mu), _ptr(rsigma), _ptr(h1), rows, hidden, ffn, dtype, norm_type,
                                     int(zero_centered_gamma), epsilon, act_type, _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                                     _ptr(dkernel1), _ptr(dbias1), _ptr(dkernel2), _ptr(dbias2), dparam_dtype,
                                     _ptr(workspace), workspace_bytes, _stream(stream)))


def te_quantize(x, n, x_dtype, codes, meta: Fp8Meta, stream=None):
    _check(_lib.te_quantize(_ptr(x), n, x_dtype, _ptr(codes), ctypes.byref(meta.c()), _stream(stream)))


def te_dequantize(codes, n, meta: Fp8Meta, y, y_dtype, stream=None):
    _check(_lib.te_dequantize(_ptr(codes), n, ctypes.byref(meta.c()), _ptr(y), y_dtype, _stream(stream)))


def probe_mfma(fp8: bool, iters: int, blocks: int, device="cuda:0"):
    """Runs the MFMA issue-rate probe (te_probe_mfma) once on the current
    stream; returns (milliseconds, flops, shader-clock ticks, 100 MHz
    reference ticks) of the launch."""
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    ticks = torch.zeros(2, dtype=torch.int64, device=device)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    _check(_lib.te_probe_mfma(1 if fp8 else 0, iters, blocks, sink.data_ptr(), ticks.data_ptr(), _stream()))
    stop.record()
    torch.cuda.synchronize()
    flops = blocks * 4 * iters * 4 * (131072 if fp8 else 32768)
    t = ticks.cpu().tolist()
    return start.elapsed_time(stop), flops, t[0], t[1]


def te_version() -> str:
    return _lib.te_version().decode()


def te_last_error() -> str:
    return _lib.te_last_error().decode()


def te_timing_enable(enable: bool = True) -> None:
    _check(_lib.te_timing_enable(int(enable)))


def te_timing_reset() -> None:
    _lib.te_timing_reset()


def te_timing_collect() -> dict:
    """Per-kernel totals {name: (launches, total_ms)} since the last reset."""
    n = _lib.te_timing_collect()
    out = {}
    for i in range(n):
        name, cnt, ms = ctypes.c_char_p(), _i64(), ctypes.c_double()
        _check(_lib.te_timing_get(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)))
        out[name.value.decode()] = (cnt.value, ms.value)
    return out


# ---------------------------------------------------------------- page-style API
def _flat(x: torch.Tensor) -> torch.Tensor:
    return x.reshape(-1, x.shape[-1])


def layernorm(x, gamma, beta=None, norm_type="layernorm", zero_centered_gamma=False, epsilon=1e-6,
              out_dtype=None, quantizer: Optional[Fp8Meta] = None, return_stats=False):
    """The normalisation step on its own. With ``quantizer`` the result is
    the E4M3 codes (uint8) and the quantizer's meta is filled."""
    x2 = _flat(x)
    rows, hidden = x2.shape
    if quantizer is not None:
        y = torch.empty_like(x2, dtype=torch.uint8)
        yd = TE_E4M3
    else:
        y = torch.empty_like(x2, dtype=out_dtype or x.dtype)
        yd = _dtype(y)
    mu = torch.empty(rows, dtype=torch.float32, device=x.device) if return_stats else None
    rs = torch.empty(rows, dtype=torch.float32, device=x.device) if return_stats else None
    nbytes = te_layernorm_fwd_workspace_size(rows, hidden, _dtype(x2), yd)
    ws = _workspace(nbytes, x.device) if nbytes else None
    te_layernorm_fwd(x2, gamma, beta, rows, hidden, _dtype(x2), _NORM[norm_type], zero_centered_gamma,
                     epsilon, y, yd, quantizer, mu, rs, ws, nbytes)
    y = y.reshape(x.shape)
    return (y, mu, rs) if return_stats else y


def layernorm_bwd(dy, x, mu, rsigma, gamma, norm_type="layernorm", zero_centered_gamma=False,
                  dparam_dtype=torch.float32, with_params=True):
    """Gradients of the normalisation from the forward's saved mu / rsigma:
    returns (dx, dgamma, dbeta); dbeta is None for RMSNorm."""
    dy2, x2 = _flat(dy), _flat(x)
    rows, hidden = x2.shape
    dx = torch.empty_like(x2)
    dgamma = torch.empty(hidden, dtype=dparam_dtype, device=x.device) if with_params else None
    dbeta = (torch.empty(hidden, dtype=dparam_dtype, device=x.device)
             if with_params and norm_type == "layernorm" else None)
    nbytes = te_layernorm_bwd_workspace_size(rows, hidden, _dtype(x2))
    ws = _workspace(nbytes, x.device)
    te_layernorm_bwd(dy2, x2, mu, rsigma, gamma, rows, hidden, _dtype(x2), _NORM[norm_type], zero_centered_gamma,
                     dx, dgamma, dbeta, _dtype(dgamma) if dgamma is not None else TE_F32, ws, ws.numel())
    return dx.reshape(x.shape), dgamma, dbeta


def activation(x, activation_type, quantizer: Optional[Fp8Meta] = None, act_params=None):
    """"... JAX Activation" signature. With a quantizer the output is
    quantised to E4M3 and returned dequantised to x's dtype."""
    if act_params is not None:
        raise NotImplementedError("act_params (clamped SwiGLU) is not supported")
    act = act_type_of(activation_type)
    x2 = _flat(x)
    rows = x2.shape[0]
    cols = x2.shape[1] // (2 if is_gated(act) else 1)
    out_shape = (*x.shape[:-1], cols)
    if quantizer is None:
        y = torch.empty(rows, cols, dtype=x.dtype, device=x.device)
        te_act_lu(x2, rows, cols, _dtype(x2), act, y, _dtype(y))
        return y.reshape(out_shape)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    ws = _workspace(te_act_lu_workspace_size(rows, cols, act, TE_E4M3), x.device)
    te_act_lu(x2, rows, cols, _dtype(x2), act, codes, TE_E4M3, quantizer, ws, ws.numel())
    y = torch.empty(rows, cols, dtype=x.dtype, device=x.device)
    te_dequantize(codes, rows * cols, quantizer, y, _dtype(y))
    return y.reshape(out_shape)


def activation_codes(x, activation_type, quantizer: Fp8Meta):
    """act_lu with E4M3 output, returning the raw codes (uint8)."""
    act = act_type_of(activation_type)
    x2 = _flat(x)
    rows = x2.shape[0]
    cols = x2.shape[1] // (2 if is_gated(act) else 1)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    ws = _workspace(te_act_lu_workspace_size(rows, cols, act, TE_E4M3), x.device)
    te_act_lu(x2, rows, cols, _dtype(x2), act, codes, TE_E4M3, quantizer, ws, ws.numel())
    return codes


def dact_dbias(grad, x, activation_type, dbias_dtype=torch.float32, with_dbias=True):
    """Activation backward with the bias reduction: returns (dx, dbias)."""
    act = act_type_of(activation_type)
    g2, x2 = _flat(grad), _flat(x)
    rows, cols = g2.shape
    dx = torch.empty_like(x2)
    dbias = torch.empty(x2.shape[1], dtype=dbias_dtype, device=x.device) if with_dbias else None
    nbytes = te_dact_dbias_workspace_size(rows, cols, act)
    ws = _workspace(nbytes, x.device)
    te_dact_dbias(g2, x2, rows, cols, _dtype(x2), act, dx, dbias,
                  _dtype(dbias) if dbias is not None else TE_F32, ws, ws.numel())
    return dx.reshape(x.shape), dbias


def dact_dbias_quantize(grad, x, activation_type, quantizer: "Fp8Meta", dbias_dtype=torch.float32,
                        with_dbias=True):
    """Activation backward with the bias reduction and the activation gradient
    quantised to E4M3 with current scaling (the quantizer receives amax, scale
    and scale_inv): returns (dx codes as uint8, dbias)."""
    act = act_type_of(activation_type)
    g2, x2 = _flat(grad), _flat(x)
    rows, cols = g2.shape
    codes = torch.empty(x2.shape, dtype=torch.uint8, device=x.device)
    dbias = torch.empty(x2.shape[1], dtype=dbias_dtype, device=x.device) if with_dbias else None
    nbytes = te_dact_dbias_quantize_workspace_size(rows, cols, act)
    ws = _workspace(nbytes, x.device)
    te_dact_dbias_quantize(g2, x2, rows, cols, _dtype(x2), act, codes, quantizer, dbias,
                           _dtype(dbias) if dbias is not None else TE_F32, ws, ws.numel())
    return codes.reshape(x.shape), dbias


def layernorm_dense(x, kernel, gamma, beta, bias=None, norm_type="layernorm", zero_centered_gamma=False,
                    epsilon=1e-6, transpose_batch_sequence=False, layernorm_input_axes=None,
                    dot_input_axes=None, kernel_axes=None, quantizer_set: Optional[QuantizerSet] = None,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None):
    """"... JAX LayerNorm Dense" signature: LayerNorm(x) @ kernel + bias.
    Sharding axes and transpose_batch_sequence do not change the math of a
    single-device call and are accepted for signature compatibility.
    ``out_dtype`` (default x's dtype, or out's) may be float32 for bf16 x."""
    x2 = _flat(x)
    rows, hidden = x2.shape
    outf = kernel.shape[1]
    dt = _dtype(x2)
    quant = TE_QUANT_FP8_E4M3_CURRENT if quantizer_set is not None else TE_QUANT_NONE
    nbytes = te_layernorm_dense_fwd_workspace_size(rows, hidden, outf, dt, quant)
    ws = workspace if workspace is not None and workspace.numel() >= nbytes else _workspace(nbytes, x.device)
    y = out if out is not None else torch.empty(rows, outf, dtype=out_dtype or x.dtype, device=x.device)
    te_layernorm_dense_fwd(x2, kernel, gamma, beta, bias, rows, hidden, outf, dt, _NORM[norm_type],
                           zero_centered_gamma, epsilon, quant, y, _dtype(y), ws, ws.numel())
    return y.reshape(*x.shape[:-1], outf)


def layernorm_mlp(x, gamma, beta, kernels, biases, norm_type, zero_centered_gamma=False, epsilon=1e-6,
                  transpose_batch_sequence=False, norm_input_axes=None, dot_1_input_axes=None,
                  dot_2_input_axes=None, kernel_1_axes=None, kernel_2_axes=None, ffn1_ckpt_name="ffn1",
                  ffn2_ckpt_name="ffn2", activation_type=("relu",),
                  quantizer_set: Optional[QuantizerSet] = None, act_params=None,
                  workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  save_h1: bool = False, return_saved: bool = False, save_codes: bool = False,
                  out_dtype: Optional[torch.dtype] = None):
    """"... JAX LayerNorm MLP" signature: LayerNorm(x) -> GEMM1 + bias1 ->
    activation -> GEMM2 + bias2. ``biases`` may contain None. Sharding axes,
    checkpoint names and transpose_batch_sequence do not change the math of
    a single-device call and are accepted for signature compatibility.
    With ``return_saved`` the result is (y, saved) where saved holds h1 (the
    GEMM1 output plus bias1), mu and rsigma; with ``save_codes`` (fp8) also
    the E4M3 codes xq, w1q_t, w2q_t and actq. ``out_dtype`` (default x's
    dtype, or out's) may be float32 for bf16 x."""
    if act_params is not None:
        raise NotImplementedError("act_params (clamped SwiGLU) is not supported")
    act = act_type_of(activation_type)
    k1, k2 = kernels
    b1, b2 = biases
    x2 = _flat(x)
    rows, hidden = x2.shape
    g = 2 if is_gated(act) else 1
    ffn = k1.shape[1] // g
    dt = _dtype(x2)
    quant = TE_QUANT_FP8_E4M3_CURRENT if quantizer_set is not None else TE_QUANT_NONE
    nbytes = te_layernorm_mlp_fwd_workspace_size(rows, hidden, ffn, dt, act, quant)
    ws = workspace if workspace is not None and workspace.numel() >= nbytes else _workspace(nbytes, x.device)
    y = out if out is not None else torch.empty(rows, hidden, dtype=out_dtype or x.dtype, device=x.device)
    saved_t = {}
    if save_h1 or return_saved:
        saved_t["h1"] = torch.empty(rows, g * ffn, dtype=x.dtype, device=x.device)
    if return_saved:
        saved_t["mu"] = torch.empty(rows, dtype=torch.float32, device=x.device)
        saved_t["rsigma"] = torch.empty(rows, dtype=torch.float32, device=x.device)
    if save_codes and quantizer_set is not None:
        saved_t["xq"] = torch.empty(rows, hidden, dtype=torch.uint8, device=x.device)
        saved_t["w1q_t"] = torch.empty(g * ffn, hidden, dtype=torch.uint8, device=x.device)
        saved_t["w2q_t"] = torch.empty(hidden, ffn, dtype=torch.uint8, device=x.device)
        saved_t["actq"] = torch.empty(rows, ffn, dtype=torch.uint8, device=x.device)
    saved = None
    if saved_t or quantizer_set is not None:
        saved = make_saved(saved_t.get("h1"), saved_t.get("mu"), saved_t.get("rsigma"), quantizer_set,
                           saved_t.get("xq"), saved_t.get("w1q_t"), saved_t.get("w2q_t"),
                           saved_t.get("actq"))
    te_layernorm_mlp_fwd(x2, gamma, beta, k1, b1, k2, b2, rows, hidden, ffn, dt, _NORM[norm_type],
                         zero_centered_gamma, epsilon, act, quant, y, _dtype(y), saved, ws, ws.numel())
    y = y.reshape(*x.shape[:-1], hidden)
    return (y, saved_t) if return_saved else y


def layernorm_mlp_bwd(grad, x, gamma, beta, kernels, saved, norm_type="layernorm", zero_centered_gamma=False,
                      epsilon=1e-6, activation_type=("relu",), dparam_dtype=torch.float32, with_biases=True):
    """Backward of layernorm_mlp from its saved context (``saved`` as returned
    by layernorm_mlp(..., return_saved=True, save_h1=True): h1, mu, rsigma).
    Returns a dict of dx, dgamma, dbeta (None for RMSNorm), dkernel1, dbias1,
    dkernel2, dbias2 (the biases' gradients None without with_biases)."""
    act = act_type_of(activation_type)
    g2, x2 = _flat(grad), _flat(x)
    rows, hidden = x2.shape
    k1, k2 = kernels
    ffn = k2.shape[0]
    dev = x.device
    out = {"dx": torch.empty_like(x2),
           "dgamma": torch.empty(hidden, dtype=dparam_dtype, device=dev),
           "dbeta": torch.empty(hidden, dtype=dparam_dtype, device=dev) if norm_type == "layernorm" else None,
           "dkernel1": torch.empty_like(k1), "dkernel2": torch.empty_like(k2),
           "dbias1": torch.empty(k1.shape[1], dtype=dparam_dtype, device=dev) if with_biases else None,
           "dbias2": torch.empty(hidden, dtype=dparam_dtype, device=dev) if with_biases else None}
    nbytes = te_layernorm_mlp_bwd_workspace_size(rows, hidden, ffn, act)
    ws = _workspace(nbytes, dev)
    te_layernorm_mlp_bwd(g2, x2, gamma, beta, k1, k2, saved["mu"], saved["rsigma"], _flat(saved["h1"]), rows, hidden,
                         ffn, _dtype(x2), _NORM[norm_type], zero_centered_gamma, epsilon, act, out["dx"],
                         out["dgamma"], out["dbeta"], out["dkernel1"], out["dbias1"], out["dkernel2"], out["dbias2"],
                         _dtype(out["dgamma"]), ws, ws.numel())
    out["dx"] = out["dx"].reshape(x.shape)
    return out


def quantize(x, quantizer: Fp8Meta):
    """Per-tensor current-scaling E4M3 codes of x (uint8, same shape)."""
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    te_quantize(x.contiguous(), x.numel(), _dtype(x), codes, quantizer)
    return codes


def dequantize(codes, quantizer: Fp8Meta, dtype=torch.float32):
    y = torch.empty(codes.shape, dtype=dtype, device=codes.device)
    te_dequantize(codes, codes.numel(), quantizer, y, _DTYPE[dtype])
    return y
