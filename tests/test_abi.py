"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest
import torch

import rmsnorm_mlp_transformer_amd as te
from rmsnorm_mlp_transformer_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "te_mi355x.h")

# Fake, 16-byte aligned device addresses: only ever passed to calls that must
# fail validation (the tests below are skipped where a GPU is present, so a
# call that unexpectedly passed validation could never reach a real device).
P = 0x10000
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="validation probes use fake pointers")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(te_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_version():
    assert os.path.exists(te.LIB_PATH)
    assert te.te_version().startswith("temi355x")


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) >= 16, names
    lib = ctypes.CDLL(te.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(te.EXPORTED), set(names) ^ set(te.EXPORTED)


def test_struct_layouts_match_header():
    # te_fp8_meta: 3 pointers; te_mlp_saved: 3 pointers + 4 metas + 4 code pointers
    assert ctypes.sizeof(B.te_fp8_meta) == 24
    assert ctypes.sizeof(B.te_mlp_saved) == 8 * (3 + 12 + 4)


def _mlp(**kw):
    args = dict(x=P, gamma=P, beta=P, k1=P, b1=None, k2=P, b2=None, rows=8, hidden=64, ffn=128,
                dtype=B.TE_BF16, norm=B.TE_LAYERNORM, zcg=0, eps=1e-6, act=B.TE_ACT_GELU,
                quant=B.TE_QUANT_NONE, y=P, y_dtype=None, saved=None, ws=P, ws_bytes=1 << 30)
    args.update(kw)
    y_dtype = args["dtype"] if args["y_dtype"] is None else args["y_dtype"]
    return B._lib.te_layernorm_mlp_fwd(args["x"], args["gamma"], args["beta"], args["k1"], args["b1"],
                                       args["k2"], args["b2"], args["rows"], args["hidden"], args["ffn"],
                                       args["dtype"], args["norm"], args["zcg"], args["eps"], args["act"],
                                       args["quant"], args["y"], y_dtype, args["saved"], args["ws"],
                                       args["ws_bytes"], None)


@no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(gamma=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(beta=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(k1=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(k2=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(y=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(hidden=40), B.TE_ERR_INVALID_ARGUMENT),
    (dict(hidden=0), B.TE_ERR_INVALID_ARGUMENT),
    (dict(ffn=24), B.TE_ERR_INVALID_ARGUMENT),
    (dict(rows=-1), B.TE_ERR_INVALID_ARGUMENT),
    (dict(norm=7), B.TE_ERR_INVALID_ARGUMENT),
    (dict(act=99), B.TE_ERR_INVALID_ARGUMENT),
    (dict(dtype=9), B.TE_ERR_INVALID_ARGUMENT),
    (dict(quant=5), B.TE_ERR_INVALID_ARGUMENT),
    (dict(eps=-1.0), B.TE_ERR_INVALID_ARGUMENT),
    (dict(x=P + 4), B.TE_ERR_INVALID_ARGUMENT),
    (dict(b1=P + 8), B.TE_ERR_INVALID_ARGUMENT),
    (dict(dtype=B.TE_F32, quant=B.TE_QUANT_FP8_E4M3_CURRENT), B.TE_ERR_UNSUPPORTED),
    (dict(dtype=B.TE_E4M3), B.TE_ERR_UNSUPPORTED),
    (dict(ws_bytes=100), B.TE_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=None), B.TE_ERR_INVALID_ARGUMENT),
    (dict(y_dtype=7), B.TE_ERR_INVALID_ARGUMENT),
    (dict(y_dtype=B.TE_E4M3), B.TE_ERR_UNSUPPORTED),
    (dict(dtype=B.TE_F32, y_dtype=B.TE_BF16), B.TE_ERR_UNSUPPORTED),
    # one size past the largest accepted: a 2 GiB kernel (plain, then gated),
    # and features beyond 2^22
    (dict(hidden=256, ffn=1 << 22), B.TE_ERR_UNSUPPORTED),
    (dict(hidden=4096, ffn=1 << 17, act=B.TE_ACT_SWIGLU), B.TE_ERR_UNSUPPORTED),
    (dict(hidden=16, ffn=(1 << 22) + 16), B.TE_ERR_INVALID_ARGUMENT),
    (dict(hidden=(1 << 22) + 16), B.TE_ERR_INVALID_ARGUMENT),
])
def test_mlp_validation(kw, status):
    assert _mlp(**kw) == status
    assert te.te_last_error() != ""


@no_gpu
def test_mlp_rmsnorm_accepts_null_beta_and_zero_rows_is_a_no_op():
    # rows = 0 succeeds without any HIP call (so it succeeds without a GPU)
    assert _mlp(rows=0) == B.TE_SUCCESS
    assert _mlp(rows=0, beta=None, norm=B.TE_RMSNORM) == B.TE_SUCCESS
    # an empty batch may come with NULL x / y (an empty tensor's data pointer)
    assert _mlp(rows=0, x=None, y=None) == B.TE_SUCCESS
    assert te.te_last_error() == ""
    assert _mlp(rows=1, x=None) == B.TE_ERR_INVALID_ARGUMENT


@no_gpu
def test_valid_call_without_gpu_maps_to_hip_error():
    # passes validation, then the launch fails: TE_ERR_HIP with a message
    st = _mlp()
    assert st == B.TE_ERR_HIP
    assert te.te_last_error() != ""
    # fp32 output from bf16 inputs is a supported combination (plain and fp8)
    assert _mlp(y_dtype=B.TE_F32) == B.TE_ERR_HIP
    assert _mlp(y_dtype=B.TE_F32, quant=B.TE_QUANT_FP8_E4M3_CURRENT) == B.TE_ERR_HIP


@no_gpu
def test_dense_validation():
    def call(**kw):
        a = dict(x=P, k=P, g=P, b=P, bias=None, rows=4, hidden=32, out=48, dtype=B.TE_BF16,
                 norm=B.TE_LAYERNORM, quant=B.TE_QUANT_NONE, y=P, y_dtype=None, ws=P, wsb=1 << 30)
        a.update(kw)
        return B._lib.te_layernorm_dense_fwd(a["x"], a["k"], a["g"], a["b"], a["bias"], a["rows"],
                                             a["hidden"], a["out"], a["dtype"], a["norm"], 0, 1e-5,
                                             a["quant"], a["y"], a["dtype"] if a["y_dtype"] is None else a["y_dtype"],
                                             a["ws"], a["wsb"], None)
    assert call(out=40) == B.TE_ERR_INVALID_ARGUMENT
    assert call(k=None) == B.TE_ERR_INVALID_ARGUMENT
    assert call(b=None) == B.TE_ERR_INVALID_ARGUMENT
    assert call(dtype=B.TE_F32, quant=B.TE_QUANT_FP8_E4M3_CURRENT) == B.TE_ERR_UNSUPPORTED
    assert call(wsb=0) == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert call(y_dtype=B.TE_E4M3) == B.TE_ERR_UNSUPPORTED
    assert call(dtype=B.TE_F32, y_dtype=B.TE_BF16) == B.TE_ERR_UNSUPPORTED
    assert call(y_dtype=-1) == B.TE_ERR_INVALID_ARGUMENT
    assert call(rows=0) == B.TE_SUCCESS
    assert call(rows=0, y_dtype=B.TE_F32) == B.TE_SUCCESS


@no_gpu
def test_norm_act_dact_quant_validation():
    lib = B._lib
    m = B.te_fp8_meta(P, P + 4, P + 8)
    bad_meta = B.te_fp8_meta(P, None, P + 8)
    # norm
    assert lib.te_layernorm_fwd(P, P, None, 4, 64, B.TE_BF16, B.TE_LAYERNORM, 0, 1e-6, P, B.TE_BF16,
                                None, None, None, None, 0, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_layernorm_fwd(P, P, P, 4, 64, B.TE_BF16, B.TE_LAYERNORM, 0, 1e-6, P, B.TE_E4M3,
                                ctypes.byref(bad_meta), None, None, None, 0, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_layernorm_fwd(P, P, P, 4, 64, B.TE_E4M3, B.TE_LAYERNORM, 0, 1e-6, P, B.TE_BF16,
                                None, None, None, None, 0, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_layernorm_fwd(P, P, None, 0, 64, B.TE_BF16, B.TE_RMSNORM, 0, 1e-6, P, B.TE_BF16,
                                None, None, None, None, 0, None) == B.TE_SUCCESS
    # an E4M3 output needs the amax pass's partials: one float per workgroup
    # (a workgroup takes 4 rows; at most 512 partials)
    assert lib.te_layernorm_fwd_workspace_size(64, 4096, B.TE_BF16, B.TE_BF16) == 0
    assert lib.te_layernorm_fwd_workspace_size(0, 4096, B.TE_BF16, B.TE_E4M3) == 0
    assert lib.te_layernorm_fwd_workspace_size(64, 4096, B.TE_BF16, B.TE_E4M3) == 16 * 4
    assert lib.te_layernorm_fwd_workspace_size(63, 4096, B.TE_BF16, B.TE_E4M3) == 16 * 4
    assert lib.te_layernorm_fwd_workspace_size(1 << 20, 4096, B.TE_BF16, B.TE_E4M3) == 512 * 4
    assert lib.te_layernorm_fwd(P, P, P, 64, 64, B.TE_BF16, B.TE_LAYERNORM, 0, 1e-6, P, B.TE_E4M3,
                                ctypes.byref(m), None, None, P, 63, None) == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert lib.te_layernorm_fwd(P, P, P, 64, 64, B.TE_BF16, B.TE_LAYERNORM, 0, 1e-6, P, B.TE_E4M3,
                                ctypes.byref(m), None, None, None, 64, None) == B.TE_ERR_INVALID_ARGUMENT
    # act
    assert lib.te_act_lu(P, 4, 24, B.TE_BF16, B.TE_ACT_GELU, P, B.TE_BF16, None, None, 0, None) \
        == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_act_lu(P, 4, 32, B.TE_BF16, 9, P, B.TE_BF16, None, None, 0, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_act_lu(P, 4, 32, B.TE_BF16, B.TE_ACT_GELU, P, B.TE_E4M3, None, P, 1 << 20, None) \
        == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_act_lu(None, 4, 32, B.TE_BF16, B.TE_ACT_GELU, P, B.TE_BF16, None, None, 0, None) \
        == B.TE_ERR_INVALID_ARGUMENT
    # E4M3 output needs the partial-maximum workspace; other outputs need none
    assert lib.te_act_lu_workspace_size(64, 32, B.TE_ACT_GELU, B.TE_BF16) == 0
    need_a = lib.te_act_lu_workspace_size(64, 32, B.TE_ACT_GELU, B.TE_E4M3)
    assert need_a >= 4
    assert lib.te_act_lu(P, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, B.TE_E4M3, ctypes.byref(m), P, need_a - 1, None) \
        == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert lib.te_act_lu(P, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, B.TE_E4M3, ctypes.byref(m), None, need_a, None) \
        == B.TE_ERR_INVALID_ARGUMENT
    # dact
    need = lib.te_dact_dbias_workspace_size(64, 32, B.TE_ACT_GELU)
    assert need > 0
    assert lib.te_dact_dbias(P, P, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, P, B.TE_F32, P, need - 1, None) \
        == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert lib.te_dact_dbias(P, P, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, P, B.TE_E4M3, P, need, None) \
        == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_dact_dbias(P, None, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, None, B.TE_F32, None, 0, None) \
        == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_dact_dbias(P, P, 0, 32, B.TE_BF16, B.TE_ACT_SWIGLU, P, None, B.TE_F32, None, 0, None) \
        == B.TE_SUCCESS
    # quantised dact
    needq = lib.te_dact_dbias_quantize_workspace_size(64, 32, B.TE_ACT_GELU)
    assert needq > need
    assert lib.te_dact_dbias_quantize(P, P, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, ctypes.byref(m), P, B.TE_F32, P,
                                      needq - 1, None) == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert lib.te_dact_dbias_quantize(P, P, 64, 32, B.TE_BF16, B.TE_ACT_GELU, P, None, P, B.TE_F32, P, needq,
                                      None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_dact_dbias_quantize(P, P, 64, 24, B.TE_BF16, B.TE_ACT_GELU, P, ctypes.byref(m), P, B.TE_F32, P,
                                      needq, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_dact_dbias_quantize(P, P, 64, 32, B.TE_E4M3, B.TE_ACT_GELU, P, ctypes.byref(m), P, B.TE_F32, P,
                                      needq, None) == B.TE_ERR_INVALID_ARGUMENT
    # normalisation backward
    nb = lib.te_layernorm_bwd_workspace_size(64, 4096, B.TE_BF16)
    assert nb > 0
    assert lib.te_layernorm_bwd(P, P, P, P, P, 64, 4096, B.TE_BF16, B.TE_LAYERNORM, 0, P, P, P, B.TE_F32, P, nb - 1,
                                None) == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert lib.te_layernorm_bwd(P, P, None, P, P, 64, 4096, B.TE_BF16, B.TE_LAYERNORM, 0, P, P, P, B.TE_F32, P, nb,
                                None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_layernorm_bwd(P, P, P, P, P, 64, 32768, B.TE_BF16, B.TE_LAYERNORM, 0, P, P, P, B.TE_F32, P, 1 << 30,
                                None) == B.TE_ERR_UNSUPPORTED
    assert lib.te_layernorm_bwd(P, P, P, P, P, 64, 16384, B.TE_F32, B.TE_RMSNORM, 0, P, P, None, B.TE_F32, P, 1 << 30,
                                None) == B.TE_ERR_UNSUPPORTED
    assert lib.te_layernorm_bwd(P, P, P, P, P, 64, 40, B.TE_BF16, B.TE_LAYERNORM, 0, P, P, P, B.TE_F32, P, nb,
                                None) == B.TE_ERR_INVALID_ARGUMENT
    # LayerNorm-MLP backward
    nm = lib.te_layernorm_mlp_bwd_workspace_size(256, 512, 1024, B.TE_ACT_GELU)
    assert nm > lib.te_layernorm_mlp_bwd_workspace_size(128, 512, 1024, B.TE_ACT_GELU) > 0
    assert lib.te_layernorm_mlp_bwd_workspace_size(256, 512, 1024, B.TE_ACT_SWIGLU) > nm

    def mlp_bwd(dtype=B.TE_BF16, ffn=1024, act=B.TE_ACT_GELU, mu=P, h1=P, ws=nm, norm=B.TE_LAYERNORM):
        return lib.te_layernorm_mlp_bwd(P, P, P, P, P, P, mu, P, h1, 256, 512, ffn, dtype, norm, 0, 1e-6, act,
                                        P, P, P, P, P, P, P, B.TE_F32, P, ws, None)
    assert mlp_bwd(dtype=B.TE_F32) == B.TE_ERR_UNSUPPORTED
    assert mlp_bwd(ws=nm - 1) == B.TE_ERR_WORKSPACE_TOO_SMALL
    assert mlp_bwd(ffn=1000) == B.TE_ERR_INVALID_ARGUMENT
    assert mlp_bwd(mu=None) == B.TE_ERR_INVALID_ARGUMENT
    assert mlp_bwd(h1=None) == B.TE_ERR_INVALID_ARGUMENT
    assert mlp_bwd(act=99) == B.TE_ERR_INVALID_ARGUMENT
    # quantiser
    assert lib.te_quantize(P, 24, B.TE_BF16, P, ctypes.byref(m), None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_quantize(P, 32, B.TE_BF16, P, None, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_dequantize(P, 32, ctypes.byref(m), P, B.TE_E4M3, None) == B.TE_ERR_INVALID_ARGUMENT


def test_workspace_sizes_cover_the_buffers():
    lib = B._lib
    r, h, f = 8192, 4096, 16384
    bf16 = lib.te_layernorm_mlp_fwd_workspace_size(r, h, f, B.TE_BF16, B.TE_ACT_GELU, B.TE_QUANT_NONE)
    assert bf16 >= r * h * 2 + r * f * 2
    fp8 = lib.te_layernorm_mlp_fwd_workspace_size(r, h, f, B.TE_BF16, B.TE_ACT_GELU, B.TE_QUANT_FP8_E4M3_CURRENT)
    assert fp8 >= r * h + 2 * h * f + r * f * 2 + r * f
    gated = lib.te_layernorm_mlp_fwd_workspace_size(r, h, f, B.TE_BF16, B.TE_ACT_SWIGLU,
                                                     B.TE_QUANT_FP8_E4M3_CURRENT)
    assert gated > fp8
    d = lib.te_layernorm_dense_fwd_workspace_size(4096, 4096, 12288, B.TE_BF16, B.TE_QUANT_FP8_E4M3_CURRENT)
    assert d >= 4096 * 4096 + 4096 * 12288 + 512 * 4
    assert fp8 >= r * h + 2 * h * f + r * f * 2 + r * f + 512 * 4
    assert lib.te_layernorm_mlp_fwd_workspace_size(100, 64, 128, B.TE_F32, B.TE_ACT_RELU, B.TE_QUANT_NONE) \
        < lib.te_layernorm_mlp_fwd_workspace_size(200, 64, 128, B.TE_F32, B.TE_ACT_RELU, B.TE_QUANT_NONE)


def test_workspace_sizes_hold_the_tiled_operands():
    """The GEMM operands kept in the workspace are stored as 16 KiB blocks of
    256 rows x 64 bytes, a partial row tile or k stage taking a whole block
    (the gated GEMM1's transposed kernel: tiles of 128 rows of each half), so
    the sizes cover the padded blocks."""
    lib = B._lib
    blk = 16384

    def tiled(rows, row_bytes, tile_rows=256):
        return -(-rows // tile_rows) * -(-row_bytes // 64) * blk

    r, h, f = 300, 80, 144
    bf16 = lib.te_layernorm_mlp_fwd_workspace_size(r, h, f, B.TE_BF16, B.TE_ACT_GELU, B.TE_QUANT_NONE)
    assert bf16 >= tiled(r, 2 * h) + tiled(r, 2 * f) == (6 + 10) * blk
    fp8 = lib.te_layernorm_mlp_fwd_workspace_size(r, h, f, B.TE_BF16, B.TE_ACT_SWIGLU, B.TE_QUANT_FP8_E4M3_CURRENT)
    assert fp8 >= tiled(r, h) + tiled(f, h, 128) + tiled(h, f) + r * 2 * f * 2 + tiled(r, f)
    d = lib.te_layernorm_dense_fwd_workspace_size(r, h, 528, B.TE_BF16, B.TE_QUANT_FP8_E4M3_CURRENT)
    assert d >= tiled(r, h) + tiled(528, h)
    # fp32 operands stay row-major
    assert lib.te_layernorm_mlp_fwd_workspace_size(r, h, f, B.TE_F32, B.TE_ACT_GELU, B.TE_QUANT_NONE) \
        < tiled(r, 4 * h) + tiled(r, 4 * f)


def test_timing_api_without_launches():
    te.te_timing_reset()
    te.te_timing_enable(True)
    assert te.te_timing_collect() == {}
    te.te_timing_enable(False)
    with pytest.raises(te.TEError):
        B._check(B._lib.te_timing_get(0, None, None, None))


def test_act_type_names():
    assert te.act_type_of(("silu", "linear")) == B.TE_ACT_SWIGLU
    assert te.act_type_of(("gelu_erf", "linear")) == B.TE_ACT_GEGLU_ERF
    assert B.is_gated(B.TE_ACT_GEGLU_ERF) and not B.is_gated(B.TE_ACT_GELU_ERF)
    assert te.act_type_of("gelu") == B.TE_ACT_GELU
    with pytest.raises(ValueError):
        te.act_type_of(("tanh",))


def test_mfma_probe_rejects_bad_arguments():
    """The probe's argument checks run before any GPU work."""
    lib = B._lib
    assert lib.te_probe_mfma(0, 0, 4, 1, None, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_probe_mfma(0, 10, 0, 1, None, None) == B.TE_ERR_INVALID_ARGUMENT
    assert lib.te_probe_mfma(1, 10, 4, None, None, None) == B.TE_ERR_INVALID_ARGUMENT


def test_host_tensors_are_rejected_before_any_launch():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensors"):
        te.layernorm(x, g, torch.zeros_like(g))
    with pytest.raises(ValueError, match="GPU tensors"):
        te.activation(x, ("gelu",))
