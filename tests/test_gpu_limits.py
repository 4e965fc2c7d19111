"""GPU parity at the largest sizes the C ABI accepts, against the fp64 oracle:
rows of 2^22 features (the widest the norm, activation and activation-gradient
entry points take) and GEMM kernels just under 2 GiB, where the 32-bit byte
offsets of the GEMM's operand buffers reach the end of their range. The calls
one size further are rejected on the host (test_abi)."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import TOL, assert_rel, check_codes, check_elementwise, codes_np, dev, f64, to_dev
from tolerances import rounding_bound

pytestmark = pytest.mark.gpu

WIDEST = 1 << 22          # the largest hidden / feature count the entry points accept
LIMIT = 1 << 31           # kernels must be smaller than this many bytes
ACTS = [("gelu",), ("silu", "linear")]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_norm_widest_rows(dtype, norm):
    rows = 3
    print(f"norm {norm} {dtype} {rows}x{WIDEST}", flush=True)
    g = torch.Generator().manual_seed(41)
    dt = W.TORCH_DTYPE[dtype]
    x = (torch.randn(rows, WIDEST, generator=g) * 1.7 + 0.3).to(dt)
    gamma = (torch.randn(WIDEST, generator=g) * 0.1 + 1.0).to(dt)
    beta = (torch.randn(WIDEST, generator=g) * 0.1).to(dt)
    xd, gd, bd = x.to(dev()), gamma.to(dev()), beta.to(dev())
    y, mu, rs = te.layernorm(xd, gd, bd if norm == "layernorm" else None, norm, False, 1e-5,
                             out_dtype=torch.float32, return_stats=True)
    q = te.Fp8Meta()
    codes = te.layernorm(xd, gd, bd if norm == "layernorm" else None, norm, False, 1e-5, quantizer=q) \
        if dtype == "bf16" else None
    torch.cuda.synchronize()
    ry, rmu, rrs = O.normalize(f64(x), f64(gamma), f64(beta), norm, 1e-5, False)
    assert_rel(f64(y), ry, TOL["fp32"], "y fp32")
    assert_rel(f64(rs), rrs, 1e-5, "rsigma")
    if norm == "layernorm":
        assert np.max(np.abs(f64(mu) - rmu)) <= 1e-5 * np.abs(f64(x)).mean()
    if codes is not None:
        rq, rm = O.quantize(ry)
        assert abs(q.values()["amax"] - rm["amax"]) <= 1e-5 * rm["amax"]
        check_codes(codes_np(codes), rq, "xq")


@pytest.mark.parametrize("act", ACTS, ids=["-".join(a) for a in ACTS])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_act_lu_widest_rows(act, dtype):
    rows = 3
    print(f"act_lu {act} {dtype} {rows}x{WIDEST}", flush=True)
    a = W.make_act_inputs(rows, WIDEST, len(act) == 2, dtype, seed=43)
    x = a["x"].to(dev())
    y = te.activation(x, act)
    q = te.Fp8Meta()
    codes = te.activation_codes(x, act, q) if dtype == "bf16" else None
    torch.cuda.synchronize()
    ref = O.activation(f64(a["x"]), act)
    assert_rel(f64(y), ref, TOL[dtype], "act")
    if codes is not None:
        rq, rm = O.quantize(ref)
        assert abs(q.values()["amax"] - rm["amax"]) <= 1e-5 * rm["amax"]
        check_codes(codes_np(codes), rq, "act codes")


@pytest.mark.parametrize("act", ACTS, ids=["-".join(a) for a in ACTS])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_dact_dbias_widest_rows(act, dtype):
    rows = 3
    print(f"dact_dbias {act} {dtype} {rows}x{WIDEST}", flush=True)
    a = W.make_act_inputs(rows, WIDEST, len(act) == 2, dtype, seed=47)
    g, x = a["grad"].to(dev()), a["x"].to(dev())
    dx, db = te.dact_dbias(g, x, act)
    q = te.Fp8Meta()
    codes, dbq = te.dact_dbias_quantize(g, x, act, q)
    torch.cuda.synchronize()
    rdx, rdb = O.dact_dbias(f64(a["grad"]), f64(a["x"]), act)
    assert_rel(f64(dx), rdx, TOL[dtype], "dx")
    assert_rel(f64(db), rdb, 1e-5, "dbias")
    assert torch.equal(dbq, db), "dbias of the quantising variant"
    rq, rm = O.quantize(rdx)
    m = q.values()
    assert abs(m["amax"] - rm["amax"]) <= 1e-5 * rm["amax"], (m, rm)
    assert m["scale"] == float(np.float32(448.0) / np.float32(m["amax"]))
    check_codes(codes_np(codes), rq, "dx codes")


@pytest.mark.parametrize("name,rows,hidden,ffn", [
    # both kernels 8 KiB under 2 GiB, ffn at the widest; the activation is
    # stored row-major (rows of 8 MiB are past the tiled layout's limit)
    ("ln_mlp_gelu_bf16", 40, 256, WIDEST - 16),
    # gated: kernel1 256 KiB under 2 GiB, both GEMMs on the tiled operands
    ("rms_swiglu_bf16", 40, 4096, (1 << 17) - 16),
])
def test_mlp_kernels_just_under_2gib(name, rows, hidden, ffn):
    w = W.WORKLOADS[name].scaled(rows, hidden, ffn)
    k1_bytes = hidden * (2 if w.gated else 1) * ffn * 2
    assert LIMIT - (1 << 20) < k1_bytes < LIMIT
    print(f"layernorm_mlp {w.name} (kernel1 {k1_bytes} bytes)", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    y, saved = te.layernorm_mlp(g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]],
                                [g.get("bias1"), g.get("bias2")], w.norm_type,
                                zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                                activation_type=w.activation_type, return_saved=True)
    torch.cuda.synchronize()
    got, got_h1 = f64(y), f64(saved["h1"])
    del y, saved, g
    torch.cuda.empty_cache()
    f = {k: f64(v) for k, v in t.items()}
    del t
    o = O.layernorm_mlp_fwd(f["x"], f["gamma"], f.get("beta"), f["kernel1"], f["kernel2"], f.get("bias1"),
                            f.get("bias2"), norm_type=w.norm_type, zero_centered_gamma=w.zero_centered_gamma,
                            epsilon=w.epsilon, activation_type=w.activation_type)
    e = assert_rel(got, o["y"], TOL["bf16"], "y")
    m = check_elementwise(got, o["y"], rounding_bound(2), "y")
    check_elementwise(got_h1, o["h"], rounding_bound(1), "h1")
    print(f"  rel_l2 {e:.3e}, max |err| / rms {m:.3e}", flush=True)


# rows of a 256 -> 16384 -> 256 MLP whose [rows, ffn] activation (bf16 h1 and
# act, E4M3 codes) passes 2 GiB and, in bf16, 4 GiB
MANY_ROWS = (1 << 17) + 40
# y of the fp8 forward against the exact one: E4M3 keeps 3 mantissa bits, so a
# value's rounding error is uniform within half a step, a relative rms of at
# most 2^-4 / sqrt(3) = 3.6% (at the bottom of a binade). x-hat, kernel1, the
# activation and kernel2 are rounded independently, the first two through
# GELU's slope (at most 1.13): 3.6% * sqrt(2 * 1.13^2 + 2) = 7.7% at most.
FP8_VS_EXACT = 0.08


def _rows_at_offset_limits(rows, row_bytes):
    """The first and last rows, and the rows on either side of the 2 GiB and
    4 GiB byte offsets of a [rows, row_bytes] buffer."""
    idx = set(range(8)) | set(range(rows - 8, rows))
    for lim in (1 << 31, 1 << 32):
        r = lim // row_bytes
        idx |= set(range(max(r - 8, 0), min(r + 8, rows)))
    return np.array(sorted(idx))


@pytest.mark.parametrize("quant", ["none", "fp8_e4m3_current"])
def test_mlp_activation_past_4gib(quant):
    name = "ln_mlp_gelu_bf16" if quant == "none" else "ln_mlp_gelu_fp8"
    w = W.WORKLOADS[name].scaled(MANY_ROWS, 256, 16384)
    print(f"layernorm_mlp {w.name} {quant}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    idx = _rows_at_offset_limits(w.rows, w.ffn * 2)
    assert idx.max() >= (1 << 32) // (w.ffn * 2)
    it = torch.from_numpy(idx).to(dev())
    kw = dict(return_saved=True)
    if quant != "none":
        q = te.QuantizerSet()
        kw.update(quantizer_set=q, save_codes=True)
    y, saved = te.layernorm_mlp(g["x"], g["gamma"], g["beta"], [g["kernel1"], g["kernel2"]],
                                [g["bias1"], g["bias2"]], w.norm_type, epsilon=w.epsilon,
                                activation_type=w.activation_type, **kw)
    got_y, got_h1 = f64(y[it]), f64(saved["h1"][it])
    codes = {k: codes_np(saved[k]) for k in ("w1q_t", "w2q_t")} if quant != "none" else {}
    if quant != "none":
        codes["xq"] = codes_np(saved["xq"][it])
    torch.cuda.synchronize()
    del y, saved, g
    torch.cuda.empty_cache()
    f = {k: f64(v) for k, v in t.items()}
    # the sampled rows' exact forward (rows are independent)
    o = O.layernorm_mlp_fwd(f["x"][idx], f["gamma"], f["beta"], f["kernel1"], f["kernel2"], f["bias1"],
                            f["bias2"], norm_type=w.norm_type, epsilon=w.epsilon,
                            activation_type=w.activation_type)
    if quant == "none":
        assert_rel(got_y, o["y"], TOL["bf16"], "y")
        check_elementwise(got_y, o["y"], rounding_bound(2), "y")
        check_elementwise(got_h1, o["h"], rounding_bound(1), "h1")
        return
    # current scaling over the whole tensors: the normalised input of every
    # row sets x's scale, which the sampled rows' codes must use
    xn, _, _ = O.normalize(f["x"], f["gamma"], f["beta"], w.norm_type, w.epsilon, False)
    mx = O.current_scaling(xn)
    assert abs(q.x.values()["amax"] - mx["amax"]) <= 1e-5 * mx["amax"]
    w1q, m1 = O.quantize(f["kernel1"])
    w2q, m2 = O.quantize(f["kernel2"])
    assert np.array_equal(codes["w1q_t"].T, w1q), "w1 codes"
    assert np.array_equal(codes["w2q_t"].T, w2q), "w2 codes"
    xq, _ = O.quantize(xn[idx], mx)
    check_codes(codes["xq"], xq, "xq")
    h1 = O.fp8_dense(xq, mx, w1q, m1, f["bias1"])
    assert_rel(got_h1, h1, TOL["bf16"], "h1")
    # the activation's scale needs every row's h1, so y is held to the exact
    # forward within the quantisation noise of its four E4M3 operands
    assert_rel(got_y, o["y"], FP8_VS_EXACT, "y")


def test_mlp_fp8_kernels_just_under_2gib():
    """The fp8 forward with both kernels 8 KiB under 2 GiB (bf16; their codes
    are 1 GiB): the weights' amax and quantise-transpose over the whole range.
    The kernels' scales come from their full amax; their codes are checked
    bit-exact on the first, middle and last columns of kernel1 and rows of
    kernel2, h1 on those columns, and y against the exact forward within the
    E4M3 noise (the activation's full-width codes are not emulated)."""
    w = W.WORKLOADS["ln_mlp_gelu_fp8"].scaled(40, 256, WIDEST - 16)
    assert LIMIT - (1 << 20) < w.hidden * w.ffn * 2 < LIMIT
    print(f"layernorm_mlp fp8 {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    q = te.QuantizerSet()
    y, saved = te.layernorm_mlp(g["x"], g["gamma"], g["beta"], [g["kernel1"], g["kernel2"]],
                                [g["bias1"], g["bias2"]], w.norm_type, epsilon=w.epsilon,
                                activation_type=w.activation_type, quantizer_set=q, return_saved=True,
                                save_codes=True)
    cols = np.concatenate([np.arange(16), np.arange(w.ffn // 2 - 8, w.ffn // 2 + 8), np.arange(w.ffn - 16, w.ffn)])
    ct = torch.from_numpy(cols).to(dev())
    got_y, got_h1 = f64(y), f64(saved["h1"][:, ct])
    w1q_got, w2q_got = codes_np(saved["w1q_t"][ct]).T, codes_np(saved["w2q_t"][:, ct])
    xq_got = codes_np(saved["xq"])
    metas = {k: getattr(q, k).values() for k in ("x", "w1", "w2")}
    torch.cuda.synchronize()
    del y, saved, g
    torch.cuda.empty_cache()
    f = {k: f64(v) for k, v in t.items()}
    del t
    m1, m2 = O.current_scaling(f["kernel1"]), O.current_scaling(f["kernel2"])
    for key, m in (("w1", m1), ("w2", m2)):
        assert abs(metas[key]["amax"] - m["amax"]) <= 1e-5 * m["amax"], key
    w1q, _ = O.quantize(f["kernel1"][:, cols], m1)
    w2q, _ = O.quantize(f["kernel2"][cols, :], m2)
    assert np.array_equal(w1q_got, w1q), "w1 codes"
    assert np.array_equal(w2q_got, w2q.T), "w2 codes"
    xn, _, _ = O.normalize(f["x"], f["gamma"], f["beta"], w.norm_type, w.epsilon, False)
    xq, mx = O.quantize(xn)
    assert abs(metas["x"]["amax"] - mx["amax"]) <= 1e-5 * mx["amax"]
    check_codes(xq_got, xq, "xq")
    assert_rel(got_h1, O.fp8_dense(xq, mx, w1q, m1, f["bias1"][cols]), TOL["bf16"], "h1")
    o = O.layernorm_mlp_fwd(f["x"], f["gamma"], f["beta"], f["kernel1"], f["kernel2"], f["bias1"], f["bias2"],
                            norm_type=w.norm_type, epsilon=w.epsilon, activation_type=w.activation_type)
    assert_rel(got_y, o["y"], FP8_VS_EXACT, "y")
