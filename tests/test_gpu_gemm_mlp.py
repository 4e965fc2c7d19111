"""GPU parity of the GEMM paths against the fp64 oracle, through the page-style
calls: LayerNorm+Dense and the fused LayerNorm-MLP, in fp32, bf16 and fp8, at
sizes that span several 256 x 256 tiles with ragged edges in M, N and K."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import (H1_ACC_REL, TOL, assert_rel, check_codes, check_elementwise, check_fp8_forward, codes_np,
                      dev, f64, to_dev)
from tolerances import rounding_bound

pytestmark = pytest.mark.gpu


def _dense_case(rows, hidden, out, dtype, quant, norm="layernorm", seed=0, bias=True):
    w = W.Workload("dense", "dense", rows, hidden, out, dtype, quant, norm, False, 1e-5, (), bias)
    return w, W.make_inputs(w, seed)


@pytest.mark.parametrize("rows,hidden,out", [(1, 16, 16), (300, 272, 400), (257, 80, 528),
                                             (512, 1024, 768), (64, 4096, 256), (2100, 272, 400),
                                             (2048, 1040, 784), (2305, 80, 16)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_layernorm_dense(rows, hidden, out, dtype):
    print(f"layernorm_dense {dtype} {rows}x{hidden}->{out}", flush=True)
    w, t = _dense_case(rows, hidden, out, dtype, "none", seed=rows)
    g = to_dev(t)
    y = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g["bias"], epsilon=1e-5)
    y2 = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g["bias"], epsilon=1e-5)
    torch.cuda.synchronize()
    f = {k: f64(v) for k, v in t.items()}
    ref = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f["beta"], f["bias"], epsilon=1e-5)["y"]
    assert_rel(f64(y), ref, TOL[dtype], "y")
    if dtype == "bf16":
        check_elementwise(f64(y), ref, rounding_bound(1), "y")
        # against the oracle with the normalised input rounded to bf16 as the GPU stores it
        refr = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f["beta"], f["bias"], epsilon=1e-5,
                                     round_intermediates=True)["y"]
        assert_rel(f64(y), refr, 3e-3, "y (bf16 intermediates)")
    assert torch.equal(y, y2), "not bitwise reproducible"


@pytest.mark.parametrize("rows,hidden,out", [(300, 272, 400), (512, 1024, 768)])
@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_layernorm_dense_fp8(rows, hidden, out, norm):
    print(f"layernorm_dense fp8 {norm} {rows}x{hidden}->{out}", flush=True)
    w, t = _dense_case(rows, hidden, out, "bf16", "fp8_e4m3_current", norm=norm, seed=5)
    g = to_dev(t)
    y = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g.get("beta"), g["bias"], norm_type=norm,
                           epsilon=1e-5, quantizer_set=te.QuantizerSet())
    torch.cuda.synchronize()
    f = {k: f64(v) for k, v in t.items()}
    o = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f.get("beta"), f["bias"], norm_type=norm,
                              epsilon=1e-5, quant="fp8_e4m3_current")
    exact = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f.get("beta"), f["bias"], norm_type=norm,
                                  epsilon=1e-5)["y"]
    assert_rel(f64(y), o["y"], TOL["fp8"], "y vs fp8 oracle")
    # y depends on the codes alone; at most 0.1% of the normalised input's codes
    # may sit one E4M3 step (2^-3 of the value) away
    check_elementwise(f64(y), o["y"], 1.5 * np.sqrt(rounding_bound(1) ** 2 + 1e-3 * 2.0 ** -6), "y")
    assert_rel(f64(y), exact, 0.1, "y vs unquantised")


MLP_ACTS = [("gelu",), ("relu",), ("silu",), ("gelu_erf",), ("linear",),
            ("silu", "linear"), ("gelu", "linear"), ("relu", "linear"), ("gelu_erf", "linear")]


def _mlp_oracle(w, t, **kw):
    f = {k: f64(v) for k, v in t.items()}
    return O.layernorm_mlp_fwd(f["x"], f["gamma"], f.get("beta"), f["kernel1"], f["kernel2"], f.get("bias1"),
                               f.get("bias2"), norm_type=w.norm_type, zero_centered_gamma=w.zero_centered_gamma,
                               epsilon=w.epsilon, activation_type=w.activation_type, **kw)


def _mlp_gpu(w, g, **kw):
    return te.layernorm_mlp(g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]],
                            [g.get("bias1"), g.get("bias2")], w.norm_type,
                            zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                            activation_type=w.activation_type, **kw)


def test_mlp_tiny_fp32_workload():
    """The whole 64 x 128 -> 512 -> 128 fp32 workload (LayerNorm, GELU-tanh)."""
    w = W.WORKLOADS["ln_mlp_tiny_fp32"]
    print(f"layernorm_mlp {w.name}", flush=True)
    t = W.make_inputs(w)
    y, saved = _mlp_gpu(w, to_dev(t), return_saved=True)
    torch.cuda.synchronize()
    o = _mlp_oracle(w, t)
    assert_rel(f64(y), o["y"], TOL["fp32"], "y")
    assert_rel(f64(saved["h1"]), o["h"], TOL["fp32"], "h1")
    assert_rel(f64(saved["rsigma"]), o["rsigma"], 1e-6, "rsigma")


@pytest.mark.parametrize("act", MLP_ACTS, ids=["-".join(a) for a in MLP_ACTS])
@pytest.mark.parametrize("dtype,rows", [("fp32", 300), ("bf16", 300), ("bf16", 2100)])
def test_mlp_activations(act, dtype, rows):
    w = W.Workload("mlp", "mlp", rows, 272, 400, dtype, "none", "layernorm", False, 1e-6, act, True)
    print(f"layernorm_mlp {dtype} {act} {rows}x272x400", flush=True)
    t = W.make_inputs(w, seed=11)
    y, saved = _mlp_gpu(w, to_dev(t), return_saved=True)
    torch.cuda.synchronize()
    o = _mlp_oracle(w, t)
    assert_rel(f64(y), o["y"], TOL[dtype], "y")
    assert_rel(f64(saved["h1"]), o["h"], TOL[dtype], "h1")
    if dtype == "bf16":
        check_elementwise(f64(y), o["y"], rounding_bound(2), "y")
        check_elementwise(f64(saved["h1"]), o["h"], rounding_bound(1), "h1")


@pytest.mark.parametrize("name,rows,hidden,ffn", [
    ("ln_mlp_gelu_bf16", 300, 272, 400),
    ("ln_mlp_gelu_bf16", 513, 512, 1024),
    ("rms_swiglu_bf16", 257, 256, 288),
    ("rms_swiglu_bf16", 512, 1024, 1536),
    ("ln_mlp_gelu_bf16", 2300, 512, 1040),
    ("rms_swiglu_bf16", 2049, 256, 288),
])
def test_mlp_bf16_workload_recipes(name, rows, hidden, ffn):
    w = W.WORKLOADS[name].scaled(rows, hidden, ffn)
    print(f"layernorm_mlp {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    y, saved = _mlp_gpu(w, g, return_saved=True)
    y2 = _mlp_gpu(w, g)
    torch.cuda.synchronize()
    o = _mlp_oracle(w, t)
    assert_rel(f64(y), o["y"], TOL["bf16"], "y")
    check_elementwise(f64(y), o["y"], rounding_bound(2), "y")
    orr = _mlp_oracle(w, t, round_intermediates=True)
    assert_rel(f64(y), orr["y"], 3e-3, "y (bf16 intermediates)")
    assert torch.equal(y, y2), "not bitwise reproducible"
    if w.norm_type == "layernorm":
        assert np.max(np.abs(f64(saved["mu"]) - o["mu"])) <= 1e-5


@pytest.mark.parametrize("name,rows,hidden,ffn", [
    ("ln_mlp_gelu_fp8", 300, 272, 400),
    ("ln_mlp_gelu_fp8", 512, 512, 1024),
])
@pytest.mark.parametrize("gated", [False, True])
def test_mlp_fp8(name, rows, hidden, ffn, gated):
    base = W.WORKLOADS[name].scaled(rows, hidden, ffn)
    if gated:
        import dataclasses
        base = dataclasses.replace(base, activation_type=("silu", "linear"), name=base.name + "-swiglu")
    w = base
    print(f"layernorm_mlp fp8 {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    q = te.QuantizerSet()
    y, saved = _mlp_gpu(w, g, quantizer_set=q, return_saved=True, save_codes=True)
    # without caller code buffers the codes stay in the workspace in the tiled
    # GEMM operand layout: the same values in the same summation order, so y
    # and h1 are bit-identical to the run above, whose codes are checked
    y_t, saved_t = _mlp_gpu(w, g, quantizer_set=te.QuantizerSet(), return_saved=True)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y) and torch.equal(saved_t["h1"], saved["h1"]), "tiled workspace codes"
    o = _mlp_oracle(w, t, quant="fp8_e4m3_current")
    check_fp8_forward(q, saved, y, o, w.activation_type, w.name)


@pytest.mark.parametrize("act", ["gelu", "gelu_erf", "silu", "relu", "linear"])
@pytest.mark.parametrize("regime", ["small", "negative"])
def test_mlp_fp8_activation_amax_regimes(act, regime):
    """The amax of act(h) that GEMM1's epilogue reduces, where every value is
    small (kernel1 scaled by 0.05: |act(h)| < 0.1) or h is mostly negative
    (bias1 = -2: GELU and SiLU take their negative-side values): the epilogue
    then evaluates the activation of every element instead of taking it from
    the largest h, and must still match the oracle."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["ln_mlp_gelu_fp8"].scaled(300, 272, 400), activation_type=(act,),
                            name=f"fp8-{act}-{regime}")
    print(f"layernorm_mlp fp8 amax {act} {regime}", flush=True)
    t = W.make_inputs(w, seed=3)
    if regime == "small":
        t["kernel1"] = (t["kernel1"].float() * 0.05).to(t["kernel1"].dtype)
    else:
        t["bias1"] = torch.full_like(t["bias1"], -2.0)
    g = to_dev(t)
    q = te.QuantizerSet()
    y, saved = _mlp_gpu(w, g, quantizer_set=q, return_saved=True, save_codes=True)
    torch.cuda.synchronize()
    o = _mlp_oracle(w, t, quant="fp8_e4m3_current")
    got, ref = q.act.values()["amax"], o["act_meta"]["amax"]
    assert abs(got - ref) <= 1e-5 * ref, (got, ref)
    if ref > 0:
        assert_rel(f64(y), o["y"], TOL["fp8"], "y")


def test_mlp_zero_rows():
    w = W.WORKLOADS["ln_mlp_gelu_bf16"].scaled(1, 64, 128)
    t = to_dev(W.make_inputs(w))
    x0 = t["x"][:0]
    y = te.layernorm_mlp(x0, t["gamma"], t["beta"], [t["kernel1"], t["kernel2"]], [t["bias1"], t["bias2"]],
                         "layernorm", activation_type=("gelu",))
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


@pytest.mark.parametrize("quant", ["none", "fp8_e4m3_current"])
@pytest.mark.parametrize("rows,hidden,out", [(300, 272, 400), (513, 1024, 784)])
def test_layernorm_dense_f32_output(rows, hidden, out, quant):
    """y_dtype fp32 from bf16 inputs: the fp32 accumulator plus bias without
    the final bf16 rounding. Rounding it to bf16 must give the bf16-output
    call bit for bit (same kernel, same summation order)."""
    print(f"layernorm_dense {quant} f32 output {rows}x{hidden}->{out}", flush=True)
    w, t = _dense_case(rows, hidden, out, "bf16", quant, seed=rows + 1)
    g = to_dev(t)
    q = (lambda: te.QuantizerSet()) if quant != "none" else (lambda: None)
    y32 = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g["bias"], epsilon=1e-5,
                             quantizer_set=q(), out_dtype=torch.float32)
    y16 = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g["bias"], epsilon=1e-5,
                             quantizer_set=q())
    torch.cuda.synchronize()
    assert y32.dtype == torch.float32 and y16.dtype == torch.bfloat16
    assert torch.equal(y32.to(torch.bfloat16), y16), "fp32 output does not round to the bf16 output"
    f = {k: f64(v) for k, v in t.items()}
    if quant == "none":
        ref = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f["beta"], f["bias"], epsilon=1e-5,
                                    round_intermediates=True)["y"]
        # the normalised input is the bf16 A operand; the rest is fp32 accumulation
        assert_rel(f64(y32), ref, 1e-4, "y (fp32 output)")
    else:
        ref = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f["beta"], f["bias"], epsilon=1e-5,
                                    quant=quant)["y"]
        assert_rel(f64(y32), ref, TOL["fp8"], "y (fp32 output)")


@pytest.mark.parametrize("quant", ["none", "fp8_e4m3_current"])
def test_mlp_f32_output(quant):
    w = W.WORKLOADS["ln_mlp_gelu_bf16"].scaled(300, 272, 400)
    print(f"layernorm_mlp {quant} f32 output {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    q = (lambda: te.QuantizerSet()) if quant != "none" else (lambda: None)
    y32 = _mlp_gpu(w, g, quantizer_set=q(), out_dtype=torch.float32)
    y16 = _mlp_gpu(w, g, quantizer_set=q())
    torch.cuda.synchronize()
    assert y32.dtype == torch.float32
    assert torch.equal(y32.to(torch.bfloat16), y16), "fp32 output does not round to the bf16 output"
    o = _mlp_oracle(w, t, quant=quant) if quant != "none" else _mlp_oracle(w, t)
    assert_rel(f64(y32), o["y"], TOL["fp8" if quant != "none" else "bf16"], "y (fp32 output)")


# Summation error of one fp8 matrix instruction (64 products) relative to the
# largest of its products, as an upper bound: the per-64-block maxima of |a| and
# |b| multiplied. Measured at most 6.2e-5 (K = 400) and 1.4e-5 (K = 4096) of
# the sum over blocks of those bounds; twice the larger.
FP8_BLOCK_REL = 1.25e-4


@pytest.mark.parametrize("rows,hidden,ffn", [(512, 1024, 4096), (300, 272, 400)])
def test_fp8_gemm_summation_error(rows, hidden, ffn):
    """The fp8 GEMM's accumulator against the exact sum of its own operand
    codes. GEMM2 of the fp8 MLP with an fp32 output returns acc * s + bias2,
    s = fl32(scale_inv(act) * scale_inv(kernel2)); the saved act and kernel2
    codes give the exact sum in fp64 (E4M3 products span fewer than 53 bits).
    The difference is the summation error of the fp8 matrix instruction. Each
    instruction's error scales with the largest of its 64 products (the test
    holds the error to FP8_BLOCK_REL of the sum over k blocks of max|a| max|b|
    in the block); over a long K it is also within H1_ACC_REL of
    sum_k |a_k b_k|, the form the h1 rule of the fp8 parity checks uses."""
    w = W.WORKLOADS["ln_mlp_gelu_bf16"].scaled(rows, hidden, ffn)
    print(f"fp8 GEMM summation error {rows}x{hidden}x{ffn}", flush=True)
    t = W.make_inputs(w, seed=5)
    q = te.QuantizerSet()
    y, s = _mlp_gpu(w, to_dev(t), quantizer_set=q, out_dtype=torch.float32, return_saved=True, save_codes=True)
    torch.cuda.synchronize()
    a = O.e4m3_decode(codes_np(s["actq"]))
    b = O.e4m3_decode(codes_np(s["w2q_t"]))
    sc = float(np.float32(q.act.values()["scale_inv"]) * np.float32(q.w2.values()["scale_inv"]))
    exact = (a @ b.T) * sc + f64(t["bias2"])[None, :]
    yv = f64(y)
    # the epilogue's own roundings (acc * s and + bias2 in fp32), at most one ulp of y each
    ulp = np.spacing(np.abs(yv).astype(np.float32)).astype(np.float64)
    excess = np.maximum(np.abs(yv - exact) - 2 * ulp, 0)
    nb = (ffn + 63) // 64
    ma = np.stack([np.abs(a[:, 64 * j:64 * j + 64]).max(1) for j in range(nb)], 1)
    mb = np.stack([np.abs(b[:, 64 * j:64 * j + 64]).max(1) for j in range(nb)], 1)
    blk = (ma @ mb.T) * sc
    mag = (np.abs(a) @ np.abs(b).T) * sc
    r_blk = (excess / np.where(blk > 0, blk, 1)).max()
    r_mag = (excess / np.where(mag > 0, mag, 1)).max()
    print(f"  K = {ffn}: max error / sum of block max products {r_blk:.3g} (bound {FP8_BLOCK_REL:g}); "
          f"/ sum|a b| {r_mag:.3g}", flush=True)
    assert r_blk <= FP8_BLOCK_REL, f"fp8 GEMM summation error {r_blk:.3g} of the block bound"
    if ffn >= 4096:
        assert r_mag <= H1_ACC_REL, f"fp8 GEMM summation error {r_mag:.3g} of sum|a b| beyond {H1_ACC_REL:g}"
    # an error of the sum, not of the operands: a wrong code or element would be far larger
    assert np.abs(yv - exact).max() < 1e-3 * np.abs(exact).max()
