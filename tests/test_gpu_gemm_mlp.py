"""GPU parity of the GEMM paths against the fp64 oracle, through the page-style
calls: LayerNorm+Dense and the fused LayerNorm-MLP, in fp32, bf16 and fp8, at
sizes that span several 256 x 256 tiles with ragged edges in M, N and K."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import (ACT_CODE_ONE_STEP_MAX, CODE_ONE_STEP_MAX, TOL, assert_rel, check_codes,
                      check_codes_combined, codes_np, dev, f64, to_dev)

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
    assert_rel(f64(y), exact, 0.1, "y vs unquantised")


MLP_ACTS = [("gelu",), ("relu",), ("silu",), ("gelu_erf",), ("linear",),
            ("silu", "linear"), ("gelu", "linear"), ("relu", "linear")]


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
    torch.cuda.synchronize()
    o = _mlp_oracle(w, t, quant="fp8_e4m3_current")
    for key, meta in (("x_meta", q.x), ("w1_meta", q.w1), ("w2_meta", q.w2), ("act_meta", q.act)):
        got, ref = meta.values(), o[key]
        assert abs(got["amax"] - ref["amax"]) <= 1e-5 * ref["amax"], key
        assert got["scale"] == float(np.float32(448.0) / np.float32(got["amax"])), key
    # the kernels' codes are computed from exact inputs: bit-exact
    assert np.array_equal(codes_np(saved["w1q_t"]), o["w1q"].T)
    assert np.array_equal(codes_np(saved["w2q_t"]), o["w2q"].T)
    check_codes_combined([("xq", codes_np(saved["xq"]), o["xq"], CODE_ONE_STEP_MAX),
                          ("w1q", codes_np(saved["w1q_t"]).T, o["w1q"], CODE_ONE_STEP_MAX),
                          ("w2q", codes_np(saved["w2q_t"]).T, o["w2q"], CODE_ONE_STEP_MAX),
                          ("actq", codes_np(saved["actq"]), o["actq"], ACT_CODE_ONE_STEP_MAX)])
    assert_rel(f64(saved["h1"]), o["h1"], TOL["bf16"], "h1")
    assert_rel(f64(y), o["y"], TOL["fp8"], "y")


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
