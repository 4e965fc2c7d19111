"""GPU parity of the LayerNorm-MLP backward (te_layernorm_mlp_bwd) against the
fp64 oracle: every input and parameter gradient, for LayerNorm/RMSNorm,
plain and gated activations, at shapes that span several 256 x 256 tiles
with ragged edges (rows, hidden and ffn not multiples of the tile), and at
the 8192 x 4096 -> 16384 workload on sampled rows and columns.

The oracle is compared twice: with the tensors the bf16 forward/backward
pair materialises rounded to bf16 (xn, the saved h1, act, dact, dh1, dxn),
which is the dataflow the library computes, to the bf16 tolerance; and in
pure fp64, to a looser bound that the extra roundings account for."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import TOL, assert_rel, dev, f64, to_dev

pytestmark = pytest.mark.gpu

EXACT_TOL = 2e-2
NAMES = ("dx", "dgamma", "dbeta", "dkernel1", "dbias1", "dkernel2", "dbias2")


def _grad(w, seed=3):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(w.rows, w.hidden, generator=gen).to(torch.bfloat16)


def _run(w, t, gy):
    g = to_dev(t)
    gyd = gy.to(dev())
    _, saved = te.layernorm_mlp(g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]],
                                [g.get("bias1"), g.get("bias2")], w.norm_type,
                                zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                                activation_type=w.activation_type, return_saved=True)
    out = te.layernorm_mlp_bwd(gyd, g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]], saved,
                               w.norm_type, zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                               activation_type=w.activation_type)
    torch.cuda.synchronize()
    return out


def _oracle(w, t, gy, rounded):
    f = {k: f64(v) for k, v in t.items()}
    return O.layernorm_mlp_bwd(f64(gy), f["x"], f["gamma"], f.get("beta"), f["kernel1"], f["kernel2"],
                               f.get("bias1"), f.get("bias2"), norm_type=w.norm_type,
                               zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                               activation_type=w.activation_type, round_intermediates=rounded)


@pytest.mark.parametrize("name,rows,hidden,ffn", [
    ("ln_mlp_gelu_bf16", 300, 272, 400),
    ("ln_mlp_gelu_bf16", 513, 512, 1040),
    ("rms_swiglu_bf16", 257, 256, 288),
    ("rms_swiglu_bf16", 600, 1024, 1536),
])
def test_mlp_bwd_workload_recipes(name, rows, hidden, ffn):
    w = W.WORKLOADS[name].scaled(rows, hidden, ffn)
    print(f"layernorm_mlp_bwd {w.name}", flush=True)
    t = W.make_inputs(w)
    gy = _grad(w)
    out = _run(w, t, gy)
    ref_r, ref_x = _oracle(w, t, gy, True), _oracle(w, t, gy, False)
    for k in NAMES:
        if ref_r[k] is None:
            assert out[k] is None or w.norm_type == "rmsnorm", k
            continue
        assert_rel(f64(out[k]), ref_r[k], TOL["bf16"], f"{k} (bf16 dataflow)")
        assert_rel(f64(out[k]), ref_x[k], EXACT_TOL, f"{k} (fp64)")


@pytest.mark.parametrize("act", [("relu",), ("silu",), ("gelu_erf",), ("linear",), ("gelu", "linear"),
                                 ("relu", "linear")], ids=lambda a: "-".join(a))
def test_mlp_bwd_activations(act):
    w = W.Workload("mlpb", "mlp", 384, 272, 528, "bf16", "none", "layernorm", False, 1e-6, act, True)
    print(f"layernorm_mlp_bwd {act} 384x272x528", flush=True)
    t = W.make_inputs(w, seed=4)
    gy = _grad(w, seed=9)
    out = _run(w, t, gy)
    ref = _oracle(w, t, gy, True)
    for k in NAMES:
        assert_rel(f64(out[k]), ref[k], TOL["bf16"], k)


def test_mlp_bwd_zero_rows():
    w = W.WORKLOADS["ln_mlp_gelu_bf16"].scaled(1, 64, 128)
    t = to_dev(W.make_inputs(w))
    x0 = t["x"][:0]
    saved = {"h1": torch.empty(0, 128, dtype=torch.bfloat16, device=dev()),
             "mu": torch.empty(0, dtype=torch.float32, device=dev()),
             "rsigma": torch.empty(0, dtype=torch.float32, device=dev())}
    out = te.layernorm_mlp_bwd(x0, x0, t["gamma"], t["beta"], [t["kernel1"], t["kernel2"]], saved, "layernorm",
                               activation_type=("gelu",))
    torch.cuda.synchronize()
    assert out["dx"].shape == (0, 64)
    for k in ("dgamma", "dbeta", "dkernel1", "dbias1", "dkernel2", "dbias2"):
        assert not out[k].any(), k


def test_full_mlp_bwd_ln_gelu_bf16():
    """8192 x 4096 -> 16384 backward: dx on sampled rows, dkernel1 / dkernel2 /
    dbias1 on sampled ffn columns (the oracle run on those columns of the
    kernels, which they depend on alone), dbias2 over all rows."""
    w = W.WORKLOADS["ln_mlp_gelu_bf16"]
    print("full layernorm_mlp_bwd 8192x4096x16384", flush=True)
    t = W.make_inputs(w)
    gy = _grad(w)
    out = _run(w, t, gy)
    rows = np.array([0, 1, 255, 256, 4095, 5000, 8191])
    tr = dict(t, x=t["x"][torch.as_tensor(rows)])
    ref = _oracle(w.scaled(rows=len(rows)), tr, gy[torch.as_tensor(rows)], True)
    assert_rel(f64(out["dx"][torch.as_tensor(rows, device=dev())]), ref["dx"], TOL["bf16"], "dx (sampled rows)")
    cols = np.array([0, 1, 255, 256, 8191, 12000, 16383])
    ct = torch.as_tensor(cols)
    tc = dict(t, kernel1=t["kernel1"][:, ct], bias1=t["bias1"][ct], kernel2=t["kernel2"][ct, :])
    refc = _oracle(w.scaled(ffn=len(cols)), tc, gy, True)
    cd = torch.as_tensor(cols, device=dev())
    assert_rel(f64(out["dkernel1"][:, cd]), refc["dkernel1"], TOL["bf16"], "dkernel1 (sampled columns)")
    assert_rel(f64(out["dkernel2"][cd, :]), refc["dkernel2"], TOL["bf16"], "dkernel2 (sampled rows)")
    assert_rel(f64(out["dbias1"][cd]), refc["dbias1"], TOL["bf16"], "dbias1 (sampled)")
    assert_rel(f64(out["dbias2"]), refc["dbias2"], 1e-5, "dbias2")
