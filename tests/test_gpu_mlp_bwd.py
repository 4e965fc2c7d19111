"""GPU parity of the LayerNorm-MLP backward (te_layernorm_mlp_bwd) against the
fp64 oracle: every input and parameter gradient, for LayerNorm/RMSNorm,
plain and gated activations, at shapes that span several 256 x 256 tiles
with ragged edges (rows, hidden and ffn not multiples of the tile), and at
the 8192 x 4096 -> 16384 workload on sampled rows and columns.

The oracle is compared twice: with the tensors the bf16 forward/backward
pair materialises rounded to bf16 (xn, the saved h1, act, dact, dh1, dxn),
which is the dataflow the library computes, to the bf16 tolerance; and in
pure fp64, to a bound derived per gradient from the number k of bf16
roundings on its chain (tolerances.rounding_bound: 1.5 sqrt(k) x the error
of one rounding), counting the output rounding of the bf16 gradients."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import TOL, assert_rel, check_elementwise, dev, f64, to_dev
from tolerances import bwd_roundings, rounding_bound

pytestmark = pytest.mark.gpu

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
        n = bwd_roundings(k, w.gated, output_rounded=True)
        e = assert_rel(f64(out[k]), ref_x[k], rounding_bound(n) if n else 1e-5, f"{k} (fp64)")
        print(f"  {k}: rel_l2 vs fp64 {e:.3e} (k = {n}, bound {rounding_bound(n) if n else 1e-5:.2e})", flush=True)


@pytest.mark.parametrize("act", [("relu",), ("silu",), ("gelu_erf",), ("linear",), ("gelu", "linear"),
                                 ("relu", "linear"), ("gelu_erf", "linear")], ids=lambda a: "-".join(a))
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
    """8192 x 4096 -> 16384 backward, every element of every gradient: rel-L2
    against the rounded dataflow and against fp64 (derived bound), and the
    per-element guard under the k-rounding model."""
    w = W.WORKLOADS["ln_mlp_gelu_bf16"]
    print("full layernorm_mlp_bwd 8192x4096x16384", flush=True)
    t = W.make_inputs(w)
    gy = _grad(w)
    out = {k: (f64(v) if v is not None else None) for k, v in _run(w, t, gy).items()}
    torch.cuda.empty_cache()
    ref_r = _oracle(w, t, gy, True)
    for k in NAMES:
        assert_rel(out[k], ref_r[k], TOL["bf16"], f"{k} (bf16 dataflow)")
    del ref_r
    ref_x = _oracle(w, t, gy, False)
    for k in NAMES:
        n = bwd_roundings(k, w.gated, output_rounded=True)
        bound = rounding_bound(n) if n else 1e-5
        e = assert_rel(out[k], ref_x[k], bound, f"{k} (fp64)")
        m = check_elementwise(out[k], ref_x[k], bound, k)
        print(f"  {k}: rel_l2 vs fp64 {e:.3e} (k = {n}), max |err| / rms {m:.3e}", flush=True)


def test_mlp_bwd_activation_just_under_2gib():
    """65528 x 256 -> 16384: the [rows, ffn] activation and its gradient are
    256 KiB under 2 GiB, the backward's limit, where both weight-gradient
    GEMMs read them through one buffer descriptor. Every element of every
    gradient against fp64, the oracle run in row blocks (dx per block, the
    parameter gradients summed over the blocks). The activation is linear:
    the GEMMs under test are the same for every activation, and the oracle's
    GELU over 2^30 elements would take minutes."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS["ln_mlp_gelu_bf16"].scaled(65528, 256, 16384), activation_type=("linear",))
    assert (1 << 31) - (1 << 20) < w.rows * w.ffn * 2 < 1 << 31
    print(f"layernorm_mlp_bwd {w.name}", flush=True)
    t = W.make_inputs(w)
    gy = _grad(w)
    out = {k: (f64(v) if v is not None else None) for k, v in _run(w, t, gy).items()}
    torch.cuda.empty_cache()
    f = {k: f64(v) for k, v in t.items()}
    g64 = f64(gy)
    ref = {k: None for k in NAMES}
    ref["dx"] = np.empty_like(out["dx"])
    for r0 in range(0, w.rows, 8192):
        b = O.layernorm_mlp_bwd(g64[r0:r0 + 8192], f["x"][r0:r0 + 8192], f["gamma"], f["beta"], f["kernel1"],
                                f["kernel2"], f["bias1"], f["bias2"], norm_type=w.norm_type, epsilon=w.epsilon,
                                activation_type=w.activation_type)
        ref["dx"][r0:r0 + 8192] = b["dx"]
        for k in NAMES[1:]:
            ref[k] = b[k] if ref[k] is None else ref[k] + b[k]
    for k in NAMES:
        n = bwd_roundings(k, w.gated, output_rounded=True)
        bound = rounding_bound(n) if n else 1e-5
        e = assert_rel(out[k], ref[k], bound, f"{k} (fp64)")
        m = check_elementwise(out[k], ref[k], bound, k)
        print(f"  {k}: rel_l2 vs fp64 {e:.3e} (k = {n}), max |err| / rms {m:.3e}", flush=True)
