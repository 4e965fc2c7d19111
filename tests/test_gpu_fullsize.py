"""GPU parity at the full workload sizes, launched as bench.py launches them
(same entry points and tensor shapes). The GPU computes every row; the oracle
computes a sample of rows spread over tiles (first/last rows of 256-row tiles
and of the whole tensor). Rows are independent once the whole-tensor fp8
amaxes are known, and those the oracle computes over every row."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import (ACT_CODE_ONE_STEP_MAX, CODE_ONE_STEP_MAX, TOL, assert_rel, check_codes,
                      check_codes_combined, codes_np, dev, f64, to_dev)

pytestmark = pytest.mark.gpu


def sample_rows(n):
    r = [0, 1, 2, 127, 255, 256, 511, 1023, 1024, 2047, 3000, 4095, 4096, 5555, 6143, 8190, 8191]
    return np.array(sorted({x for x in r if x < n} | {n - 1}))


def _f64_rows(t, rows):
    return f64(t[torch.as_tensor(rows)])


def test_full_ln_dense_bf16():
    w = W.WORKLOADS["ln_dense_bf16"]
    print(f"full {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    y = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g["bias"], epsilon=w.epsilon)
    torch.cuda.synchronize()
    rows = sample_rows(w.rows)
    ref = O.layernorm_dense_fwd(_f64_rows(t["x"], rows), f64(t["kernel"]), f64(t["gamma"]), f64(t["beta"]),
                                f64(t["bias"]), epsilon=w.epsilon)["y"]
    got = f64(y[torch.as_tensor(rows, device=dev())])
    assert_rel(got, ref, TOL["bf16"], "y")
    assert torch.isfinite(y).all()


@pytest.mark.parametrize("name", ["ln_mlp_gelu_bf16", "rms_swiglu_bf16"])
def test_full_mlp_bf16(name):
    w = W.WORKLOADS[name]
    print(f"full {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    y = te.layernorm_mlp(g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]],
                         [g.get("bias1"), g.get("bias2")], w.norm_type,
                         zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                         activation_type=w.activation_type)
    torch.cuda.synchronize()
    rows = sample_rows(w.rows)
    f = {k: f64(v) for k, v in t.items() if k != "x"}
    ref = O.layernorm_mlp_fwd(_f64_rows(t["x"], rows), f["gamma"], f.get("beta"), f["kernel1"], f["kernel2"],
                              f.get("bias1"), f.get("bias2"), norm_type=w.norm_type,
                              zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                              activation_type=w.activation_type)["y"]
    got = f64(y[torch.as_tensor(rows, device=dev())])
    assert_rel(got, ref, TOL["bf16"], "y")
    assert torch.isfinite(y).all()


def test_full_mlp_fp8_forward():
    w = W.WORKLOADS["ln_mlp_gelu_fp8"]
    print(f"full {w.name} forward", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    q = te.QuantizerSet()
    y, saved = te.layernorm_mlp(g["x"], g["gamma"], g["beta"], [g["kernel1"], g["kernel2"]],
                                [g["bias1"], g["bias2"]], w.norm_type, epsilon=w.epsilon,
                                activation_type=w.activation_type, quantizer_set=q, return_saved=True,
                                save_codes=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.rows)
    rt = torch.as_tensor(rows, device=dev())
    f = {k: f64(v) for k, v in t.items() if k != "grad"}
    o = O.layernorm_mlp_fwd(f["x"], f["gamma"], f["beta"], f["kernel1"], f["kernel2"], f["bias1"], f["bias2"],
                            epsilon=w.epsilon, activation_type=w.activation_type, quant="fp8_e4m3_current",
                            rows=rows)
    for key, meta in (("x_meta", q.x), ("w1_meta", q.w1), ("w2_meta", q.w2), ("act_meta", q.act)):
        got, ref = meta.values(), o[key]
        assert abs(got["amax"] - ref["amax"]) <= 1e-5 * ref["amax"], key
        assert got["scale"] == float(np.float32(448.0) / np.float32(got["amax"])), key
    w1q = codes_np(saved["w1q_t"]).T
    w2q = codes_np(saved["w2q_t"]).T
    assert np.array_equal(w1q, o["w1q"]) and np.array_equal(w2q, o["w2q"])
    check_codes_combined([("xq", codes_np(saved["xq"]), o["xq"], CODE_ONE_STEP_MAX),
                          ("w1q", w1q, o["w1q"], CODE_ONE_STEP_MAX),
                          ("w2q", w2q, o["w2q"], CODE_ONE_STEP_MAX),
                          ("actq (sampled rows)", codes_np(saved["actq"][rt]), o["actq"], ACT_CODE_ONE_STEP_MAX)])
    assert_rel(f64(saved["h1"][rt]), o["h1"], TOL["bf16"], "h1")
    assert_rel(f64(y[rt]), o["y"], TOL["fp8"], "y")
    assert torch.isfinite(y).all()


def test_full_dact_dbias():
    """grad [8192, 16384] ~ N(0, 1) and a pre-activation of GEMM1's spread."""
    w = W.WORKLOADS["ln_mlp_gelu_fp8"]
    print("full dact_dbias 8192x16384 gelu", flush=True)
    a = W.make_act_inputs(w.rows, w.ffn, gated=False, dtype="bf16", seed=0, std=1.3)
    gd, xd = a["grad"].to(dev()), a["x"].to(dev())
    dx, db = te.dact_dbias(gd, xd, ("gelu",))
    torch.cuda.synchronize()
    rows = sample_rows(w.rows)
    rdx, rdb = O.dact_dbias(f64(a["grad"]), f64(a["x"]), ("gelu",))
    assert_rel(f64(dx[torch.as_tensor(rows, device=dev())]), rdx[rows], TOL["bf16"], "dx")
    assert_rel(f64(db), rdb, 1e-5, "dbias")


def test_full_dact_dbias_swiglu():
    """Gated (silu, linear) at the RMSNorm-SwiGLU shape: grad [8192, 14336],
    pre-activation [8192, 2 x 14336]."""
    w = W.WORKLOADS["rms_swiglu_bf16"]
    print("full dact_dbias 8192x2x14336 swiglu", flush=True)
    a = W.make_act_inputs(w.rows, w.ffn, gated=True, dtype="bf16", seed=0, std=1.3)
    gd, xd = a["grad"].to(dev()), a["x"].to(dev())
    dx, db = te.dact_dbias(gd, xd, ("silu", "linear"))
    torch.cuda.synchronize()
    rows = sample_rows(w.rows)
    rdx, rdb = O.dact_dbias(_f64_rows(a["grad"], rows), _f64_rows(a["x"], rows), ("silu", "linear"))
    assert_rel(f64(dx[torch.as_tensor(rows, device=dev())]), rdx, TOL["bf16"], "dx")
    # dbias over all rows, in column blocks (the same columns of both halves)
    # to bound the oracle's memory
    F = w.ffn
    for c0 in range(0, F, 2048):
        c1 = min(c0 + 2048, F)
        n = c1 - c0
        xab = np.concatenate([f64(a["x"][:, c0:c1]), f64(a["x"][:, F + c0:F + c1])], axis=1)
        ref = O.dact_dbias(f64(a["grad"][:, c0:c1]), xab, ("silu", "linear"))[1]
        assert_rel(f64(db[c0:c1]), ref[:n], 1e-5, f"dbias a[{c0}:{c1}]")
        assert_rel(f64(db[F + c0:F + c1]), ref[n:], 1e-5, f"dbias b[{c0}:{c1}]")


def test_full_dact_dbias_quantize():
    """quantize_dact_dbias at 8192 x 16384 (GELU): amax over the whole dx, codes
    of sampled rows, dbias over all rows."""
    w = W.WORKLOADS["ln_mlp_gelu_fp8"]
    print("full dact_dbias_quantize 8192x16384 gelu", flush=True)
    a = W.make_act_inputs(w.rows, w.ffn, gated=False, dtype="bf16", seed=0, std=1.3)
    gd, xd = a["grad"].to(dev()), a["x"].to(dev())
    q = te.Fp8Meta()
    codes, db = te.dact_dbias_quantize(gd, xd, ("gelu",), q)
    torch.cuda.synchronize()
    rdx, rdb = O.dact_dbias(f64(a["grad"]), f64(a["x"]), ("gelu",))
    meta = O.current_scaling(rdx)
    m = q.values()
    assert abs(m["amax"] - meta["amax"]) <= 1e-5 * meta["amax"]
    rows = sample_rows(w.rows)
    rq, _ = O.quantize(rdx[rows], meta)
    check_codes(codes_np(codes[torch.as_tensor(rows, device=dev())]), rq, "dx codes (sampled rows)")
    assert_rel(f64(db), rdb, 1e-5, "dbias")


def test_full_norm_bwd_ln_bf16():
    """LayerNorm backward at 8192 x 4096 bf16 from the forward's saved statistics."""
    w = W.WORKLOADS["ln_mlp_gelu_bf16"]
    print("full norm_bwd 8192x4096 layernorm bf16", flush=True)
    t = W.make_inputs(w)
    gen = torch.Generator(device="cpu").manual_seed(5)
    dy = torch.randn(w.rows, w.hidden, generator=gen).to(torch.bfloat16)
    x, gamma, beta = t["x"].to(dev()), t["gamma"].to(dev()), t["beta"].to(dev())
    _, mu, rs = te.layernorm(x, gamma, beta, "layernorm", False, w.epsilon, return_stats=True)
    dx, dg, db = te.layernorm_bwd(dy.to(dev()), x, mu, rs, gamma, "layernorm")
    torch.cuda.synchronize()
    rdx, rdg, rdb = O.norm_bwd(f64(dy), f64(t["x"]), f64(t["gamma"]), "layernorm", w.epsilon)
    rows = sample_rows(w.rows)
    assert_rel(f64(dx[torch.as_tensor(rows, device=dev())]), rdx[rows], TOL["bf16"], "dx")
    assert_rel(f64(dg), rdg, 1e-5, "dgamma")
    assert_rel(f64(db), rdb, 1e-5, "dbeta")
