"""GPU parity at the full workload sizes, launched as bench.py launches them
(same entry points and tensor shapes), against the fp64 oracle on every
element: rel-L2 over the whole tensor plus the per-element guard of
gpu_util.check_elementwise, whose error model for the bf16 forwards is k
bf16 roundings between the inputs and the output (tolerances.rounding_bound).

The fp8 forward and the backward of its activation (dact + dbias on the
saved GEMM1 pre-activation) share one GPU run and one oracle run."""

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import TOL, assert_rel, bf16_ulp, check_codes, check_elementwise, check_fp8_forward, codes_np, dev, f64, to_dev
from tolerances import rounding_bound

pytestmark = pytest.mark.gpu

# dact: the kernel evaluates act' in fp32 (exp2, reciprocal); near a zero of
# act' the terms cancel and the error is a few fp32 ulps of the largest term,
# not of the result. 4e-6 of the tensor's rms bounds it for |grad| up to ~25.
DACT_FP32_REL = 4e-6


def test_full_ln_dense_bf16():
    w = W.WORKLOADS["ln_dense_bf16"]
    print(f"full {w.name}", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    y = te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g["bias"], epsilon=w.epsilon)
    torch.cuda.synchronize()
    f = {k: f64(v) for k, v in t.items()}
    ref = O.layernorm_dense_fwd(f["x"], f["kernel"], f["gamma"], f["beta"], f["bias"], epsilon=w.epsilon)["y"]
    got = f64(y)
    e = assert_rel(got, ref, TOL["bf16"], "y")
    m = check_elementwise(got, ref, rounding_bound(1), "y")     # one rounding: the normalised input
    print(f"  rel_l2 {e:.3e}, max |err| / rms {m:.3e}", flush=True)


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
    got = f64(y)
    del y, g
    f = {k: f64(v) for k, v in t.items()}
    # row blocks bound the oracle's memory (the SwiGLU h is 8192 x 28672)
    ref = np.empty_like(got)
    for r0 in range(0, w.rows, 2048):
        ref[r0:r0 + 2048] = O.layernorm_mlp_fwd(
            f["x"][r0:r0 + 2048], f["gamma"], f.get("beta"), f["kernel1"], f["kernel2"], f.get("bias1"),
            f.get("bias2"), norm_type=w.norm_type, zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
            activation_type=w.activation_type)["y"]
    e = assert_rel(got, ref, TOL["bf16"], "y")
    m = check_elementwise(got, ref, rounding_bound(2), "y")     # the normalised input and the activation output
    print(f"  rel_l2 {e:.3e}, max |err| / rms {m:.3e}", flush=True)


@pytest.fixture(scope="module")
def fp8_run():
    """The 8192 x 4096 -> 16384 -> 4096 fp8 forward (codes and h1 saved) and
    the activation backward on its saved h1, with the oracle of both."""
    w = W.WORKLOADS["ln_mlp_gelu_fp8"]
    print(f"full {w.name} forward + dact_dbias on the saved h1", flush=True)
    t = W.make_inputs(w)
    g = to_dev(t)
    q = te.QuantizerSet()
    y, saved = te.layernorm_mlp(g["x"], g["gamma"], g["beta"], [g["kernel1"], g["kernel2"]],
                                [g["bias1"], g["bias2"]], w.norm_type, epsilon=w.epsilon,
                                activation_type=w.activation_type, quantizer_set=q, return_saved=True,
                                save_codes=True)
    dx, db = te.dact_dbias(g["grad"], saved["h1"], w.activation_type, dbias_dtype=torch.bfloat16)
    # as bench.py runs it: no saved context, the codes in the workspace's tiled layout
    y_bench = te.layernorm_mlp(g["x"], g["gamma"], g["beta"], [g["kernel1"], g["kernel2"]],
                               [g["bias1"], g["bias2"]], w.norm_type, epsilon=w.epsilon,
                               activation_type=w.activation_type, quantizer_set=te.QuantizerSet())
    torch.cuda.synchronize()
    f = {k: f64(v) for k, v in t.items()}
    o = O.layernorm_mlp_fwd(f["x"], f["gamma"], f["beta"], f["kernel1"], f["kernel2"], f["bias1"], f["bias2"],
                            epsilon=w.epsilon, activation_type=w.activation_type, quant="fp8_e4m3_current")
    rdx, rdb = O.dact_dbias(f["grad"], o["h1"], w.activation_type)
    return dict(w=w, q=q, y=y, saved=saved, dx=dx, db=db, o=o, rdx=rdx, rdb=rdb, grad=f["grad"], y_bench=y_bench)


def test_full_mlp_fp8_forward(fp8_run):
    r = fp8_run
    print("full fp8 forward: every code, h1 and y element", flush=True)
    check_fp8_forward(r["q"], r["saved"], r["y"], r["o"], r["w"].activation_type, label="ln_mlp_gelu_fp8")
    # the benchmarked call (workspace codes, tiled) computes the same values in the same order
    assert torch.equal(r["y_bench"], r["y"]), "y of the call without saved codes"


def test_full_dact_dbias_on_fp8_saved_h1(fp8_run):
    """The backward half of the fp8 workload: te_dact_dbias on grad and the
    forward's own saved bf16 h1 (dx_act and a bf16 dbias1). Where the GPU's h1
    equals the oracle's, dx is the correctly rounded value (within one bf16
    step); where h1 is one bf16 step away, dx may move by |grad| x max|gelu''|
    (0.8) x that step."""
    r = fp8_run
    print("full dact_dbias on the fp8 forward's saved h1", flush=True)
    got, ref = f64(r["dx"]), r["rdx"]
    e = assert_rel(got, ref, TOL["bf16"], "dx")
    h_gpu = f64(r["saved"]["h1"])
    dh = np.abs(h_gpu - r["o"]["h1"])
    allowance = np.abs(r["grad"]) * 0.8 * dh
    check_elementwise(got, ref, DACT_FP32_REL, "dx", extra=allowance)
    # dbias: the fp32 column sums of dx (moved by the same allowance), rounded to bf16
    gdb = f64(r["db"])
    eb = assert_rel(gdb, r["rdb"], TOL["bf16"], "dbias")
    lim = bf16_ulp(r["rdb"]) + allowance.sum(axis=0) + 1e-5 * np.sqrt(np.mean(r["rdb"] ** 2))
    assert np.all(np.abs(gdb - r["rdb"]) <= lim), "dbias beyond one bf16 step plus the h1 allowance"
    print(f"  dx rel_l2 {e:.3e}, dbias rel_l2 {eb:.3e}, h1 values differing {np.count_nonzero(dh)}", flush=True)


def test_full_dact_dbias():
    """grad [8192, 16384] ~ N(0, 1) and a pre-activation of GEMM1's spread
    (N(0, 1.3^2)): dx is the correctly rounded bf16 of the fp32 value (one
    bf16 step of the oracle), dbias in fp32."""
    w = W.WORKLOADS["ln_mlp_gelu_fp8"]
    print("full dact_dbias 8192x16384 gelu", flush=True)
    a = W.make_act_inputs(w.rows, w.ffn, gated=False, dtype="bf16", seed=0, std=1.3)
    gd, xd = a["grad"].to(dev()), a["x"].to(dev())
    dx, db = te.dact_dbias(gd, xd, ("gelu",))
    torch.cuda.synchronize()
    rdx, rdb = O.dact_dbias(f64(a["grad"]), f64(a["x"]), ("gelu",))
    got = f64(dx)
    assert_rel(got, rdx, TOL["bf16"], "dx")
    check_elementwise(got, rdx, DACT_FP32_REL, "dx")
    assert_rel(f64(db), rdb, 1e-5, "dbias")


def test_full_dact_dbias_swiglu():
    """Gated (silu, linear) at the RMSNorm-SwiGLU shape: grad [8192, 14336],
    pre-activation [8192, 2 x 14336]; every element of dx, dbias in fp32."""
    w = W.WORKLOADS["rms_swiglu_bf16"]
    print("full dact_dbias 8192x2x14336 swiglu", flush=True)
    a = W.make_act_inputs(w.rows, w.ffn, gated=True, dtype="bf16", seed=0, std=1.3)
    gd, xd = a["grad"].to(dev()), a["x"].to(dev())
    dx, db = te.dact_dbias(gd, xd, ("silu", "linear"))
    torch.cuda.synchronize()
    got, gdb = f64(dx), f64(db)
    del dx, db
    F = w.ffn
    # column blocks (the same columns of both halves) bound the oracle's memory
    for c0 in range(0, F, 2048):
        c1 = min(c0 + 2048, F)
        n = c1 - c0
        xab = np.concatenate([f64(a["x"][:, c0:c1]), f64(a["x"][:, F + c0:F + c1])], axis=1)
        rdx, rdb = O.dact_dbias(f64(a["grad"][:, c0:c1]), xab, ("silu", "linear"))
        gblk = np.concatenate([got[:, c0:c1], got[:, F + c0:F + c1]], axis=1)
        assert_rel(gblk, rdx, TOL["bf16"], f"dx [{c0}:{c1}]")
        check_elementwise(gblk, rdx, DACT_FP32_REL, f"dx [{c0}:{c1}]")
        assert_rel(gdb[c0:c1], rdb[:n], 1e-5, f"dbias a[{c0}:{c1}]")
        assert_rel(gdb[F + c0:F + c1], rdb[n:], 1e-5, f"dbias b[{c0}:{c1}]")


def test_full_dact_dbias_quantize():
    """quantize_dact_dbias at 8192 x 16384 (GELU): amax over the whole dx, every
    code, dbias over all rows."""
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
    rq, _ = O.quantize(rdx, meta)
    n1, n = check_codes(codes_np(codes), rq, "dx codes")
    print(f"  dx codes one step away: {n1} of {n}", flush=True)
    assert_rel(f64(db), rdb, 1e-5, "dbias")


def test_full_norm_bwd_ln_bf16():
    """LayerNorm backward at 8192 x 4096 bf16 from the forward's saved
    statistics: every element of dx (the correctly rounded bf16 of an fp32
    value: one bf16 step of the oracle plus the fp32 statistics' error),
    dgamma and dbeta in fp32."""
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
    got = f64(dx)
    assert_rel(got, rdx, TOL["bf16"], "dx")
    check_elementwise(got, rdx, 1e-5, "dx")
    assert_rel(f64(dg), rdg, 1e-5, "dgamma")
    assert_rel(f64(db), rdb, 1e-5, "dbeta")
