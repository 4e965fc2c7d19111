"""The entry points inside a captured HIP graph.

Every call of the library is asynchronous on the caller's stream and
allocates, frees, copies, clears or synchronises nothing (the fp8 metadata is
cleared by a fill kernel), so a serving loop can capture a call once and
replay it. Each test captures one call, then replays it several times with
the output cleared before each replay and eager calls and synchronisations
in between, and requires every replay to reproduce the eager result bit for
bit (the eager result itself is held to the oracle by the parity tests)."""

import pytest
import torch

import rmsnorm_mlp_transformer_amd as te
import workloads as W
from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture_and_replay(fn, outs):
    """fn() runs the call; outs are the tensors it writes."""
    fn()                                  # eager reference (after any lazy set-up)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"replay {r}: output {i} differs from the eager call"
        fn()                              # eager work between replays
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e)


@pytest.mark.parametrize("quant", ["none", "fp8"])
@pytest.mark.parametrize("act", [("gelu",), ("silu", "linear")], ids=["gelu", "swiglu"])
def test_layernorm_mlp_graph_replay(quant, act):
    print(f"graph layernorm_mlp {quant} {act}", flush=True)
    gated = len(act) == 2
    w = W.WORKLOADS["ln_mlp_gelu_bf16"].scaled(rows=600, hidden=512, ffn=1024)
    t = W.make_inputs(w)
    if gated:
        gen = torch.Generator().manual_seed(5)
        t["kernel1"] = (torch.randn(w.hidden, 2 * w.ffn, generator=gen) * 0.02).to(torch.bfloat16)
        t["bias1"] = (torch.randn(2 * w.ffn, generator=gen) * 0.02).to(torch.bfloat16)
    g = to_dev(t)
    qset = te.QuantizerSet(dev()) if quant == "fp8" else None
    ws = torch.empty(te.te_layernorm_mlp_fwd_workspace_size(w.rows, w.hidden, w.ffn, 1, te.act_type_of(act),
                                                            1 if qset else 0), dtype=torch.uint8, device=dev())
    y = torch.empty(w.rows, w.hidden, dtype=torch.bfloat16, device=dev())

    def fn():
        te.layernorm_mlp(g["x"], g["gamma"], g["beta"], [g["kernel1"], g["kernel2"]], [g["bias1"], g["bias2"]],
                         "layernorm", epsilon=w.epsilon, activation_type=act, quantizer_set=qset, workspace=ws,
                         out=y)

    outs = [y]
    if qset is not None:
        outs += [m.buf for m in (qset.x, qset.w1, qset.act, qset.w2)]   # amax, scale, scale_inv
    _capture_and_replay(fn, outs)


def test_dact_dbias_graph_replay():
    print("graph dact_dbias", flush=True)
    a = W.make_act_inputs(1000, 1536, gated=False, dtype="bf16", seed=4, std=1.3)
    grad, x = a["grad"].to(dev()), a["x"].to(dev())
    B = te._binding
    act = te.act_type_of(("gelu",))
    dx = torch.empty_like(x)
    dbias = torch.empty(1536, dtype=torch.float32, device=dev())
    ws = torch.empty(max(te.te_dact_dbias_workspace_size(1000, 1536, act), 16), dtype=torch.uint8, device=dev())

    def fn():
        B.te_dact_dbias(grad, x, 1000, 1536, B.TE_BF16, act, dx, dbias, B.TE_F32, ws, ws.numel())

    _capture_and_replay(fn, [dx, dbias])
