"""The allocation-free dact + dbias (te_dact_dbias_noalloc) through the C ABI
against te_dact_dbias with a workspace: two calls in a row, the second on a
smaller input, each bitwise equal to the workspace call (same kernels, same
partial-sum layout, so the stale partials of the first call must not leak
into the second)."""

import pytest
import torch

import workloads as W
from rmsnorm_mlp_transformer_amd import _binding as B

pytestmark = pytest.mark.gpu


def _case(rows, cols, act, gated, dbias_dtype, seed):
    a = W.make_act_inputs(rows, cols, gated=gated, dtype="bf16", seed=seed, std=1.3)
    grad, x = a["grad"].cuda(), a["x"].cuda()
    g = 2 if gated else 1
    ref_dx, got_dx = torch.empty_like(x), torch.full_like(x, float("nan"))
    ref_db = torch.empty(g * cols, dtype=dbias_dtype, device="cuda")
    got_db = torch.full_like(ref_db, float("nan"))
    dt = B.TE_BF16 if dbias_dtype == torch.bfloat16 else B.TE_F32
    n = B.te_dact_dbias_workspace_size(rows, cols, act)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    B.te_dact_dbias(grad, x, rows, cols, B.TE_BF16, act, ref_dx, ref_db, dt, ws, ws.numel())
    B.te_dact_dbias_noalloc(grad, x, rows, cols, B.TE_BF16, act, got_dx, got_db, dt)
    torch.cuda.synchronize()
    assert torch.equal(got_dx, ref_dx), f"dx differs at {rows}x{cols}"
    assert torch.equal(got_db, ref_db), f"dbias differs at {rows}x{cols}"
    return n


def test_noalloc_matches_workspace_call_twice_second_smaller():
    assert B._lib.te_dact_dbias_noalloc_scratch_bytes() == 32 << 20
    print("noalloc dact_dbias 8192x16384 gelu, then 300x1040 swiglu", flush=True)
    n1 = _case(8192, 16384, B.TE_ACT_GELU, False, torch.bfloat16, seed=1)
    n2 = _case(300, 1040, B.TE_ACT_SWIGLU, True, torch.float32, seed=2)
    assert 0 < n2 < n1 <= B._lib.te_dact_dbias_noalloc_scratch_bytes()


def test_noalloc_largest_gated_shape_fits():
    print("noalloc dact_dbias 8192x2x14336 swiglu", flush=True)
    n = _case(8192, 14336, B.TE_ACT_SWIGLU, True, torch.float32, seed=3)
    assert n <= B._lib.te_dact_dbias_noalloc_scratch_bytes()


def test_noalloc_empty_batch_zeroes_dbias():
    db = torch.full((64,), 7.0, device="cuda")
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    B.te_dact_dbias_noalloc(x, x, 0, 64, B.TE_BF16, B.TE_ACT_GELU, x, db, B.TE_F32)
    torch.cuda.synchronize()
    assert not db.any()
