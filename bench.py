"""Benchmark of the fused LayerNorm-MLP forward on one MI355X.

A step is one call of the fused forward (norm -> GEMM1 + bias + GELU ->
GEMM2 + bias) on the 8192 x 4096 -> 16384 -> 4096 bf16 workload, with all
inputs resident in HBM. The value is the GEMM work of the step (2*M*N*K per
GEMM) divided by the step's wall time, in TFLOP/s. The other workloads
(LayerNorm+Dense, RMSNorm-SwiGLU, the fp8 forward and the activation
backward) are measured the same way and reported under "parts".

Each measurement starts by running steps for --settle-ms (300 ms) so that
the GPU clock has ramped up after the idle time spent generating inputs on
the host, then runs W warmup steps. It then has two timed regions of K
steps, back to back on the
same inputs. The first has no instrumentation: its wall time gives
"ms_per_step" and "value". In the second the library's per-kernel timing is
on (te_timing_enable): each launch carries two HIP events on its stream that
the runtime stamps with the kernel's own start and end (the durations sum to
the uninstrumented step time), but the event-carrying dispatches lengthen the
step by several microseconds per launch, which is why the step time comes
from the first region. The dominant kernel's average duration from the
second region is the "roofline" entry. The
"cpu_baseline" entry times the fp64 oracle on a bounded row sample.

The "traffic" entry is the HBM traffic per launch of the dominant kernel
measured with rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each in its own
run, scaled by what the same counters report for a plain device copy of
known size); it is stored in TRAFFIC below together with a hash of the
kernel's source files and reported as null once those sources change.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                       [--no-parts] [--no-cpu-baseline] [--workload NAME]
       python bench.py --copy-probe MIB      (plain copy, for counter scaling)
       python bench.py --mfma-probe ITERS    (the library's MFMA issue-rate probe, bf16 and fp8)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as W  # noqa: E402

PEAK = {"bf16": 2516.6, "fp8": 5033.2, "fp32": 157.3}   # dense TFLOP/s, MI355X spec
MFMA_PROBE_BLOCKS = 512   # the MFMA probe: two 4-wave workgroups per compute unit, the GEMMs' 8 waves
CSRC = os.path.join(ROOT, "rmsnorm_mlp_transformer_amd", "csrc")
# Source files that define each kernel (for the staleness check of TRAFFIC).
_GEMM_HDR = ["gemm_common.hpp", "gemm_lds.hpp", "te_common.hpp", "te_kernels.hpp"]
_GEMM_NC = ["gemm_bf16.hip"] + _GEMM_HDR     # N-contiguous bf16 kernel
_GEMM_KC = ["gemm_bt.hip"] + _GEMM_HDR       # K-contiguous fp8 kernel
_ELEM = ["elementwise.hip", "te_common.hpp", "gemm_lds.hpp", "te_kernels.hpp"]
KERNEL_SOURCES = {
    "gemm_bf16_act": _GEMM_NC, "gemm_bf16": _GEMM_NC, "gemm_bf16_gated": _GEMM_NC, "gemm_bf16_wgrad": _GEMM_NC,
    "gemm_bf16_dgrad": _GEMM_NC, "gemm_fp8_h_amax": _GEMM_KC, "gemm_fp8": _GEMM_KC,
    "dact_dbias": _ELEM, "dact_quant": _ELEM, "dact_dbias_amax": _ELEM, "dact_dbias_act": _ELEM,
    "norm_bwd": ["norm_bwd.hip", "te_common.hpp", "gemm_lds.hpp", "te_kernels.hpp"],
}
# Counter-measured HBM bytes per launch: {(workload, kernel): (bytes, source hash)}.
# FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (the plain-copy scales); the summary is
# profiles/counters_all_kernels_bench.md. The backward's entry is the mean of
# its two data-gradient GEMMs (dY.kernel2^T and dh1.kernel1^T), one launch each per step.
TRAFFIC = {
    ("ln_mlp_gelu_bf16", "gemm_bf16_act"): (1879751421, "d55708a0a33af1ce"),
    ("ln_dense_bf16", "gemm_bf16"): (704840997, "d55708a0a33af1ce"),
    ("rms_swiglu_bf16", "gemm_bf16_gated"): (3131502716, "d55708a0a33af1ce"),
    ("ln_mlp_gelu_fp8", "gemm_fp8_h_amax"): (1506785615, "7f89454f7470d907"),
    ("dact_dbias_gelu_bf16", "dact_dbias"): (822146125, "df51bb2c756db03b"),
    ("dact_dbias_swiglu_bf16", "dact_dbias"): (1208105697, "df51bb2c756db03b"),
    ("norm_bwd_ln_bf16", "norm_bwd"): (210002194, "213aacdb597a6a36"),
    ("dact_dbias_quantize_gelu_bf16", "dact_quant"): (671154152, "df51bb2c756db03b"),
    ("dact_dbias_quantize_gelu_bf16", "dact_dbias_amax"): (553980510, "df51bb2c756db03b"),
    ("ln_mlp_gelu_bf16_backward", "gemm_bf16_dgrad"): (1872582233, "d55708a0a33af1ce"),
}


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


HBM_PEAK_GBS = 8000.0
METRIC = "fused LN-MLP fwd TFLOP/s + % of MI355X bf16/fp8 MFMA peak; dact+dbias GB/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# working sets under twice the 256 MB memory-side cache can still partly hit in it across
# steps: those rotate input sets
ROTATE_BELOW = 512 << 20
ROTATE_SETS = 4


class Case:
    """Inputs on the device plus a closure running one step. When the step's
    working set (inputs, output and workspace) is under ROTATE_BELOW, the
    memory-side cache could hold much of it across steps, so ROTATE_SETS independent input sets
    (seeds 0, 1, ...) are cycled through, one per step."""

    def __init__(self, w: W.Workload, te, dev):
        self.w = w
        sets = [{k: v.to(dev) for k, v in W.make_inputs(w).items()}]
        g0 = sets[0]
        self.qset = te.QuantizerSet(dev) if w.quant != "none" else None
        if w.kind == "dense":
            ws_n = te.te_layernorm_dense_fwd_workspace_size(w.rows, w.hidden, w.ffn, 1,
                                                            1 if self.qset else 0)
            out_shape = (w.rows, w.ffn)
        else:
            act = te.act_type_of(w.activation_type)
            ws_n = te.te_layernorm_mlp_fwd_workspace_size(w.rows, w.hidden, w.ffn,
                                                          0 if w.dtype == "fp32" else 1, act,
                                                          1 if self.qset else 0)
            out_shape = (w.rows, w.hidden)
        self.ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
        self.y = torch.empty(*out_shape, dtype=g0["x"].dtype, device=dev)
        working = sum(v.numel() * v.element_size() for v in g0.values()) + ws_n + \
            self.y.numel() * self.y.element_size()
        self.rotated = working < ROTATE_BELOW
        if self.rotated:
            sets += [{k: v.to(dev) for k, v in W.make_inputs(w, seed=i).items()} for i in range(1, ROTATE_SETS)]
        self.working_set = working
        self.i = 0

        def fn():
            g = sets[self.i % len(sets)]
            self.i += 1
            if w.kind == "dense":
                return te.layernorm_dense(g["x"], g["kernel"], g["gamma"], g["beta"], g.get("bias"),
                                          epsilon=w.epsilon, quantizer_set=self.qset, workspace=self.ws, out=self.y)
            return te.layernorm_mlp(
                g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]], [g.get("bias1"), g.get("bias2")],
                w.norm_type, zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                activation_type=w.activation_type, quantizer_set=self.qset, workspace=self.ws, out=self.y)
        self.fn = fn

    def flops(self):
        return self.w.gemm_flops()


class DactCase:
    """dact + dbias on the pre-activation h1 [M, G*F] that the workload's own
    forward saved (bf16) and grad [M, F]: for the fp8 workload its grad tensor
    (~N(0, 1), bf16) and the fp8 forward's h1, with dbias written in bf16 as
    the workload states; for the others grad ~ N(0, 1) drawn after the
    forward's inputs and dbias in fp32."""

    def __init__(self, w: W.Workload, te, dev):
        self.w = w
        g = 2 if w.gated else 1
        t = {k: v.to(dev) for k, v in W.make_inputs(w).items()}
        qset = te.QuantizerSet(dev) if w.quant != "none" else None
        _, saved = te.layernorm_mlp(t["x"], t["gamma"], t.get("beta"), [t["kernel1"], t["kernel2"]],
                                    [t.get("bias1"), t.get("bias2")], w.norm_type,
                                    zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                                    activation_type=w.activation_type, quantizer_set=qset, return_saved=True)
        self.h1 = saved["h1"]
        del saved
        if "grad" in t:
            self.grad = t["grad"]
        else:
            gen = torch.Generator(device="cpu").manual_seed(7)
            self.grad = torch.randn(w.rows, w.ffn, generator=gen).to(torch.bfloat16).to(dev)
        del t
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        self.dx = torch.empty_like(self.h1)
        dbias_bf16 = w.quant != "none"
        self.dbias = torch.empty(g * w.ffn, dtype=torch.bfloat16 if dbias_bf16 else torch.float32, device=dev)
        act = te.act_type_of(w.activation_type)
        n = te.te_dact_dbias_workspace_size(w.rows, w.ffn, act)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        B = te._binding
        ddt = B.TE_BF16 if dbias_bf16 else B.TE_F32

        def fn():
            B.te_dact_dbias(self.grad, self.h1, w.rows, w.ffn, B.TE_BF16, act, self.dx, self.dbias, ddt,
                            self.ws, self.ws.numel())
        self.fn = fn

    def bytes(self):
        # grad + h1 read, dx written (bf16), dbias written
        g = 2 if self.w.gated else 1
        return (1 + 2 * g) * self.w.rows * self.w.ffn * 2 + g * self.w.ffn * self.dbias.element_size()


class DactQuantCase(DactCase):
    """dact + dbias with dx quantised to E4M3 (current scaling): two passes over
    grad and h1 (amax, then codes)."""

    def __init__(self, w: W.Workload, te, dev):
        super().__init__(w, te, dev)
        g = 2 if w.gated else 1
        self.codes = torch.empty(w.rows, g * w.ffn, dtype=torch.uint8, device=dev)
        self.meta = te.Fp8Meta()
        act = te.act_type_of(w.activation_type)
        n = te.te_dact_dbias_quantize_workspace_size(w.rows, w.ffn, act)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        B = te._binding

        def fn():
            B.te_dact_dbias_quantize(self.grad, self.h1, w.rows, w.ffn, B.TE_BF16, act, self.codes, self.meta,
                                     self.dbias, B.TE_F32, self.ws, self.ws.numel())
        self.fn = fn

    def bytes(self):
        # grad + h1 read in each of the two passes, codes written once, dbias written
        g = 2 if self.w.gated else 1
        return 2 * (1 + g) * self.w.rows * self.w.ffn * 2 + g * self.w.rows * self.w.ffn + g * self.w.ffn * 4


class NormBwdCase:
    """LayerNorm backward at the bench workload's normalisation shape: dy, x
    (bf16) and the forward's saved mu / rsigma -> dx, dgamma, dbeta (fp32).
    The working set (dy, x, dx: 192 MB) is under the 256 MB memory-side
    cache, so ROTATE_SETS input sets (x from seeds 0.., dy from seeds 5..)
    are cycled through."""

    def __init__(self, w: W.Workload, te, dev):
        self.w = w
        B = te._binding
        sets = []
        for i in range(ROTATE_SETS):
            t = W.make_inputs(w, seed=i)
            gen = torch.Generator(device="cpu").manual_seed(5 + i)
            dy = torch.randn(w.rows, w.hidden, generator=gen).to(torch.bfloat16).to(dev)
            x, gamma = t["x"].to(dev), t["gamma"].to(dev)
            _, mu, rs = te.layernorm(x, gamma, t["beta"].to(dev), "layernorm", False, w.epsilon, return_stats=True)
            sets.append((dy, x, gamma, mu, rs, torch.empty_like(x)))
        self.dg = torch.empty(w.hidden, dtype=torch.float32, device=dev)
        self.db = torch.empty(w.hidden, dtype=torch.float32, device=dev)
        n = B.te_layernorm_bwd_workspace_size(w.rows, w.hidden, B.TE_BF16)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        self.i = 0

        def fn():
            dy, x, gamma, mu, rs, dx = sets[self.i % len(sets)]
            self.i += 1
            B.te_layernorm_bwd(dy, x, mu, rs, gamma, w.rows, w.hidden, B.TE_BF16, B.TE_LAYERNORM, 0, dx, self.dg,
                               self.db, B.TE_F32, self.ws, self.ws.numel())
        self.fn = fn

    def bytes(self):
        # dy and x read, dx written (bf16); mu, rsigma read; dgamma, dbeta written
        M, H = self.w.rows, self.w.hidden
        return 3 * M * H * 2 + 2 * M * 4 + 2 * H * 4


class MlpBwdCase:
    """The LayerNorm-MLP backward from the forward's saved context (h1, mu,
    rsigma): 4 GEMMs (two data-gradient, two weight-gradient), the activation
    backward with dbias1, dbias2, and the normalisation backward."""

    def __init__(self, w: W.Workload, te, dev):
        self.w = w
        t = W.make_inputs(w)
        self.g = {k: v.to(dev) for k, v in t.items()}
        g = self.g
        gen = torch.Generator(device="cpu").manual_seed(3)
        self.gy = torch.randn(w.rows, w.hidden, generator=gen).to(torch.bfloat16).to(dev)
        _, self.saved = te.layernorm_mlp(g["x"], g["gamma"], g.get("beta"), [g["kernel1"], g["kernel2"]],
                                         [g.get("bias1"), g.get("bias2")], w.norm_type,
                                         zero_centered_gamma=w.zero_centered_gamma, epsilon=w.epsilon,
                                         activation_type=w.activation_type, return_saved=True)
        B = te._binding
        act = te.act_type_of(w.activation_type)
        gg = 2 if w.gated else 1
        self.out = {"dx": torch.empty_like(g["x"]), "dgamma": torch.empty(w.hidden, device=dev),
                    "dbeta": torch.empty(w.hidden, device=dev), "dkernel1": torch.empty_like(g["kernel1"]),
                    "dkernel2": torch.empty_like(g["kernel2"]), "dbias1": torch.empty(gg * w.ffn, device=dev),
                    "dbias2": torch.empty(w.hidden, device=dev)}
        n = B.te_layernorm_mlp_bwd_workspace_size(w.rows, w.hidden, w.ffn, act)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        o, sv = self.out, self.saved
        norm = B.TE_LAYERNORM if w.norm_type == "layernorm" else B.TE_RMSNORM

        def fn():
            B.te_layernorm_mlp_bwd(self.gy, g["x"], g["gamma"], g.get("beta"), g["kernel1"], g["kernel2"], sv["mu"],
                                   sv["rsigma"], sv["h1"], w.rows, w.hidden, w.ffn, B.TE_BF16, norm,
                                   w.zero_centered_gamma, w.epsilon, act, o["dx"], o["dgamma"], o["dbeta"],
                                   o["dkernel1"], o["dbias1"], o["dkernel2"], o["dbias2"], B.TE_F32, self.ws,
                                   self.ws.numel())
        self.fn = fn

    def flops(self):
        # two data-gradient and two weight-gradient GEMMs, each 2*M*N*K
        return 2 * self.w.gemm_flops()


SETTLE_MS = 300.0


def settle(fn, min_ms):
    """Runs steps until the GPU has been busy for about min_ms. After an idle
    period (the host generating the next workload's inputs) the GPU clock
    takes tens of milliseconds to ramp up: the first 20 steps of an
    8192 x 4096 -> 12288 dense call measured 0.78, 0.37, 0.36, 0.35 ms per
    step, then a steady 0.346. Every timed step is still a whole step."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def time_steps(fn, steps, warmup, te=None, settle_ms=None):
    """(ms per step over `steps` uninstrumented steps, per-kernel timing of
    `steps` more steps with the library's launch events on). Before the
    `warmup` steps, steps run until the clock has settled (settle())."""
    settle(fn, SETTLE_MS if settle_ms is None else settle_ms)
    for _ in range(warmup):
        fn()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    kernels = {}
    if te is not None:
        te.te_timing_reset()
        te.te_timing_enable(True)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        kernels = te.te_timing_collect()
        te.te_timing_enable(False)
    return ms, kernels


def kernel_work(w: W.Workload, name: str):
    """Algorithmic work of one launch of a kernel of the given workload:
    (amount, unit, bound)."""
    g = 2 if w.gated else 1
    M, H, F = w.rows, w.hidden, w.ffn
    if name.startswith("gemm"):
        if w.kind == "dense":
            return 2 * M * H * F, "flop", "mfma"
        if name in ("gemm_bf16_act", "gemm_bf16_gated", "gemm_fp8_h_amax"):
            return 2 * M * H * g * F, "flop", "mfma"
        if name in ("gemm_bf16_dgrad", "gemm_bf16_wgrad"):   # average of the launch pair (GEMM1 and GEMM2 shapes)
            return (2 * M * H * g * F + 2 * M * F * H) // 2, "flop", "mfma"
        return 2 * M * F * H, "flop", "mfma"
    if name == "dact_dbias":   # grad [M, F], h1 and dx [M, G*F], bf16
        return (1 + 2 * g) * M * F * 2, "byte", "hbm"
    if name == "norm_bwd":   # dy, x read and dx written (bf16), mu and rsigma read
        return 3 * M * H * 2 + 2 * M * 4, "byte", "hbm"
    if name == "dact_dbias_amax":   # grad and h1 read
        return (1 + g) * M * F * 2, "byte", "hbm"
    if name == "dact_quant":   # grad and h1 read, E4M3 codes [M, G*F] written
        return (1 + g) * M * F * 2 + g * M * F, "byte", "hbm"
    if name == "norm_fwd":
        return 2 * M * H * 2 + 2 * H * 2, "byte", "hbm"
    return None


def traffic_of(workload, kernel):
    rec = TRAFFIC.get((workload, kernel))
    if rec is None or kernel not in KERNEL_SOURCES or rec[1] != source_hash(kernel):
        return None
    return rec[0]


def roofline(w, kernels, dtype_key, wname=None):
    if not kernels:
        return None
    name, (cnt, total) = max(kernels.items(), key=lambda kv: kv[1][1])
    work = kernel_work(w, name)
    if work is None:
        return None
    amount, unit, bound = work
    avg_s = total / cnt / 1e3
    if unit == "flop":
        achieved = amount / avg_s / 1e12
        peak = PEAK[dtype_key]
        u = "TFLOP/s"
    else:
        achieved = amount / avg_s / 1e9
        peak = HBM_PEAK_GBS
        u = "GB/s"
    return {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": u,
            "frac": round(achieved / peak, 4), "traffic": traffic_of(wname or w.name, name),
            "work_per_launch": amount, "work_unit": unit, "avg_ms": round(total / cnt, 4),
            "launches": cnt}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        return os.cpu_count()


def cpu_baseline(w: W.Workload, budget_s: float = 15.0):
    """Times the fp64 oracle forward on a bounded row sample of workload w:
    blocks of consecutive rows (16, 32, ... up to 1024), taken from the start
    of the input and wrapping round, until about budget_s of CPU work."""
    import oracle as O
    threads = _blas_threads()
    t = W.make_inputs(w)
    f = {k: W.to_f64(v) for k, v in t.items()}
    rows = 16
    done_rows, elapsed = 0, 0.0
    while elapsed < budget_s and done_rows < w.rows:
        start = done_rows % w.rows
        sel = slice(start, min(start + rows, w.rows))
        t0 = time.perf_counter()
        O.layernorm_mlp_fwd(f["x"][sel], f["gamma"], f.get("beta"), f["kernel1"], f["kernel2"], f.get("bias1"),
                            f.get("bias2"), norm_type=w.norm_type, zero_centered_gamma=w.zero_centered_gamma,
                            epsilon=w.epsilon, activation_type=w.activation_type)
        elapsed += time.perf_counter() - t0
        done_rows += sel.stop - sel.start
        rows = min(rows * 2, 1024)
    flops = w.scaled(rows=done_rows).gemm_flops()
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle forward of {done_rows} rows in blocks of the {w.rows}-row input "
                      f"({elapsed:.1f} s of CPU work)"}


def cpu_baseline_fp8(w: W.Workload, rows: int = 512):
    """The oracle's fp8 forward (x-hat, both kernels and the activation
    quantised with current scaling, the E4M3 GEMMs in fp64) on the first
    `rows` rows of the workload (its scales taken over that sample), then its
    dact + dbias on those rows' h1 and grad: seconds, TFLOP/s and GB/s at the
    workload's own work per row."""
    import oracle as O
    t = W.make_inputs(w)
    f = {k: W.to_f64(v) for k, v in t.items()}
    t0 = time.perf_counter()
    o = O.layernorm_mlp_fwd(f["x"][:rows], f["gamma"], f["beta"], f["kernel1"], f["kernel2"], f["bias1"], f["bias2"],
                            epsilon=w.epsilon, activation_type=w.activation_type, quant="fp8_e4m3_current")
    fwd_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.dact_dbias(f["grad"][:rows], o["h1"], w.activation_type)
    bwd_s = time.perf_counter() - t0
    g = 2 if w.gated else 1
    return {"fwd": {"value": round(w.scaled(rows=rows).gemm_flops() / fwd_s / 1e12, 6), "unit": "TFLOP/s",
                    "seconds": round(fwd_s, 2)},
            "dact_dbias": {"value": round((1 + 2 * g) * rows * w.ffn * 2 / bwd_s / 1e9, 3), "unit": "GB/s",
                           "seconds": round(bwd_s, 3)},
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"fp64 oracle fp8 forward of the first {rows} rows (scales over the sample, both kernels "
                      f"quantised in full), then its dact + dbias on those rows"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ln_mlp_gelu_bf16")
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="run steps for this long before the warmup steps of each measurement (clock ramp)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times)")
    ap.add_argument("--mfma-probe", type=int, default=0,
                    help="only run the library's MFMA issue-rate probe with this many iterations per chain")
    args = ap.parse_args()
    if args.mfma_probe:
        import rmsnorm_mlp_transformer_amd as te
        out = {"blocks": MFMA_PROBE_BLOCKS, "iters": args.mfma_probe}
        for name, fp8, peak in (("bf16", False, PEAK["bf16"]), ("fp8", True, PEAK["fp8"])):
            t_end = time.perf_counter() + SETTLE_MS / 1e3   # clock settle, as for the workloads
            while time.perf_counter() < t_end:
                te.probe_mfma(fp8, args.mfma_probe, MFMA_PROBE_BLOCKS)
            runs = [te.probe_mfma(fp8, args.mfma_probe, MFMA_PROBE_BLOCKS) for _ in range(3)]
            ms, flops, sticks, rticks = sorted(runs)[1]
            tflops = flops / (ms * 1e-3) / 1e12
            out[name] = {"ms": round(ms, 4), "TFLOP/s": round(tflops, 1), "frac_of_peak": round(tflops / peak, 4),
                         "clock_GHz": round(sticks / rticks * 0.1, 3)}
        print(json.dumps({"mfma_probe": out}), flush=True)
        return
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this library has no "
              "multi-GPU path; the value is the single-GPU throughput", file=sys.stderr)
        sys.exit(2)
    import rmsnorm_mlp_transformer_amd as te
    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    dkey = "fp8" if w.quant != "none" else w.dtype
    log(f"bench: {w.name} rows={w.rows} hidden={w.hidden} ffn={w.ffn} dtype={dkey}")
    case = Case(w, te, dev)
    ms, kernels = time_steps(case.fn, args.steps, args.warmup, te, args.settle_ms)
    value = case.flops() / (ms / 1e3) / 1e12
    log(f"bench: {ms:.4f} ms/step, {value:.1f} TFLOP/s, kernels {kernels}")
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dkey == "bf16" else dkey, "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "hidden": w.hidden, "ffn": w.ffn,
                   "norm": w.norm_type, "activation": list(w.activation_type), "quant": w.quant,
                   "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK[dkey], 4),
        "roofline": roofline(w, kernels, dkey),
        "kernels_ms": {k: round(v[1] / v[0], 4) for k, v in kernels.items()},
    }
    if not args.no_parts:
        parts = {}
        for name in ("ln_dense_bf16", "rms_swiglu_bf16", "ln_mlp_gelu_fp8"):
            if name == w.name:
                continue
            pw = W.WORKLOADS[name]
            c = Case(pw, te, dev)
            pms, pk = time_steps(c.fn, max(10, args.steps), 3, te, args.settle_ms)
            pv = c.flops() / (pms / 1e3) / 1e12
            pkey = "fp8" if pw.quant != "none" else pw.dtype
            parts[name] = {"ms_per_step": round(pms, 4), "TFLOP/s": round(pv, 2),
                           "frac_of_peak": round(pv / PEAK[pkey], 4),
                           "kernels_ms": {k: round(v[1] / v[0], 4) for k, v in pk.items()},
                           "roofline": roofline(pw, pk, pkey)}
            if c.rotated:
                parts[name]["input_sets"] = ROTATE_SETS
            if pw.quant != "none" and pk:
                # the same step with the kernels' amax and quantise-transpose
                # passes taken out (weights quantised once, ahead of the
                # steps), and the two fp8 GEMMs alone, from the measured
                # per-kernel durations of the instrumented region
                per = {k: v[1] / v[0] for k, v in pk.items()}
                wq_ms = per.get("amax", 0.0) + per.get("quantize_transpose", 0.0)
                gemm_ms = sum(v for k, v in per.items() if k.startswith("gemm"))
                parts[name]["prequantised_weights"] = {
                    "ms_per_step": round(pms - wq_ms, 4),
                    "TFLOP/s": round(c.flops() / ((pms - wq_ms) / 1e3) / 1e12, 2),
                    "frac_of_peak": round(c.flops() / ((pms - wq_ms) / 1e3) / 1e12 / PEAK[pkey], 4)}
                parts[name]["gemm_only"] = {
                    "ms": round(gemm_ms, 4), "TFLOP/s": round(c.flops() / (gemm_ms / 1e3) / 1e12, 2),
                    "frac_of_peak": round(c.flops() / (gemm_ms / 1e3) / 1e12 / PEAK[pkey], 4)}
            log(f"bench part {name}: {pms:.4f} ms, {pv:.1f} TFLOP/s")
            del c
            torch.cuda.empty_cache()
        # activation backward: the fp8 workload's backward half (its grad and the
        # h1 its fp8 forward saved, bf16 dbias) and, gated, at the SwiGLU
        # workload's shape on the h1 its bf16 forward saved
        for pname, wname in (("dact_dbias_gelu_bf16", "ln_mlp_gelu_fp8"), ("dact_dbias_swiglu_bf16", "rms_swiglu_bf16")):
            dw = W.WORKLOADS[wname]
            d = DactCase(dw, te, dev)
            dms, dk = time_steps(d.fn, max(10, args.steps), 3, te, args.settle_ms)
            gbs = d.bytes() / (dms / 1e3) / 1e9
            parts[pname] = {"shape": [dw.rows, (2 if dw.gated else 1) * dw.ffn],
                            "activation": list(dw.activation_type),
                            "h1": f"saved by the {wname} forward", "dbias_dtype": str(d.dbias.dtype)[6:],
                            "ms_per_step": round(dms, 4), "GB/s": round(gbs, 1),
                            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                            "kernels_ms": {k: round(v[1] / v[0], 4) for k, v in dk.items()},
                            "roofline": roofline(dw, {k: v for k, v in dk.items() if k == "dact_dbias"}, "bf16",
                                                 pname)}
            log(f"bench part {pname}: {dms:.4f} ms, {gbs:.0f} GB/s")
            del d
            torch.cuda.empty_cache()
        # the whole LayerNorm-MLP backward at the bench workload's shape
        bw = W.WORKLOADS["ln_mlp_gelu_bf16"]
        bc = MlpBwdCase(bw, te, dev)
        bms, bk = time_steps(bc.fn, max(5, args.steps // 2), 2, te, args.settle_ms)
        bv = bc.flops() / (bms / 1e3) / 1e12
        parts["ln_mlp_gelu_bf16_backward"] = {
            "ms_per_step": round(bms, 4), "TFLOP/s": round(bv, 2), "frac_of_peak": round(bv / PEAK["bf16"], 4),
            "kernels_ms": {k: round(v[1] / v[0], 4) for k, v in bk.items()},
            "roofline": roofline(bw, {k: v for k, v in bk.items() if k.startswith("gemm")}, "bf16",
                                 "ln_mlp_gelu_bf16_backward")}
        log(f"bench part backward: {bms:.4f} ms, {bv:.1f} TFLOP/s")
        del bc
        torch.cuda.empty_cache()
        # normalisation backward at the bench workload's shape
        nw = W.WORKLOADS["ln_mlp_gelu_bf16"]
        nbc = NormBwdCase(nw, te, dev)
        nms, nk = time_steps(nbc.fn, max(10, args.steps), 3, te, args.settle_ms)
        gbs = nbc.bytes() / (nms / 1e3) / 1e9
        parts["norm_bwd_ln_bf16"] = {
            "shape": [nw.rows, nw.hidden], "ms_per_step": round(nms, 4), "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "kernels_ms": {k: round(v[1] / v[0], 4) for k, v in nk.items()},
            "roofline": roofline(nw, {k: v for k, v in nk.items() if k == "norm_bwd"}, "bf16", "norm_bwd_ln_bf16")}
        log(f"bench part norm_bwd: {nms:.4f} ms, {gbs:.0f} GB/s")
        del nbc
        torch.cuda.empty_cache()
        # the quantising variant (fp8 backward), GELU shape
        dw = W.WORKLOADS["ln_mlp_gelu_fp8"]
        d = DactQuantCase(dw, te, dev)
        dms, dk = time_steps(d.fn, max(10, args.steps), 3, te, args.settle_ms)
        gbs = d.bytes() / (dms / 1e3) / 1e9
        parts["dact_dbias_quantize_gelu_bf16"] = {
            "shape": [dw.rows, dw.ffn], "activation": list(dw.activation_type), "ms_per_step": round(dms, 4),
            "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "kernels_ms": {k: round(v[1] / v[0], 4) for k, v in dk.items()},
            "roofline": roofline(dw, {k: v for k, v in dk.items() if k in ("dact_dbias_amax", "dact_quant")},
                                 "bf16", "dact_dbias_quantize_gelu_bf16")}
        log(f"bench part dact_dbias_quantize: {dms:.4f} ms, {gbs:.0f} GB/s")
        del d
        torch.cuda.empty_cache()
        result["parts"] = parts
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"bench cpu baseline: {result['cpu_baseline']}")
        if not args.no_parts:
            result["cpu_baseline_fp8"] = cpu_baseline_fp8(W.WORKLOADS["ln_mlp_gelu_fp8"])
            log(f"bench cpu baseline fp8: {result['cpu_baseline_fp8']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
