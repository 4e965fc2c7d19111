"""Host-side logic of bench.py, on the CPU: the algorithmic work per launch
that the roofline's `achieved` divides by a measured duration, the roofline
fraction itself, the rule that counter traffic is reported only while the
kernel's sources are the ones it was measured on, and the one-GPU contract."""
import importlib.util
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
B = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(B)

M, H, F, G = 8192, 4096, 16384, 14336


def test_gemm_work_is_two_m_n_k():
    w = W.WORKLOADS["ln_mlp_gelu_bf16"]
    assert B.kernel_work(w, "gemm_bf16_act") == (2 * M * H * F, "flop", "mfma")
    assert B.kernel_work(w, "gemm_bf16") == (2 * M * F * H, "flop", "mfma")
    assert B.kernel_work(W.WORKLOADS["rms_swiglu_bf16"], "gemm_bf16_gated")[0] == 2 * M * H * 2 * G
    assert B.kernel_work(W.WORKLOADS["ln_dense_bf16"], "gemm_bf16")[0] == 2 * 4096 * 4096 * 12288
    assert B.kernel_work(W.WORKLOADS["ln_mlp_gelu_fp8"], "gemm_fp8_h_amax")[0] == 2 * M * H * F
    # the backward's data- and weight-gradient launches have the forward GEMMs' flops
    assert B.kernel_work(w, "gemm_bf16_dgrad")[0] == 2 * M * H * F


def test_streaming_work_counts_each_tensor_once():
    fp8 = W.WORKLOADS["ln_mlp_gelu_fp8"]
    assert B.kernel_work(fp8, "dact_dbias") == (3 * M * F * 2, "byte", "hbm")       # grad, h1 read; dx written
    assert B.kernel_work(fp8, "dact_dbias_amax")[0] == 2 * M * F * 2               # grad, h1 read
    assert B.kernel_work(fp8, "dact_quant")[0] == 2 * M * F * 2 + M * F            # + one code per element
    swiglu = W.WORKLOADS["rms_swiglu_bf16"]
    assert B.kernel_work(swiglu, "dact_dbias")[0] == (M * G + 2 * 2 * M * G) * 2   # grad; h1 and dx of width 2G
    w = W.WORKLOADS["ln_mlp_gelu_bf16"]
    assert B.kernel_work(w, "norm_bwd")[0] == 3 * M * H * 2 + 2 * M * 4            # dy, x, dx; mu, rsigma
    assert B.kernel_work(w, "norm_fwd")[0] == 2 * M * H * 2 + 2 * H * 2            # x, y; gamma, beta
    assert B.kernel_work(w, "fill_zero") is None


def test_roofline_takes_the_dominant_kernel_and_its_peak():
    w = W.WORKLOADS["ln_mlp_gelu_bf16"]
    r = B.roofline(w, {"gemm_bf16_act": (10, 8.7), "gemm_bf16": (10, 8.2), "norm_fwd": (10, 0.24)}, "bf16")
    assert (r["kernel"], r["bound"], r["unit"], r["peak"]) == ("gemm_bf16_act", "mfma", "TFLOP/s", 2516.6)
    assert r["avg_ms"] == 0.87 and r["launches"] == 10
    assert r["achieved"] == pytest.approx(2 * M * H * F / 0.87e-3 / 1e12, abs=0.01)
    assert r["frac"] == pytest.approx(r["achieved"] / 2516.6, abs=1e-4)
    d = B.roofline(W.WORKLOADS["ln_mlp_gelu_fp8"], {"dact_dbias": (10, 1.28)}, "bf16", "dact_dbias_gelu_bf16")
    assert (d["bound"], d["unit"], d["peak"]) == ("hbm", "GB/s", 8000.0)
    assert d["achieved"] == pytest.approx(3 * M * F * 2 / 0.128e-3 / 1e9, abs=0.1)
    f8 = B.roofline(W.WORKLOADS["ln_mlp_gelu_fp8"], {"gemm_fp8_h_amax": (1, 0.46)}, "fp8")
    assert f8["peak"] == 5033.2


def test_traffic_only_while_the_sources_are_unchanged(monkeypatch):
    key = ("ln_mlp_gelu_bf16", "gemm_bf16_act")
    nbytes = B.TRAFFIC[key][0]
    monkeypatch.setitem(B.TRAFFIC, key, (nbytes, B.source_hash("gemm_bf16_act")))
    assert B.traffic_of(*key) == nbytes
    monkeypatch.setitem(B.TRAFFIC, key, (nbytes, "0" * 16))
    assert B.traffic_of(*key) is None
    assert B.traffic_of("ln_mlp_gelu_bf16", "not_a_kernel") is None


def test_source_hash_follows_every_listed_file(tmp_path, monkeypatch):
    for f in ("a.hip", "b.hpp"):
        (tmp_path / f).write_text(f"// {f}\n")
    monkeypatch.setattr(B, "CSRC", str(tmp_path))
    monkeypatch.setitem(B.KERNEL_SOURCES, "k", ["a.hip", "b.hpp"])
    h0 = B.source_hash("k")
    (tmp_path / "b.hpp").write_text("// b.hpp changed\n")
    assert B.source_hash("k") != h0


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
