"""Seeded synthetic inputs for the fused norm-MLP workloads.

This module only draws random tensors: it holds none of the method's
arithmetic. Both the fp64 oracle (through the tests) and the GPU path are fed
from it, so the two sides always see the very same rounded values.

Recipe (shared by every workload):
  * one ``torch.Generator('cpu')`` per call, seeded with ``seed`` (default 0);
  * tensors are drawn in the fixed order x, gamma, beta, kernel1, bias1,
    kernel2, bias2, grad (a tensor the workload does not use is skipped, so
    it consumes no random numbers);
  * every tensor is drawn as float32 ``torch.randn``, multiplied by its
    standard deviation, shifted by its mean, and then cast once to the
    workload dtype with round-to-nearest-even.

Workloads (sizes are rows x hidden -> ffn -> hidden unless noted):
  ln_mlp_tiny_fp32   64 x 128 -> 512 -> 128, fp32, LayerNorm eps 1e-6, GELU(tanh)
  ln_dense_bf16      4096 x 4096 -> 12288, bf16, LayerNorm eps 1e-5, with bias
  ln_mlp_gelu_bf16   8192 x 4096 -> 16384 -> 4096, bf16, LayerNorm eps 1e-6, GELU(tanh)
  rms_swiglu_bf16    8192 x 4096 -> 2x14336 -> 4096, bf16, RMSNorm eps 1e-6,
                     zero-centred gamma, gated (silu, linear), no biases
  ln_mlp_gelu_fp8    the ln_mlp_gelu_bf16 tensors with per-tensor E4M3 current
                     scaling, plus grad [8192, 16384] ~ N(0, 1) for the
                     activation backward (dact + dbias)

Distributions: x ~ N(0,1); gamma = 1 + N(0,0.1) (zero-centred: N(0,0.1));
beta ~ N(0,0.1); kernels and biases ~ N(0,0.02); grad ~ N(0,1).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str               # "mlp" or "dense"
    rows: int
    hidden: int
    ffn: int                # output features for "dense"
    dtype: str              # "fp32" or "bf16"
    quant: str              # "none" or "fp8_e4m3_current"
    norm_type: str          # "layernorm" or "rmsnorm"
    zero_centered_gamma: bool
    epsilon: float
    activation_type: tuple  # e.g. ("gelu",) or ("silu", "linear")
    biases: bool
    with_grad: bool = False

    @property
    def gated(self) -> bool:
        return len(self.activation_type) == 2

    def scaled(self, rows: Optional[int] = None, hidden: Optional[int] = None,
               ffn: Optional[int] = None) -> "Workload":
        """The same recipe at other sizes (for parity tests the oracle can finish)."""
        return dataclasses.replace(
            self,
            name=f"{self.name}@{rows or self.rows}x{hidden or self.hidden}x{ffn or self.ffn}",
            rows=rows or self.rows, hidden=hidden or self.hidden, ffn=ffn or self.ffn)

    def gemm_flops(self) -> int:
        """2*M*N*K summed over the GEMMs of one forward."""
        g = 2 if self.gated else 1
        if self.kind == "dense":
            return 2 * self.rows * self.hidden * self.ffn
        return 2 * self.rows * self.hidden * g * self.ffn + 2 * self.rows * self.ffn * self.hidden


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("ln_mlp_tiny_fp32", "mlp", 64, 128, 512, "fp32", "none", "layernorm",
                 False, 1e-6, ("gelu",), True),
        Workload("ln_dense_bf16", "dense", 4096, 4096, 12288, "bf16", "none", "layernorm",
                 False, 1e-5, (), True),
        Workload("ln_mlp_gelu_bf16", "mlp", 8192, 4096, 16384, "bf16", "none", "layernorm",
                 False, 1e-6, ("gelu",), True),
        Workload("rms_swiglu_bf16", "mlp", 8192, 4096, 14336, "bf16", "none", "rmsnorm",
                 True, 1e-6, ("silu", "linear"), False),
        Workload("ln_mlp_gelu_fp8", "mlp", 8192, 4096, 16384, "bf16", "fp8_e4m3_current",
                 "layernorm", False, 1e-6, ("gelu",), True, with_grad=True),
    ]
}

TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _draw(gen: torch.Generator, shape, std: float, mean: float, dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def make_inputs(w: Workload, seed: int = 0) -> Dict[str, torch.Tensor]:
    """CPU tensors of workload ``w`` in its dtype, drawn in the fixed order.

    Keys: x, gamma, beta (layernorm only), kernel1, bias1, kernel2, bias2
    (biases only when the workload has them) for "mlp"; x, gamma, beta,
    kernel, bias for "dense"; grad when ``w.with_grad``.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    dt = TORCH_DTYPE[w.dtype]
    out: Dict[str, torch.Tensor] = {}
    out["x"] = _draw(gen, (w.rows, w.hidden), 1.0, 0.0, dt)
    out["gamma"] = _draw(gen, (w.hidden,), 0.1, 0.0 if w.zero_centered_gamma else 1.0, dt)
    if w.norm_type == "layernorm":
        out["beta"] = _draw(gen, (w.hidden,), 0.1, 0.0, dt)
    if w.kind == "dense":
        out["kernel"] = _draw(gen, (w.hidden, w.ffn), 0.02, 0.0, dt)
        if w.biases:
            out["bias"] = _draw(gen, (w.ffn,), 0.02, 0.0, dt)
    else:
        g = 2 if w.gated else 1
        out["kernel1"] = _draw(gen, (w.hidden, g * w.ffn), 0.02, 0.0, dt)
        if w.biases:
            out["bias1"] = _draw(gen, (g * w.ffn,), 0.02, 0.0, dt)
        out["kernel2"] = _draw(gen, (w.ffn, w.hidden), 0.02, 0.0, dt)
        if w.biases:
            out["bias2"] = _draw(gen, (w.hidden,), 0.02, 0.0, dt)
    if w.with_grad:
        out["grad"] = _draw(gen, (w.rows, w.ffn), 1.0, 0.0, dt)
    return out


def make_act_inputs(rows: int, cols: int, gated: bool, dtype: str = "bf16", seed: int = 0,
                    std: float = 2.0) -> Dict[str, torch.Tensor]:
    """Pre-activation ``x`` [rows, G*cols] ~ N(0, std) and ``grad`` [rows, cols] ~ N(0, 1)
    for the standalone activation forward / backward."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    dt = TORCH_DTYPE[dtype]
    g = 2 if gated else 1
    return {"x": _draw(gen, (rows, g * cols), std, 0.0, dt),
            "grad": _draw(gen, (rows, cols), 1.0, 0.0, dt)}


def to_f64(t: torch.Tensor):
    """Exact widening of a CPU tensor's values to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
