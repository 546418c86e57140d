"""Seeded synthetic inputs for the block-scaled FP8 linear-layer path.

This module only *draws* tensors. It holds none of the quantisation or GEMM
arithmetic; both the CPU oracle (``oracle/``) and the HIP path consume the
bf16 bit patterns produced here, which is the only thing they share.

Workload shapes follow the linear layers of a ~2B dense decoder trained with
micro-batch 2 x 4096-token sequences (Puro-2B report, as summarised on the
paperlayer.ai page, appendix C "Production Training Details": sequence length
4,096, micro-batch size 2), i.e. M = 8192 tokens per GPU. Hidden 2048 and
FFN 6144 are the layer sizes of the five configurations below.

Recipe (identical for every configuration):

* numpy ``Generator(PCG64)``; seed 0; one independent child stream per tensor
  from ``SeedSequence(0).spawn(n)`` in the order the tensors are listed.
* ``standard_normal`` drawn in float32, multiplied by sigma in float32
  (sigma read as the standard deviation).
* "p% outliers x50": exactly ``round(p * numel)`` distinct flat positions,
  drawn uniformly without replacement from the same child stream after the
  normal draw, multiplied by 50 in float32.
* "SiLU-gated product": ``a * sigmoid(a) * b`` with a, b ~ N(0, 1) drawn from
  the tensor's child stream in that order, evaluated in float32.
* Finally float32 -> bf16 with round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "TensorSpec",
    "Workload",
    "WORKLOADS",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "draw_tensor",
    "generate",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, int]
    kind: str  # "normal" | "silu_gated"
    sigma: float = 1.0
    outlier_frac: float = 0.0
    outlier_mult: float = 50.0


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    tensors: Tuple[TensorSpec, ...]
    # GEMMs the workload runs: (layout, m, n, k) with D[m, n] = sum_k A[m, k] B[n, k]
    gemms: Tuple[Tuple[str, int, int, int], ...] = field(default_factory=tuple)

    def spec(self, name: str) -> TensorSpec:
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)


def draw_tensor(spec: TensorSpec, rng: np.random.Generator) -> np.ndarray:
    """Draw one tensor as bf16 bit patterns (uint16) from its own child stream."""
    rows, cols = spec.shape
    n = rows * cols
    if spec.kind == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        x *= np.float32(spec.sigma)
        if spec.outlier_frac > 0.0:
            cnt = int(round(spec.outlier_frac * n))
            pos = rng.choice(n, size=cnt, replace=False)
            x[pos] *= np.float32(spec.outlier_mult)
    elif spec.kind == "silu_gated":
        a = rng.standard_normal(n, dtype=np.float32)
        b = rng.standard_normal(n, dtype=np.float32)
        sig = np.float32(1.0) / (np.float32(1.0) + np.exp(-a, dtype=np.float32))
        x = (a * sig * b).astype(np.float32)
    else:
        raise ValueError(f"unknown tensor kind {spec.kind!r}")
    return f32_to_bf16_bits(x).reshape(rows, cols)


def generate(workload: "Workload | str", seed: int = 0, only: "List[str] | None" = None) -> Dict[str, np.ndarray]:
    """Return {tensor name: uint16 bf16 bits [rows, cols]} for a workload.

    Child streams are spawned for every listed tensor, so asking for a subset
    (``only``) yields exactly the same bits as generating the whole set.
    """
    wl = WORKLOADS[workload] if isinstance(workload, str) else workload
    children = np.random.SeedSequence(seed).spawn(len(wl.tensors))
    out: Dict[str, np.ndarray] = {}
    for spec, child in zip(wl.tensors, children):
        if only is not None and spec.name not in only:
            continue
        out[spec.name] = draw_tensor(spec, np.random.Generator(np.random.PCG64(child)))
    return out


def _normal(name, shape, sigma=1.0, outliers=0.0):
    return TensorSpec(name, shape, "normal", sigma, outliers)


M_TOK = 8192  # micro-batch 2 x 4096-token sequences

WORKLOADS: Dict[str, Workload] = {
    # tiny fprop, sized for the oracle and for several 128-tiles plus a ragged 256-tile tail
    "tiny_fprop": Workload(
        "tiny_fprop",
        "Tiny fprop 256x384x512",
        (_normal("X", (256, 512), 1.0, 0.005), _normal("W", (384, 512), 0.02)),
        (("fprop", 256, 384, 512),),
    ),
    "attn_fprop": Workload(
        "attn_fprop",
        "Attention-projection fprop 8192x2048x2048",
        (_normal("X", (M_TOK, 2048), 1.0, 0.001), _normal("W", (2048, 2048), 0.02)),
        (("fprop", M_TOK, 2048, 2048),),
    ),
    "mlp_gateup_fprop": Workload(
        "mlp_gateup_fprop",
        "Fused MLP gate+up fprop 8192x12288x2048",
        (_normal("X", (M_TOK, 2048), 1.0, 0.001), _normal("W", (12288, 2048), 0.02)),
        (("fprop", M_TOK, 12288, 2048),),
    ),
    "mlp_down_fprop_dgrad": Workload(
        "mlp_down_fprop_dgrad",
        "MLP down fprop 8192x2048x6144 + dgrad 8192x6144x2048",
        (
            TensorSpec("X", (M_TOK, 6144), "silu_gated"),
            _normal("W", (2048, 6144), 0.01),
            _normal("dY", (M_TOK, 2048), 1e-3),
        ),
        (("fprop", M_TOK, 2048, 6144), ("dgrad", M_TOK, 6144, 2048)),
    ),
    "wgrad": Workload(
        "wgrad",
        "wgrad dW[2048,6144] = dY^T X over 8192 tokens",
        (_normal("dY", (M_TOK, 2048), 1e-3), _normal("X", (M_TOK, 6144), 1.0, 0.001)),
        (("wgrad", 2048, 6144, M_TOK),),
    ),
    # One linear layer's full FP8 training pass at the gate+up shape: fprop, dgrad and wgrad.
    # X and W as in mlp_gateup_fprop; dY [8192, 12288] ~ N(0, 1e-3) like the other gradients.
    "mlp_gateup_layer_step": Workload(
        "mlp_gateup_layer_step",
        "Gate+up linear layer fprop+dgrad+wgrad, X[8192,2048] W[12288,2048] dY[8192,12288]",
        (
            _normal("X", (M_TOK, 2048), 1.0, 0.001),
            _normal("W", (12288, 2048), 0.02),
            _normal("dY", (M_TOK, 12288), 1e-3),
        ),
        (("fprop", M_TOK, 12288, 2048), ("dgrad", M_TOK, 2048, 12288), ("wgrad", 12288, 2048, M_TOK)),
    ),
}
