"""Seeded synthetic inputs for the routed-experts MoE decode step.

This module only draws random numbers in the shapes and distributions of the five
workloads; it holds none of the method's arithmetic (no quantization, no routing
logic, no matmuls).  Both the oracle-side tests and the GPU-side tests/benchmark use
it, so that both sides see identical inputs.

Canonical layouts of what it returns (all numpy):
  x        uint16 [B, D]       BF16 bits
  ids      int32  [B, K]       distinct expert ids per token (top-k order)
  weights  float32 [B, K]      routing weights (softmax of N(0,1) logits)
  w13      uint8  [E, 2I, D/2] two e2m1 codes per byte, low nibble = even k;
                               rows 0..I-1 gate, I..2I-1 up
  s13      uint8  [E, 2I, D/32] E8M0 bytes (127 + exponent)
  w2       uint8  [E, D, I/2]
  s2       uint8  [E, D, I/32]

Draw order per workload (torch.Generator('cpu').manual_seed(seed)):
  1. x = randn(B, D) -> bfloat16
  2. scaled rows (x30) -- only for the workloads that ask for them
  3. ids (uniform-distinct: rand(B, E).argsort(1)[:, :K];
          Zipf(s):         top-K of -s*log(1+e) + Gumbel noise, descending)
  4. routing logits randn(B, K) -> softmax
  5. w13 codes  randint(0, 16), expert by expert
  6. s13 exponents randint(lo, hi + 1)
  7. w2 codes, 8. s2 exponents.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    E: int
    K: int
    D: int
    I: int
    routing: str          # "uniform" or "zipf"
    scale_lo: int         # E8M0 exponent range of the weight scales (inclusive)
    scale_hi: int
    scaled_rows: float = 0.0   # fraction of x rows multiplied by 30 (at least one if > 0)
    zipf_s: float = 1.1
    seed: int = 1


# The five workloads: sizes, routing and scale ranges of the decode MoE layer.
WORKLOADS = {
    "tiny": Workload("tiny", B=1, E=16, K=4, D=512, I=128, routing="uniform",
                     scale_lo=-8, scale_hi=-4, seed=1),
    "decode_b1": Workload("decode_b1", B=1, E=160, K=16, D=3584, I=384, routing="uniform",
                          scale_lo=-9, scale_hi=-5, seed=2),
    "decode_b8": Workload("decode_b8", B=8, E=160, K=16, D=3584, I=384, routing="zipf",
                          scale_lo=-9, scale_hi=-5, scaled_rows=0.05, seed=3),
    "grouped_b64": Workload("grouped_b64", B=64, E=160, K=16, D=3584, I=256, routing="zipf",
                            scale_lo=-9, scale_hi=-5, seed=4),
    "wide_b256": Workload("wide_b256", B=256, E=160, K=16, D=3584, I=384, routing="uniform",
                          scale_lo=-8, scale_hi=-4, seed=5),
}
ORDER = ["tiny", "decode_b1", "decode_b8", "grouped_b64", "wide_b256"]


def custom(name="custom", *, B, E, K, D, I, routing="uniform", scale_lo=-8, scale_hi=-4,
           scaled_rows=0.0, seed=0) -> Workload:
    return Workload(name, B=B, E=E, K=K, D=D, I=I, routing=routing, scale_lo=scale_lo,
                    scale_hi=scale_hi, scaled_rows=scaled_rows, seed=seed)


def _pack_nibbles(codes: torch.Tensor) -> np.ndarray:
    c = codes.to(torch.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).numpy()


def _routing(g: torch.Generator, w: Workload) -> torch.Tensor:
    if w.routing == "uniform":
        return torch.rand(w.B, w.E, generator=g).argsort(dim=1)[:, : w.K].to(torch.int32)
    if w.routing == "zipf":
        u = torch.rand(w.B, w.E, generator=g, dtype=torch.float64).clamp_min(1e-300)
        gumbel = -torch.log(-torch.log(u))
        logits = -w.zipf_s * torch.log1p(torch.arange(w.E, dtype=torch.float64))
        return torch.topk(logits + gumbel, w.K, dim=1).indices.to(torch.int32)
    raise ValueError(w.routing)


def generate(w: Workload | str, *, with_weights: bool = True) -> dict:
    """All inputs of one workload as numpy arrays (see module docstring)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = torch.Generator("cpu").manual_seed(w.seed)
    x = torch.randn(w.B, w.D, generator=g).to(torch.bfloat16)
    if w.scaled_rows > 0:
        n = max(1, int(round(w.scaled_rows * w.B)))
        rows = torch.randperm(w.B, generator=g)[:n]
        x[rows] = (x[rows].float() * 30.0).to(torch.bfloat16)
    ids = _routing(g, w)
    logits = torch.randn(w.B, w.K, generator=g)
    weights = torch.softmax(logits, dim=1)
    out = {"workload": w, "x": x.view(torch.uint16).numpy().copy(), "ids": ids.numpy().copy(),
           "weights": weights.numpy().astype(np.float32)}
    if not with_weights:
        return out
    E, D, I = w.E, w.D, w.I
    w13 = np.empty((E, 2 * I, D // 2), np.uint8)
    for e in range(E):
        w13[e] = _pack_nibbles(torch.randint(0, 16, (2 * I, D), generator=g, dtype=torch.uint8))
    s13 = (torch.randint(w.scale_lo, w.scale_hi + 1, (E, 2 * I, D // 32), generator=g) + 127)
    w2 = np.empty((E, D, I // 2), np.uint8)
    for e in range(E):
        w2[e] = _pack_nibbles(torch.randint(0, 16, (D, I), generator=g, dtype=torch.uint8))
    s2 = (torch.randint(w.scale_lo, w.scale_hi + 1, (E, D, I // 32), generator=g) + 127)
    out.update(w13=w13, s13=s13.to(torch.uint8).numpy(), w2=w2, s2=s2.to(torch.uint8).numpy())
    return out


def expert_weight_bytes(D: int, I: int) -> int:
    """FP4 codes plus E8M0 scales of one expert's w13 and w2."""
    return 2 * I * D // 2 + 2 * I * D // 32 + D * I // 2 + D * I // 32
