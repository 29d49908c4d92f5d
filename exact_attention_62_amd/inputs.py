"""Seeded synthetic inputs for the FlashAttention-2 forward pass.

This module only draws random Q, K, V tensors.  It holds none of the attention
arithmetic, so that both the HIP path and the fp64 CPU oracle can be fed the
same bits without sharing any code that computes the result.

The pages ("Flash Attention V2原理解读", section on the thread-block grid) only
describe workloads qualitatively: long sequences with few batches and heads
(the case the sequence-length grid axis exists for), and a toy grid with one
batch, two heads and four row blocks.  The five named workloads below stand in
for those, with the shapes and value distributions the attention problem is
usually posed on: i.i.d. normal Q, K, V, plus a ragged length and large logits
for the stress case.

Recipe (identical for every consumer):
  * one CPU ``torch.Generator`` seeded with ``1000 * index + seed``;
  * Q, K, V drawn in that order, each a float32 tensor of shape [B, H, N, d];
  * then cast to the workload dtype (bfloat16 rounds to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention problem: sizes, dtype, masks to run, distributions."""

    index: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "bf16", "fp16" or "fp32"
    causal: Tuple[bool, ...]  # the mask settings this workload is run with
    qk: Tuple[str, float]  # ("normal", sigma) for Q and K
    v: Tuple[str, float]  # ("normal", sigma) or ("uniform", half-width) for V
    about: str

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DT[self.dtype]

    def flops(self, causal: bool) -> float:
        """Metric flop count: 4*B*H*N^2*d, halved when the causal mask is on."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if causal else f


_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}

WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(0, "tiny", 1, 1, 128, 64, "fp32", (False,), ("normal", 1.0), ("normal", 1.0),
                 "tiny non-causal fp32 problem, exact mode"),
        Workload(1, "small", 2, 4, 1024, 64, "bf16", (False, True), ("normal", 1.0), ("normal", 1.0),
                 "small batched problem, both masks"),
        Workload(2, "train", 16, 16, 2048, 128, "bf16", (True,), ("normal", 1.0), ("normal", 1.0),
                 "training-shaped causal problem"),
        Workload(3, "long", 1, 16, 16384, 128, "bf16", (True, False), ("normal", 1.0), ("normal", 1.0),
                 "long sequence, few heads: exercises the sequence-length grid axis"),
        Workload(4, "ragged", 2, 16, 8191, 256, "bf16", (True,), ("normal", 4.0), ("uniform", 1.0),
                 "ragged length with logits near 100: masking and overflow stress"),
    ]
}


def _draw(gen: torch.Generator, shape, dist: Tuple[str, float]) -> torch.Tensor:
    kind, s = dist
    if kind == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * s
    if kind == "uniform":
        return (torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0) * s
    raise ValueError(f"unknown distribution {kind!r}")


def make(workload: Workload | str, seed: int = 0, *, qk_sigma: float | None = None,
         B: int | None = None, H: int | None = None, N: int | None = None,
         d: int | None = None, dtype: str | None = None, Nk: int | None = None):
    """Draw (q, k, v) on the CPU for a named workload.

    Keyword overrides change the shape, dtype or Q/K sigma while keeping the
    recipe (used for small parity cases and benchmark variants); Nk gives K
    and V a length of their own (default: N).  Returns contiguous CPU tensors.
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    Nk = N if Nk is None else Nk
    dt = _DT[dtype or w.dtype]
    qk = w.qk if qk_sigma is None else ("normal", float(qk_sigma))
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1000 * w.index + int(seed))
    q = _draw(gen, (B, H, N, d), qk).to(dt).contiguous()
    k = _draw(gen, (B, H, Nk, d), qk).to(dt).contiguous()
    v = _draw(gen, (B, H, Nk, d), w.v).to(dt).contiguous()
    return q, k, v


def make_random(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16",
                sigma: float = 1.0, Nk: int | None = None):
    """Small ad-hoc problems for parity sweeps: N(0, sigma) Q and K, N(0, 1) V.

    Q has N rows; K and V have Nk rows (default N)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(0x5EED0000 + int(seed))
    dt = _DT[dtype]
    Nk = N if Nk is None else Nk
    q = (torch.randn((B, H, N, d), generator=gen) * sigma).to(dt).contiguous()
    k = (torch.randn((B, H, Nk, d), generator=gen) * sigma).to(dt).contiguous()
    v = torch.randn((B, H, Nk, d), generator=gen).to(dt).contiguous()
    return q, k, v


def make_upstream(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16"):
    """The upstream gradient dO for backward-pass problems: N(0, 1), seeded separately from
    the inputs (generator seed 0x6D0E0000 + seed)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(0x6D0E0000 + int(seed))
    return torch.randn((B, H, N, d), generator=gen).to(_DT[dtype]).contiguous()
