"""Seeded synthetic inputs for the causal GQA attention path.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
bench and the smoke check. It holds only shapes and random-number draws: no
attention arithmetic lives here, so neither side can borrow the other's math
through it.

Shapes follow the GPT-2-small configuration printed on the NanoEuler blog page
("Build and Run": 12 query heads, 4 KV heads, hidden size 768, sequence 1024,
batch 8), plus a tiny fp32 case, the MHA variant of the same shape, a long
context case and a wide-head stress case with peaked softmax.

Recipe (identical for every consumer):
  * one ``torch.Generator('cpu')`` seeded with ``seed``;
  * draw, in this order, Q [B,Hq,N,d], K [B,Hkv,N,d], V [B,Hkv,N,d],
    dO [B,Hq,N,d], each ``torch.randn(..., dtype=float32)``;
  * multiply Q and K by ``qk_std`` (3.0 for the stress case, else 1.0);
  * round to the config dtype with round-to-nearest-even (torch ``.to``).
The oracle receives exactly these rounded values, widened to float64.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict

import torch


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16": the arithmetic type of the inputs
    seed: int
    qk_std: float = 1.0
    causal: int = 1

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(d), rounded to float32 once; every consumer uses
        # this same float32 value (the oracle widens it to float64 exactly).
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    def flops_fwd(self) -> float:
        """Causal forward flops, N^2/2 visible pairs x 4d (two contractions)."""
        pairs = self.N * self.N / 2 if self.causal else self.N * self.N
        return 4.0 * self.d * pairs * self.B * self.Hq

    def flops_bwd(self) -> float:
        """Backward flops: five contractions (S recompute, dV, dP, dK, dQ)."""
        return 2.5 * self.flops_fwd()


# The five named workloads. Seeds are 1000 + position (1-based).
CONFIGS: Dict[str, Shape] = {
    "tiny_f32":   Shape("tiny_f32",   1, 2, 1, 64, 16, "f32", 1001),
    "gpt2_mha":   Shape("gpt2_mha",   8, 12, 12, 1024, 64, "bf16", 1002),
    "gpt2_gqa":   Shape("gpt2_gqa",   8, 12, 4, 1024, 64, "bf16", 1003),
    "long_gqa":   Shape("long_gqa",   2, 12, 4, 4096, 64, "bf16", 1004),
    "wide_d128":  Shape("wide_d128",  4, 16, 4, 8192, 128, "bf16", 1005, qk_std=3.0),
}

# The workload the throughput figure is quoted on.
HEADLINE = "gpt2_gqa"


def make_shape(B, Hq, Hkv, N, d, dtype="bf16", seed=7, qk_std=1.0, causal=1, name="adhoc") -> Shape:
    return Shape(name, B, Hq, Hkv, N, d, dtype, seed, qk_std, causal)


def make_inputs(s: Shape, seed: int | None = None):
    """Return (q, k, v, dO) as CPU tensors in the shape's dtype."""
    g = torch.Generator("cpu")
    g.manual_seed(s.seed if seed is None else seed)
    q = torch.randn((s.B, s.Hq, s.N, s.d), generator=g, dtype=torch.float32)
    k = torch.randn((s.B, s.Hkv, s.N, s.d), generator=g, dtype=torch.float32)
    v = torch.randn((s.B, s.Hkv, s.N, s.d), generator=g, dtype=torch.float32)
    do = torch.randn((s.B, s.Hq, s.N, s.d), generator=g, dtype=torch.float32)
    if s.qk_std != 1.0:
        q = q * s.qk_std
        k = k * s.qk_std
    dt = s.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt), do.to(dt)


# ---------------------------------------------------------------- decode
# Few-query attention over a cache: Nq new query rows (the last Nq positions)
# against Nk cached keys and values. Recipe: one generator seeded with
# ``seed``; draw Q [B,Hq,Nq,d], K [B,Hkv,Nk,d], V [B,Hkv,Nk,d] in that order,
# each torch.randn float32; multiply Q and K by qk_std; round to the dtype.
@dataclasses.dataclass(frozen=True)
class DecodeShape:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    seed: int
    qk_std: float = 1.0
    causal: int = 1

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    def min_bytes(self, out_bytes: int = 4) -> int:
        """HBM bytes a decode step must move: K and V once, Q, O and LSE."""
        el = 2 if self.dtype == "bf16" else 4
        kv = 2 * self.B * self.Hkv * self.Nk * self.d * el
        qo = self.B * self.Hq * self.Nq * self.d * (el + out_bytes)
        return kv + qo + self.B * self.Hq * self.Nq * 4


# Decode steps of the two model shapes: the GPT-2-small GQA heads at the
# pages' context length, and the wide-head shape at its full 8192-token context.
DECODE_CONFIGS: Dict[str, DecodeShape] = {
    "decode_gpt2_gqa": DecodeShape("decode_gpt2_gqa", 8, 12, 4, 1, 1024, 64, "bf16", 2001),
    "decode_wide_d128": DecodeShape("decode_wide_d128", 4, 16, 4, 1, 8192, 128, "bf16", 2002),
    # a serving batch of 64 sequences on the GPT-2-small GQA shape
    "decode_gpt2_gqa_b64": DecodeShape("decode_gpt2_gqa_b64", 64, 12, 4, 1, 1024, 64, "bf16", 2003),
}


def make_decode_shape(B, Hq, Hkv, Nq, Nk, d, dtype="bf16", seed=7, qk_std=1.0, causal=1,
                      name="adhoc_decode") -> DecodeShape:
    return DecodeShape(name, B, Hq, Hkv, Nq, Nk, d, dtype, seed, qk_std, causal)


def make_decode_inputs(s: DecodeShape, seed: int | None = None):
    """Return (q, k, v) as CPU tensors in the shape's dtype."""
    g = torch.Generator("cpu")
    g.manual_seed(s.seed if seed is None else seed)
    q = torch.randn((s.B, s.Hq, s.Nq, s.d), generator=g, dtype=torch.float32)
    k = torch.randn((s.B, s.Hkv, s.Nk, s.d), generator=g, dtype=torch.float32)
    v = torch.randn((s.B, s.Hkv, s.Nk, s.d), generator=g, dtype=torch.float32)
    if s.qk_std != 1.0:
        q = q * s.qk_std
        k = k * s.qk_std
    dt = s.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


# ---------------------------------------------------------------- rotary tables
def rope_tables(N: int, d: int, base: float = 10000.0):
    """Rotary tables cos/sin [N, d/2] of n * base^(-2i/d), computed in float64 and
    rounded once to float32 (CPU tensors). The GPU path receives them as they are;
    the oracle receives the same float32 values widened to float64."""
    n = torch.arange(N, dtype=torch.float64)[:, None]
    inv = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = n * inv[None, :]
    return torch.cos(ang).float().contiguous(), torch.sin(ang).float().contiguous()
