"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no part of the attention arithmetic: it only draws
N(0, 1) tensors from a seeded CPU generator, in a fixed order, and rounds them
to the requested storage dtype.  Both the GPU library and the fp64 oracle are
fed from here, so they see bit-identical inputs.

Recipe (no dataset is involved; the pages measure on none):
  * generator: ``torch.Generator('cpu').manual_seed(seed)``;
  * prefill: draw fp32 ``randn`` for Q [B,H,N,d], then K [B,Hkv,N,d], then
    V [B,Hkv,N,d]; bf16 (or fp16) workloads round each with
    round-to-nearest-even (``.to(torch.bfloat16)``), fp8 workloads likewise
    to the OCP E4M3 or E5M2 format (``torch.float8_e4m3fn`` / ``float8_e5m2``),
    and the oracle reads the rounded values;
  * decode: one generator per run, step-major: for every step draw q [B,H,d],
    then k [B,Hkv,d], then v [B,Hkv,d];
  * packed batches: sequence lengths log-uniform in [lo, hi] from their own
    seeded generator, then every sequence's q, k, v as a B = 1 prefill with
    seed + 17 * index;
  * decayed sums: the log-decay g [B,Hkv,N] (fp32) of every token is
    logsigmoid(u) / 16 with u ~ N(0,1) from its own seeded generator (a gate
    in (0, 1) close to 1: exp(g) is about 0.96 at u = 0).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
          "e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" | "bf16"
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    seed: int

    @property
    def G(self) -> int:
        return self.H // self.Hkv


# The five workloads: shapes, dtypes and seeds (seed = 1000 + index).
WORKLOADS = {
    "cfg1": Workload("causal f32 B1 H2 N256 d32", "f32", 1, 2, 2, 256, 32, 1001),
    "cfg2": Workload("causal+noncausal f32 B2 H8 N4096 d64", "f32", 2, 8, 8, 4096, 64, 1002),
    "cfg3": Workload("causal bf16 B2 H8 N16384 d64", "bf16", 2, 8, 8, 16384, 64, 1003),
    "cfg4": Workload("causal bf16 B2 H8 N65536 d64", "bf16", 2, 8, 8, 65536, 64, 1004),
    "cfg5": Workload("GQA causal bf16 B1 H32 Hkv8 N32768 d128 prefill", "bf16", 1, 32, 8, 32768, 128, 1005),
}
# Decode after the GQA prefill: batch 64, 1024 single-token steps, seed 2005.
DECODE = Workload("GQA decode bf16 batch64 H32 Hkv8 d128 x1024 steps", "bf16", 64, 32, 8, 1, 128, 2005)
DECODE_STEPS = 1024


def make_qkv(B: int, H: int, Hkv: int, N: int, d: int, dtype: str, seed: int):
    """Q [B,H,N,d], K and V [B,Hkv,N,d] on the CPU, in ``dtype`` ("f32"|"bf16")."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float32)
    t = DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def workload_qkv(w: Workload):
    return make_qkv(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed)


class DecodeStream:
    """Step-major generator of decode inputs: each ``next()`` is (q, k, v) for one step."""

    def __init__(self, B: int, H: int, Hkv: int, d: int, dtype: str, seed: int):
        self.B, self.H, self.Hkv, self.d = B, H, Hkv, d
        self.dtype = DTYPES[dtype]
        self.g = torch.Generator("cpu").manual_seed(seed)

    def next(self):
        q = torch.randn(self.B, self.H, self.d, generator=self.g, dtype=torch.float32)
        k = torch.randn(self.B, self.Hkv, self.d, generator=self.g, dtype=torch.float32)
        v = torch.randn(self.B, self.Hkv, self.d, generator=self.g, dtype=torch.float32)
        return q.to(self.dtype), k.to(self.dtype), v.to(self.dtype)


def randn(shape, seed: int, dtype: str = "f32"):
    """A single seeded N(0,1) tensor (for edge-case tests)."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(DTYPES[dtype])


# A packed batch of sequences of different lengths (head shape of cfg3):
# 64 sequences, lengths log-uniform in [128, 4096].
PACKED = dict(name="packed bf16 H8 d64, 64 sequences, lengths log-uniform 128..4096", dtype="bf16", H=8, Hkv=8, d=64,
              nseqs=64, lo=128, hi=4096, seed=3003)


def packed_lengths(nseqs: int, lo: int, hi: int, seed: int) -> list[int]:
    """Seeded sequence lengths, log-uniform in [lo, hi]."""
    g = torch.Generator("cpu").manual_seed(seed)
    u = torch.rand(nseqs, generator=g, dtype=torch.float64)
    lens = torch.exp(torch.log(torch.tensor(float(lo))) + u * (torch.log(torch.tensor(float(hi))) -
                                                               torch.log(torch.tensor(float(lo)))))
    return [int(x) for x in lens.round().clamp(lo, hi)]


def packed_qkv(p: dict = PACKED):
    """Per-sequence (q, k, v), each [1, heads, n_b, d], for the packed batch p."""
    lens = packed_lengths(p["nseqs"], p["lo"], p["hi"], p["seed"])
    return lens, [make_qkv(1, p["H"], p["Hkv"], n, p["d"], p["dtype"], p["seed"] + 17 * i) for i, n in enumerate(lens)]



def make_decay(B: int, Hkv: int, N: int, seed: int):
    """Log-decay g [B,Hkv,N] in fp32: logsigmoid(u) / 16, u ~ N(0,1) seeded (g < 0)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    u = torch.randn(B, Hkv, N, generator=gen, dtype=torch.float32)
    return torch.nn.functional.logsigmoid(u) / 16.0


# The decayed-sum workload: cfg3's shape with a per-token gate.
DECAY = Workload("decayed causal bf16 B2 H8 N16384 d64", "bf16", 2, 8, 8, 16384, 64, 1006)
