"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the oracle side (tests, the CPU baseline) and the
GPU side (tests, bench) take their inputs from here, so the two paths see the
same bytes.

Workloads (shapes and value recipes follow the five configurations the
attention-forward scope names; the pages print no data of their own):

  c1  B=1  H=2         S=256    d=64   bf16  full     Q/K/V iid N(0,1)
  c2  B=4  H=16        S=2048   d=128  bf16  causal   Q/K/V iid N(0,1)
  c3  B=2  Hq=32 Hkv=8 S=8192   d=128  bf16  causal   Q/K/V iid N(0,1)  (GQA 4:1)
  c4  varlen T=16384 (lengths U[512,4096], seed 0, last truncated) H=16 d=64
      fp16 causal within each sequence
  c5  B=1  H=16        S=16384  d=128  fp8 e4m3 (inputs fp32)  full; 4 of the 128
      channels scaled x20 in Q, K and V (outlier features), optional Hadamard
  dec B=4  Hq=32 Hkv=8 Sq=1  Sk=16384  d=128  bf16  full  Q/K/V iid N(0,1): one
      new token per sequence over a long key cache (c3's head layout), the
      decode shape that split-KV serves

Recipe: torch CPU generator, ``torch.randn`` in fp32, then a round-to-nearest-even
cast to the kernel dtype.  Seeds: Q = 10*c, K = 10*c + 1, V = 10*c + 2 for
configuration c.  Varlen lengths come from ``numpy.random.default_rng(0)``; the
outlier channels from ``default_rng(5)``; Hadamard signs from a splitmix64
counter stream (see ``hadamard_signs``).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    dtype: str          # "bf16" | "fp16" | "fp8"
    causal: bool
    varlen: bool = False
    outliers: bool = False
    seed_base: int = 0  # Q seed = 10*c

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


CONFIGS = {
    "c1": Workload("c1", B=1, Hq=2, Hkv=2, Sq=256, Sk=256, d=64, dtype="bf16", causal=False, seed_base=10),
    "c2": Workload("c2", B=4, Hq=16, Hkv=16, Sq=2048, Sk=2048, d=128, dtype="bf16", causal=True, seed_base=20),
    "c3": Workload("c3", B=2, Hq=32, Hkv=8, Sq=8192, Sk=8192, d=128, dtype="bf16", causal=True, seed_base=30),
    # varlen: B = number of sequences (10 for seed 0), Sq = Sk = total tokens
    "c4": Workload("c4", B=10, Hq=16, Hkv=16, Sq=16384, Sk=16384, d=64, dtype="fp16", causal=True,
                   varlen=True, seed_base=40),
    "c5": Workload("c5", B=1, Hq=16, Hkv=16, Sq=16384, Sk=16384, d=128, dtype="fp8", causal=False,
                   outliers=True, seed_base=50),
    # decode: one query row per sequence against 16K keys
    "dec": Workload("dec", B=4, Hq=32, Hkv=8, Sq=1, Sk=16384, d=128, dtype="bf16", causal=False, seed_base=60),
    # the 8K causal GQA shape run through the fp8 path (N(0,1) inputs, no outliers)
    "c3fp8": Workload("c3fp8", B=2, Hq=32, Hkv=8, Sq=8192, Sk=8192, d=128, dtype="fp8", causal=True,
                      seed_base=35),
}

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp8": torch.float32}


def varlen_lengths(total: int = 16384, lo: int = 512, hi: int = 4096, seed: int = 0) -> List[int]:
    """Sequence lengths drawn uniformly from [lo, hi] until they reach ``total``;
    the last one is truncated so the lengths sum to ``total`` exactly."""
    rng = np.random.default_rng(seed)
    out: List[int] = []
    acc = 0
    while acc < total:
        x = int(rng.integers(lo, hi, endpoint=True))
        x = min(x, total - acc)
        out.append(x)
        acc += x
    return out


def cu_seqlens_from_lengths(lengths: List[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def outlier_channels(d: int = 128, n: int = 4, seed: int = 5) -> np.ndarray:
    return np.random.default_rng(seed).choice(d, n, replace=False)


_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """One output of the splitmix64 generator (Steele, Lea, Flood 2014) for
    counter value x (state = x * golden-gamma)."""
    z = (x * 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def hadamard_signs(n: int = 128, seed: int = 55) -> np.ndarray:
    """Random +-1 signs for the rotation: sign i is taken from the top bit of
    splitmix64(seed * 2**32 + i + 1).  A counter stream, so any implementation
    of splitmix64 reproduces it."""
    out = np.empty(n, dtype=np.float32)
    for i in range(n):
        out[i] = -1.0 if (splitmix64((seed << 32) + i + 1) >> 63) else 1.0
    return out


def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def make_inputs(w: Workload, seed_base: Optional[int] = None, S_override: Optional[int] = None):
    """Return dict with CPU tensors q, k, v in the kernel's input dtype
    (bf16/fp16; fp32 for the fp8 path), plus cu_seqlens (int32 numpy) or None.

    Dense layout BSHD: q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d].
    Varlen layout THD: q [T, Hq, d], k/v [T, Hkv, d].
    """
    sb = w.seed_base if seed_base is None else seed_base
    Sq = w.Sq if S_override is None else S_override
    Sk = w.Sk if S_override is None else S_override
    if w.varlen:
        lengths = varlen_lengths(total=Sq)
        cu = cu_seqlens_from_lengths(lengths)
        qs = (Sq, w.Hq, w.d)
        ks = (Sk, w.Hkv, w.d)
    else:
        cu = None
        qs = (w.B, Sq, w.Hq, w.d)
        ks = (w.B, Sk, w.Hkv, w.d)
    q = _randn(qs, sb)
    k = _randn(ks, sb + 1)
    v = _randn(ks, sb + 2)
    if w.outliers:
        ch = torch.from_numpy(outlier_channels(w.d)).long()
        for t in (q, k, v):
            t[..., ch] *= 20.0
    dt = TORCH_DTYPES[w.dtype]
    return {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "cu_seqlens": cu}


def make_dense(B, Sq, Sk, Hq, Hkv, d, dtype="bf16", seed=1234, outliers=False):
    """Small ad-hoc dense inputs for tests (same recipe as ``make_inputs``)."""
    q = _randn((B, Sq, Hq, d), seed)
    k = _randn((B, Sk, Hkv, d), seed + 1)
    v = _randn((B, Sk, Hkv, d), seed + 2)
    if outliers:
        ch = torch.from_numpy(outlier_channels(d, n=min(4, d))).long()
        for t in (q, k, v):
            t[..., ch] *= 20.0
    dt = TORCH_DTYPES[dtype]
    return q.to(dt), k.to(dt), v.to(dt)


def make_varlen(lengths, Hq, Hkv, d, dtype="fp16", seed=4321):
    T = int(sum(lengths))
    q = _randn((T, Hq, d), seed)
    k = _randn((T, Hkv, d), seed + 1)
    v = _randn((T, Hkv, d), seed + 2)
    dt = TORCH_DTYPES[dtype]
    return q.to(dt), k.to(dt), v.to(dt), cu_seqlens_from_lengths(list(lengths))


# ---------------------------------------------------------------- work counts
# (bookkeeping for throughput figures: how many (query, key) pairs a
# workload's mask leaves; no attention arithmetic)
def unmasked_pairs(Sq: int, Sk: int, causal: bool) -> int:
    """(query, key) pairs a row-major mask leaves: all of them, or with the
    causal mask (key j hidden from query i when j > i) the lower triangle."""
    if not causal:
        return Sq * Sk
    n = min(Sq, Sk)
    return n * (n + 1) // 2 + max(0, Sq - Sk) * Sk


def forward_flops(w: Workload, lengths: Optional[List[int]] = None) -> float:
    """Algorithmic FLOP of one forward over workload w: 4 d per unmasked pair
    (two GEMMs, a multiply and an add each)."""
    if w.varlen:
        lengths = varlen_lengths(total=w.Sq) if lengths is None else lengths
        return 4.0 * w.d * w.Hq * sum(unmasked_pairs(n, n, w.causal) for n in lengths)
    return 4.0 * w.d * w.B * w.Hq * unmasked_pairs(w.Sq, w.Sk, w.causal)


def backward_flops(w: Workload, lengths: Optional[List[int]] = None) -> float:
    """Algorithmic FLOP of one backward: five GEMMs of 2 d per unmasked pair."""
    return 2.5 * forward_flops(w, lengths)


def dense_convention_flops(w: Workload) -> Optional[float]:
    """The 4 B H N^2 D count that also counts masked pairs (dense only)."""
    return None if w.varlen else 4.0 * w.B * w.Hq * w.Sq * w.Sk * w.d
