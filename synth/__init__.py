"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module only draws and lays out numbers: it holds none of the attention
arithmetic.  Both the oracle tests and the HIP path take their inputs from
here, so the two sides see bit-identical values.

Generator recipe (the same for every workload):
  * every tensor is drawn as float32 standard normals in chunks of
    ``CHUNK_TOKENS`` tokens, chunk ``i`` from a fresh ``torch.Generator``
    seeded with ``(seed * 1000 + tensor_id) * 100000 + i``;
  * tensor ids: Q=1, K=2, V=3, dO=4;
  * an optional multiplier (0.5 for the 32K grouped-query workload) is
    applied in float32 before any cast;
  * bfloat16 workloads round the float32 draw to bfloat16 with
    round-to-nearest-even (torch's cast), and both sides read those bits.

Because each chunk has its own seed, any token range can be regenerated
without drawing the whole tensor (used for row-sampled checks at 256K).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

CHUNK_TOKENS = 8192
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DO = 1, 2, 3, 4


def chunk_seed(seed: int, tensor_id: int, chunk: int) -> int:
    return (seed * 1000 + tensor_id) * 100000 + chunk


def randn_tokens(seed: int, tensor_id: int, t0: int, t1: int, heads: int,
                 dim: int, mult: float = 1.0) -> torch.Tensor:
    """float32 CPU tensor [t1 - t0, heads, dim] of the seeded stream.

    Token ``t`` of the stream is the same value whatever range it is drawn in.
    """
    if t1 <= t0:
        return torch.empty((0, heads, dim), dtype=torch.float32)
    out = torch.empty((t1 - t0, heads, dim), dtype=torch.float32)
    c0, c1 = t0 // CHUNK_TOKENS, (t1 - 1) // CHUNK_TOKENS
    for c in range(c0, c1 + 1):
        g = torch.Generator().manual_seed(chunk_seed(seed, tensor_id, c))
        blk = torch.randn((CHUNK_TOKENS, heads, dim), generator=g,
                          dtype=torch.float32)
        a = max(t0, c * CHUNK_TOKENS)
        b = min(t1, (c + 1) * CHUNK_TOKENS)
        out[a - t0:b - t0] = blk[a - c * CHUNK_TOKENS:b - c * CHUNK_TOKENS]
    if mult != 1.0:
        out.mul_(mult)
    return out


def cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Cast a float32 draw to the workload's storage dtype ('bf16'|'fp32')."""
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp32":
        return x.clone()
    raise ValueError(dtype)


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact upcast of stored values (bf16 or fp32) to a float64 array."""
    return x.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# Packed document lengths for the varlen workload
# ---------------------------------------------------------------------------

def doc_lengths_loguniform(seed: int, total: int, lo: int = 128,
                           hi: int = 16384, multiple: int = 32) -> List[int]:
    """Document lengths, log-uniform in [lo, hi], summing exactly to ``total``.

    Each length is ``exp(U(ln lo, ln hi))`` rounded to a multiple of
    ``multiple`` (so every document splits into that many equal chunks),
    clipped to [lo, hi]; lengths are appended until the sum reaches
    ``total``, then the last one is shortened so the sum is exact (it stays
    a positive multiple of ``multiple``, possibly below ``lo``) and dropped
    if it reaches zero.
    """
    assert total % multiple == 0
    rng = np.random.default_rng(seed)
    lens: List[int] = []
    acc = 0
    while acc < total:
        x = math.exp(rng.uniform(math.log(lo), math.log(hi)))
        L = int(round(x / multiple)) * multiple
        L = min(max(L, lo), hi)
        lens.append(L)
        acc += L
    over = acc - total
    lens[-1] -= over
    if lens[-1] == 0:
        lens.pop()
    assert sum(lens) == total and all(L > 0 and L % multiple == 0 for L in lens)
    return lens


def cu_seqlens(lengths) -> np.ndarray:
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out


# ---------------------------------------------------------------------------
# Workload table
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seqlen: int            # global tokens (packed for varlen)
    cp: int                # context-parallel size C (ranks emulated in turn)
    hq: int
    hkv: int
    dqk: int
    dv: int
    dtype: str             # 'bf16' | 'fp32'
    seed: int
    mult: float = 1.0      # multiplier on the N(0,1) draw
    varlen: bool = False
    backward: bool = False
    doc_lengths: Optional[List[int]] = field(default=None)

    def docs(self) -> List[int]:
        if not self.varlen:
            return [self.seqlen]
        if self.doc_lengths is None:
            self.doc_lengths = doc_lengths_loguniform(
                self.seed, self.seqlen, 128, 16384, 2 * self.cp)
        return self.doc_lengths

    def cu_global(self) -> np.ndarray:
        return cu_seqlens(self.docs())

    def q(self, t0=0, t1=None):
        return randn_tokens(self.seed, TENSOR_Q, t0, self.seqlen if t1 is None else t1,
                            self.hq, self.dqk, self.mult)

    def k(self, t0=0, t1=None):
        return randn_tokens(self.seed, TENSOR_K, t0, self.seqlen if t1 is None else t1,
                            self.hkv, self.dqk, self.mult)

    def v(self, t0=0, t1=None):
        return randn_tokens(self.seed, TENSOR_V, t0, self.seqlen if t1 is None else t1,
                            self.hkv, self.dv, self.mult)

    def do(self, t0=0, t1=None):
        return randn_tokens(self.seed, TENSOR_DO, t0, self.seqlen if t1 is None else t1,
                            self.hq, self.dv, 1.0)


WORKLOADS = {
    # 256 tokens, 1 head, d=64, fp32, CP=2
    "tiny_fp32": Workload("tiny_fp32", 256, 2, 1, 1, 64, 64, "fp32", seed=1),
    # 8K multi-head, CP=4
    "mha_8k": Workload("mha_8k", 8192, 4, 8, 8, 128, 128, "bf16", seed=2),
    # 32K grouped-query (32 q heads / 8 kv heads), CP=8, N(0,1)*0.5
    "gqa_32k": Workload("gqa_32k", 32768, 8, 32, 8, 128, 128, "bf16", seed=3,
                        mult=0.5),
    # 128K packed documents, 16 heads, CP=16
    "varlen_128k": Workload("varlen_128k", 131072, 16, 16, 16, 128, 128, "bf16",
                            seed=4, varlen=True),
    # 256K MLA-shaped (dqk=192, dv=128), 16 heads, CP=32, forward + backward
    "mla_256k": Workload("mla_256k", 262144, 32, 16, 16, 192, 128, "bf16", seed=5,
                         backward=True),
}


def reduced(name: str, seqlen: int, cp: int, **kw) -> Workload:
    """A smaller copy of a workload (same heads/dims/dtype/seed recipe)."""
    w = WORKLOADS[name]
    d = dict(w.__dict__)
    d.update(name=f"{name}@{seqlen}", seqlen=seqlen, cp=cp, doc_lengths=None)
    d.update(kw)
    return Workload(**d)
