"""One rank's Ulysses share on one GPU, on the same kernels as the ring share.

Ulysses sequence parallelism ("seq_len 从 4K 推到 16K、CP=2 一开就慢了
20%：Ulysses Context Parallelism 的工程取舍全记录", section 1.2;
"超长序列并行训练技术：Ulysses与Ring-Attention详解", section 3) swaps the
sequence split for a head split with an all-to-all before attention: rank r
then holds every token of query heads [r*Hq/C, (r+1)*Hq/C) and of kv heads
[r*Hkv/C, (r+1)*Hkv/C), and its attention share is plain causal attention
over the whole sequence for those heads (C must divide Hkv).  On one GPU the
all-to-all is not needed: the rank's input is a head slice of the global
buffers, passed with the global token strides.  The share runs as
``ra_rank_forward`` with cp_size = 1 (the single, causal, diagonal block),
so it uses exactly the kernels of the ring share.  Host orchestration only.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L


class UlyssesProblem:
    def __init__(self, q_glob: torch.Tensor, k_glob: torch.Tensor, v_glob: torch.Tensor,
                 cu_global: np.ndarray, cp_size: int, scale: float = 0.0):
        hq, hkv = q_glob.shape[1], k_glob.shape[1]
        if hq % cp_size or hkv % cp_size:
            raise ValueError(f"Ulysses needs cp_size ({cp_size}) to divide the query heads ({hq}) "
                             f"and the kv heads ({hkv})")
        self.cp = cp_size
        self.hs, self.gs = hq // cp_size, hkv // cp_size
        self.dqk, self.dv = q_glob.shape[2], v_glob.shape[2]
        self.cu = np.asarray(cu_global, dtype=np.int32)
        self.T = int(self.cu[-1])
        self.cu_dev = torch.from_numpy(self.cu).to(q_glob.device)
        self.scale = scale
        self.q = [q_glob[:, r * self.hs:(r + 1) * self.hs] for r in range(cp_size)]
        self.k = [k_glob[:, r * self.gs:(r + 1) * self.gs] for r in range(cp_size)]
        self.v = [v_glob[:, r * self.gs:(r + 1) * self.gs] for r in range(cp_size)]

    def q_heads(self, r: int) -> slice:
        return slice(r * self.hs, (r + 1) * self.hs)

    def kv_heads(self, r: int) -> slice:
        return slice(r * self.gs, (r + 1) * self.gs)

    def local_desc(self, r: int, causal: bool = False) -> L.AttnDesc:
        return L.attn_desc(self.q[r], self.k[r], self.v[r], self.cu_dev, self.cu_dev, self.cu,
                           self.cu, causal=causal, scale=self.scale)

    def alloc_forward(self, out_dtype=torch.bfloat16):
        """(out, lse, workspace) of one rank; the workspace holds the float32
        partials of a KV-split share (None when the library splits nothing)."""
        dev = self.q[0].device
        out = torch.empty((self.T, self.hs, self.dv), dtype=out_dtype, device=dev)
        lse = torch.empty((self.hs, self.T), dtype=torch.float32, device=dev)
        n = L.ra_rank_forward_workspace(self.forward_desc(0, out, lse))
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
        return out, lse, ws

    def forward_desc(self, r: int, out, lse, workspace=None, events=None) -> L.RankDesc:
        return L.rank_desc(self.local_desc(r), 1, 0, [self.k[r]], [self.v[r]], out, lse,
                           workspace, 2, events)

    def forward(self, r: int, out, lse, workspace=None, events=None, stream=None):
        L.ra_rank_forward(self.forward_desc(r, out, lse, workspace, events), stream)

    def work(self, r: int):
        """(visible pairs x heads, tiles visited, tiles skipped) of rank r's share."""
        return L.ra_block_attn_work(self.local_desc(r, causal=True))
