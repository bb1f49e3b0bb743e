"""Ring-attention rank shares under other shard maps, on the same kernels.

The oh-bug page's correctness section names the placements that decide how
evenly causal work lands on the ranks: contiguous token ranges, striped
(interleaved) tokens, the zig-zag mapping, and the zig-zag applied to a
packed stream as a whole.  A ``MapProblem`` places the global Q/K/V of a
workload on the ranks with ``ra_shard_tokens`` / ``ra_gather_tokens`` and
runs a rank's share step by step: at step s the rank holds the KV block of
owner (r - s) mod C and ``ra_block_attn_fwd_segments`` computes the
rectangles ``ra_step_segments`` gives for that pair (every row sees its own
token in step 0, so step 0 writes the running result and later steps merge
into it); the fp32 result is cast to bf16 at the end.  Host orchestration
and accounting only: every step runs in libra.so's kernels.
"""
from __future__ import annotations

from typing import List

import numpy as np
import torch

from . import _lib as L


class MapProblem:
    def __init__(self, kind: str, q_glob: torch.Tensor, k_glob: torch.Tensor,
                 v_glob: torch.Tensor, cu_global: np.ndarray, cp_size: int, scale: float = 0.0):
        dev = q_glob.device
        self.kind = kind
        self.cp = cp_size
        self.cu = np.asarray(cu_global, dtype=np.int32)
        self.hq, self.dqk = q_glob.shape[1], q_glob.shape[2]
        self.hkv, self.dv = v_glob.shape[1], v_glob.shape[2]
        self.scale = scale
        self.tokens = [L.ra_shard_tokens(kind, cp_size, r, self.cu) for r in range(cp_size)]
        self.Tl = len(self.tokens[0])
        self.tokens_dev = [torch.from_numpy(t).to(dev) for t in self.tokens]
        self.q = [self._gather(q_glob, r) for r in range(cp_size)]
        self.k = [self._gather(k_glob, r) for r in range(cp_size)]
        self.v = [self._gather(v_glob, r) for r in range(cp_size)]
        self.cu_local = np.array([0, self.Tl], np.int32)
        self.cu_local_dev = torch.from_numpy(self.cu_local).to(dev)
        # rectangles of every (rank, step), host and device copies
        self.segs: List[List[np.ndarray]] = []
        self.segs_dev: List[List[torch.Tensor]] = []
        for r in range(cp_size):
            hs, ds = [], []
            for s in range(cp_size):
                g = L.ra_step_segments(kind, cp_size, r, (r - s) % cp_size, self.cu)
                hs.append(g)
                ds.append(torch.from_numpy(g if len(g) else np.zeros((1, 5), np.int32)).to(dev))
            self.segs.append(hs)
            self.segs_dev.append(ds)

    def _gather(self, glob: torch.Tensor, r: int) -> torch.Tensor:
        loc = torch.empty((self.Tl,) + tuple(glob.shape[1:]), dtype=glob.dtype, device=glob.device)
        L.ra_gather_tokens(glob, loc, self.tokens_dev[r], self.tokens[r])
        return loc

    def rows(self, r: int) -> np.ndarray:
        """Global token of each local row of rank r."""
        return self.tokens[r].astype(np.int64)

    def step_desc(self, r: int, owner: int) -> L.AttnDesc:
        return L.attn_desc(self.q[r], self.k[owner], self.v[owner], self.cu_local_dev,
                           self.cu_local_dev, self.cu_local, self.cu_local, scale=self.scale)

    def alloc_forward(self):
        dev = self.q[0].device
        out = torch.empty((self.Tl, self.hq, self.dv), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((self.hq, self.Tl), dtype=torch.float32, device=dev)
        acc = torch.empty((self.Tl, self.hq, self.dv), dtype=torch.float32, device=dev)
        return out, lse, acc

    def forward(self, r: int, out, lse, acc, events=None, stream=None):
        """Rank r's share: C rectangle launches (step 0 writes, later steps
        merge), then the bf16 cast.  events: optional 2*C timing events."""
        for s in range(self.cp):
            owner = (r - s) % self.cp
            if events is not None:
                events[2 * s].record()
            L.ra_block_attn_fwd_segments(self.step_desc(r, owner), self.segs_dev[r][s],
                                         self.segs[r][s], acc, lse, merge=s > 0, stream=stream)
            if events is not None:
                events[2 * s + 1].record()
        L.ra_cast_f32_bf16(acc, out, stream)

    def work(self, r: int):
        """Per-step (visible pairs x hq, tiles visited, tiles skipped) of rank r."""
        return [L.ra_segments_work(self.segs[r][s], self.hq) for s in range(self.cp)]
