"""Rank emulation on one GPU: every simulated rank's share run in turn at its real shape.

Host orchestration and accounting only.  A ``RingProblem`` places the
global packed Q/K/V of a workload on the device, shards them with the
library's zig-zag map and gather kernel into one local buffer per rank (the
memory a rank would hold), and runs ``ra_rank_forward`` /
``ra_rank_backward`` for any rank with the KV blocks of every owner (the
blocks that would arrive over the ring).  All arithmetic happens in
libra.so's kernels.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import _lib as L


class RingProblem:
    def __init__(self, q_glob: torch.Tensor, k_glob: torch.Tensor, v_glob: torch.Tensor,
                 cu_global: np.ndarray, cp_size: int, dout_glob: Optional[torch.Tensor] = None,
                 keep_global: bool = False, scale: float = 0.0):
        dev = q_glob.device
        self.cp = cp_size
        self.cu_global = np.asarray(cu_global, dtype=np.int32)
        self.T = int(self.cu_global[-1])
        self.hq, self.dqk = q_glob.shape[1], q_glob.shape[2]
        self.hkv, self.dv = v_glob.shape[1], v_glob.shape[2]
        self.dtype = q_glob.dtype
        self.scale = scale
        self.maps = [L.ra_zigzag_shard_map(cp_size, r, self.cu_global) for r in range(cp_size)]
        self.cu_local = self.maps[0][0]
        for cl, _ in self.maps:
            assert np.array_equal(cl, self.cu_local)
        self.Tl = int(self.cu_local[-1])
        self.cu_local_dev = torch.from_numpy(self.cu_local).to(dev)
        self.src_start_dev = [torch.from_numpy(ss).to(dev) for _, ss in self.maps]
        self.q: List[torch.Tensor] = []
        self.k: List[torch.Tensor] = []
        self.v: List[torch.Tensor] = []
        self.do: List[torch.Tensor] = []
        for r in range(cp_size):
            self.q.append(self.gather(q_glob, r))
            self.k.append(self.gather(k_glob, r))
            self.v.append(self.gather(v_glob, r))
            if dout_glob is not None:
                self.do.append(self.gather(dout_glob, r))
        self.glob = (q_glob, k_glob, v_glob, dout_glob) if keep_global else None

    # -- placement -----------------------------------------------------------
    def gather(self, glob: torch.Tensor, r: int) -> torch.Tensor:
        loc = torch.empty((self.Tl,) + tuple(glob.shape[1:]), dtype=glob.dtype, device=glob.device)
        L.ra_zigzag_gather(glob, loc, self.cu_local_dev, self.src_start_dev[r], self.cu_local,
                           self.maps[r][1])
        return loc

    def scatter(self, loc: torch.Tensor, glob: torch.Tensor, r: int):
        L.ra_zigzag_scatter(loc, glob, self.cu_local_dev, self.src_start_dev[r], self.cu_local,
                            self.maps[r][1])

    def rows(self, r: int) -> np.ndarray:
        """Global token of each local row of rank r."""
        cl, ss = self.maps[r]
        out = []
        for s in range(len(cl) - 1):
            c = (cl[s + 1] - cl[s]) // 2
            out.append(np.arange(ss[2 * s], ss[2 * s] + c))
            out.append(np.arange(ss[2 * s + 1], ss[2 * s + 1] + c))
        return np.concatenate(out) if out else np.zeros(0, np.int64)

    # -- descriptors -----------------------------------------------------------
    def local_desc(self, r: int) -> L.AttnDesc:
        return L.attn_desc(self.q[r], self.k[r], self.v[r], self.cu_local_dev, self.cu_local_dev,
                           self.cu_local, self.cu_local, scale=self.scale)

    def step_desc(self, r: int, owner: int, causal: bool, q_part: int, k_part: int) -> L.AttnDesc:
        return L.attn_desc(self.q[r], self.k[owner], self.v[owner], self.cu_local_dev,
                           self.cu_local_dev, self.cu_local, self.cu_local, q_part=q_part,
                           k_part=k_part, causal=causal, scale=self.scale)

    def forward_desc(self, r: int, out: torch.Tensor, lse: torch.Tensor,
                     workspace: Optional[torch.Tensor] = None, fuse_merge: int = 0,
                     events=None) -> L.RankDesc:
        return L.rank_desc(self.local_desc(r), self.cp, r, self.k, self.v, out, lse, workspace,
                           fuse_merge, events)

    def alloc_forward(self, out_dtype=torch.bfloat16, fuse_merge=0):
        dev = self.q[0].device
        out = torch.empty((self.Tl, self.hq, self.dv), dtype=out_dtype, device=dev)
        lse = torch.empty((self.hq, self.Tl), dtype=torch.float32, device=dev)
        # the split rule reads shapes only, so every rank reports the same
        # size; the max over ranks is defensive
        n = max(L.ra_rank_forward_workspace(self.forward_desc(r, out, lse, None, fuse_merge))
                for r in range(self.cp))
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        return out, lse, ws

    def forward(self, r: int, out, lse, ws, fuse_merge=0, events=None, stream=None):
        L.ra_rank_forward(self.forward_desc(r, out, lse, ws, fuse_merge, events), stream)

    def backward_desc(self, r, out, lse, dq, dk_blocks, dv_blocks, workspace, events=None):
        return L.rank_bwd_desc(self.local_desc(r), self.cp, r, self.k, self.v, out, self.do[r],
                               lse, dq, dk_blocks, dv_blocks, workspace, events)

    def backward(self, r, out, lse, dq, dk_blocks, dv_blocks, ws, events=None, stream=None):
        L.ra_rank_backward(self.backward_desc(r, out, lse, dq, dk_blocks, dv_blocks, ws, events),
                           stream)

    # -- accounting ------------------------------------------------------------
    def step_plan(self, r: int):
        """(owner, causal, q_part, k_part) per step, the plan ra_rank_forward follows."""
        plan = []
        for s in range(self.cp):
            j = (r - s) % self.cp
            if s == 0:
                plan.append((j, True, L.PART_ALL, L.PART_ALL))
            elif j < r:
                plan.append((j, False, L.PART_ALL, L.PART_FIRST_HALF))
            else:
                plan.append((j, False, L.PART_SECOND_HALF, L.PART_ALL))
        return plan

    def work(self, r: int):
        """Per-step (visible pairs x hq, tiles visited, tiles skipped) of rank r."""
        return [L.ra_block_attn_work(self.step_desc(r, j, c, qp, kp))
                for (j, c, qp, kp) in self.step_plan(r)]
