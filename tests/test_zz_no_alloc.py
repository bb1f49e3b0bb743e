"""ra_rank_forward_noalloc against ra_rank_forward, through the C ABI.

The allocation-free entry point runs the same kernels with its workspace in
the library's fixed per-device scratch array.  Two calls in a row, the
second with a smaller input, must each give bit-for-bit the output of
ra_rank_forward with a caller workspace, and both must meet the fixed bf16
bars against the oracle.  A share needing more workspace than the scratch
holds is rejected before anything is queued.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_lse, check_out, log, make_problem, to_np

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")


def _both(prob, r, fuse):
    out_a, lse_a, ws = prob.alloc_forward(torch.bfloat16, fuse)
    need = L.ra_rank_forward_workspace(prob.forward_desc(r, out_a, lse_a, None, fuse))
    assert 0 < need <= L.RA_NOALLOC_SCRATCH_BYTES, need
    prob.forward(r, out_a, lse_a, ws, fuse_merge=fuse)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    # the workspace fields are ignored: pass none
    L.ra_rank_forward_noalloc(prob.forward_desc(r, out_b, lse_b, None, fuse))
    torch.cuda.synchronize()
    log(f"  rank {r} fuse_merge={fuse}: workspace {need} bytes")
    return (to_np(out_a), to_np(lse_a)), (to_np(out_b), to_np(lse_b))


def test_noalloc_matches_rank_forward_two_calls(monkeypatch):
    monkeypatch.delenv("RA_FWD_KV_SPLIT", raising=False)
    monkeypatch.delenv("RA_FWD_KERNEL", raising=False)
    # call 1: the 8K MHA share, fused and KV-split (float32 partials of 4
    # parts in the scratch, ~34 MB)
    w = synth.WORKLOADS["mha_8k"]
    prob, (q, k, v, _) = make_problem(w)
    ro, rl = oracle.full_attention(to_np(q), to_np(k), to_np(v), w.cu_global(),
                                   rows=np.sort(prob.rows(1)))
    (oa, la), (ob, lb) = _both(prob, 1, 2)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    order = np.argsort(prob.rows(1))
    check_out(ob[order], ro, "bf16", "noalloc call 1 (mha_8k rank 1, fused split)")
    check_lse(lb[:, order], rl, "noalloc call 1")
    # call 2: a smaller share, per-step partials merged by ra_lse_merge
    # (accumulator and one partial in the scratch, ~4 MB)
    w2 = synth.reduced("mha_8k", 2048, 4)
    prob2, (q2, k2, v2, _) = make_problem(w2)
    ro2, rl2 = oracle.full_attention(to_np(q2), to_np(k2), to_np(v2), w2.cu_global())
    (oa, la), (ob, lb) = _both(prob2, 2, 0)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    rows = prob2.rows(2)
    check_out(ob, ro2[rows], "bf16", "noalloc call 2 (2K MHA rank 2, per-step merge)")
    check_lse(lb, rl2[:, rows], "noalloc call 2")


def test_noalloc_rejects_shares_beyond_the_scratch():
    """The 256K MLA fused share splits in 2 parts (~135 MB of partials):
    more than the scratch holds, rejected before any launch."""
    w = synth.WORKLOADS["mla_256k"]
    cu_local, _ = L.ra_zigzag_shard_map(w.cp, 0, w.cu_global())
    z = torch.zeros((int(cu_local[-1]), w.hq, w.dqk), dtype=torch.bfloat16, device=DEV)
    zv = torch.zeros((int(cu_local[-1]), w.hkv, w.dv), dtype=torch.bfloat16, device=DEV)
    cud = torch.from_numpy(cu_local).to(DEV)
    desc = L.attn_desc(z, z, zv, cud, cud, cu_local, cu_local)
    out = torch.empty((int(cu_local[-1]), w.hq, w.dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((w.hq, int(cu_local[-1])), dtype=torch.float32, device=DEV)
    rd = L.rank_desc(desc, w.cp, 0, [z] * w.cp, [zv] * w.cp, out, lse, None, 2, None)
    assert L.ra_rank_forward_workspace(rd) > L.RA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(L.RaError) as e:
        L.ra_rank_forward_noalloc(rd)
    assert e.value.status == L.RA_ERR_INVALID_ARG
    assert "fixed scratch" in str(e.value)


def test_noalloc_under_graph_capture(monkeypatch):
    """Captured in a HIP graph (one of the callers the entry point is for),
    the allocation-free rank forward replays bit-identical to the eager
    call, with eager work on the same output buffers between replays."""
    monkeypatch.delenv("RA_FWD_KV_SPLIT", raising=False)
    monkeypatch.delenv("RA_FWD_KERNEL", raising=False)
    w = synth.WORKLOADS["mha_8k"]
    prob, _ = make_problem(w)
    outs = [prob.alloc_forward(torch.bfloat16, 2)[:2] for _ in range(prob.cp)]
    for r in range(prob.cp):
        L.ra_rank_forward_noalloc(prob.forward_desc(r, *outs[r], None, 2))
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        # torch.cuda.graph makes `side` current while it captures
        for r in range(prob.cp):
            L.ra_rank_forward_noalloc(prob.forward_desc(r, *outs[r], None, 2), side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        for o, l in outs:
            o.fill_(float("nan"))
            l.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(prob.cp):
            assert torch.equal(outs[r][0], ref[r][0]) and torch.equal(outs[r][1], ref[r][1]), \
                (i, r)
        log(f"  replay {i}: every rank bit-identical to eager")
