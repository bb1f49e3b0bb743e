"""Rank shares under HIP graph capture.

The library only enqueues kernels (and optional events) on the caller's
stream: it never allocates, copies, clears memory or synchronises.  So a
caller can capture a whole step.  Every rank's forward (whole share per
launch, and per-block launches with merges) and backward is captured once
and replayed several times, with eager work on the same buffers in between.
Each replay must equal the eager result bit for bit (the kernels are
deterministic).  Accumulators the backward adds to are cleared inside the
graph by torch's fill kernel, not by a memset node.
"""
import pytest
import torch

import synth
from gpu_util import log, make_problem

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")
REPLAYS = 3


@pytest.mark.parametrize("fuse", [2, 0])
def test_rank_forward_graph_replays(fuse):
    w = synth.reduced("gqa_32k", 4096, 8)
    log(f"forward graph, fuse_merge {fuse}: S={w.seqlen} C={w.cp}")
    prob, _ = make_problem(w)
    bufs = [prob.alloc_forward(torch.bfloat16, fuse) for _ in range(prob.cp)]
    for r in range(prob.cp):
        prob.forward(r, *bufs[r], fuse_merge=fuse)
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone()) for o, l, _ in bufs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            for r in range(prob.cp):
                prob.forward(r, *bufs[r], fuse_merge=fuse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o, l, _ in bufs:                      # eager work on the same buffers
            o.fill_(float("nan"))
            l.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(prob.cp):
            assert torch.equal(bufs[r][0], ref[r][0]), f"replay {i} rank {r} out"
            assert torch.equal(bufs[r][1], ref[r][1]), f"replay {i} rank {r} lse"
        log(f"  replay {i}: every rank bit-identical to eager")


@pytest.mark.parametrize("form", ["1", "0"], ids=["rank_fused", "per_step"])
def test_rank_backward_graph_replays(form, monkeypatch):
    monkeypatch.setenv("RA_BWD_RANK_FUSED", form)
    w = synth.reduced("mla_256k", 2048, 4)
    log(f"backward graph ({'rank-fused' if form == '1' else 'per step'}): S={w.seqlen} "
        f"C={w.cp} d={w.dqk}/{w.dv}")
    prob, _ = make_problem(w, with_dout=True)
    outs, lses = [], []
    for r in range(prob.cp):
        out, lse, ws = prob.alloc_forward(torch.bfloat16, 2)
        prob.forward(r, out, lse, ws, fuse_merge=2)
        outs.append(out)
        lses.append(lse)
    dqs = [torch.empty((prob.Tl, prob.hq, prob.dqk), device=DEV) for _ in range(prob.cp)]
    dks = [torch.empty((prob.Tl, prob.hkv, prob.dqk), device=DEV) for _ in range(prob.cp)]
    dvs = [torch.empty((prob.Tl, prob.hkv, prob.dv), device=DEV) for _ in range(prob.cp)]
    n = L.ra_rank_backward_workspace(prob.backward_desc(0, outs[0], lses[0], dqs[0], dks, dvs,
                                                        None))
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)

    def step():
        for t in dqs + dks + dvs:
            t.zero_()
        for r in range(prob.cp):
            prob.backward(r, outs[r], lses[r], dqs[r], dks, dvs, ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in dqs + dks + dvs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for t in dqs + dks + dvs:                 # eager work on the same buffers
            t.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(dqs + dks + dvs, ref):
            assert torch.equal(a, b), f"replay {i}"
        log(f"  replay {i}: dQ, dK, dV bit-identical to eager")
