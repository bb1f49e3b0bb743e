"""GPU parity of one rank's Ulysses share against the fp64 oracle.

After the all-to-all of Ulysses sequence parallelism a rank holds every
token of Hq/C query heads and Hkv/C kv heads; its share is causal
attention over the whole sequence for those heads ("seq_len 从 4K 推到
16K、CP=2 一开就慢了 20%：Ulysses Context Parallelism 的工程取舍全记录",
section 1.2).  It runs as ra_rank_forward with cp_size = 1 over
a head slice of the global buffers, i.e. on the ring share's kernels.  The
oracle's full attention restricted to the rank's heads is the reference.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_lse, check_out, global_inputs, log, to_np

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402
from context_blockwise_softmax_ra_amd.ulysses import UlyssesProblem  # noqa: E402

DEV = torch.device("cuda:0")


def _problem(w):
    q, k, v, _ = global_inputs(w)
    return UlyssesProblem(q.to(DEV), k.to(DEV), v.to(DEV), w.cu_global(), w.cp), (q, k, v)


def _run(prob, r, kernel=None):
    old = os.environ.get("RA_FWD_KERNEL")
    if kernel:
        os.environ["RA_FWD_KERNEL"] = kernel
    try:
        out, lse, ws = prob.alloc_forward()
        prob.forward(r, out, lse, ws)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("RA_FWD_KERNEL", None)
        else:
            os.environ["RA_FWD_KERNEL"] = old
    return to_np(out), to_np(lse)


@pytest.mark.parametrize("kernel", ["4w", "pp"])
@pytest.mark.parametrize("name,seqlen,cp", [("gqa_32k", 4096, 8), ("mha_8k", 2048, 4),
                                             ("varlen_128k", 8192, 4)])
def test_ulysses_share_reduced_full_parity(name, seqlen, cp, kernel):
    w = synth.reduced(name, seqlen, cp)
    if name == "varlen_128k":
        w.doc_lengths = synth.doc_lengths_loguniform(4, seqlen, 8, 2048, 8)
    log(f"ulysses {w.name}: S={w.seqlen} C={w.cp} hq={w.hq} hkv={w.hkv} kernel={kernel}")
    prob, (q, k, v) = _problem(w)
    q64, k64, v64 = to_np(q), to_np(k), to_np(v)
    cu = w.cu_global()
    for r in range(w.cp):
        qs, ks = prob.q_heads(r), prob.kv_heads(r)
        ro, rl = oracle.full_attention(q64[:, qs], k64[:, ks], v64[:, ks], cu)
        out, lse = _run(prob, r, kernel)
        check_out(out, ro, w.dtype, f"rank{r}")
        check_lse(lse, rl, f"rank{r}")


def test_ulysses_share_full_size_sampled():
    w = synth.WORKLOADS["gqa_32k"]
    prob, (q, k, v) = _problem(w)
    q64, k64, v64 = to_np(q), to_np(k), to_np(v)
    del q, k, v
    cu = w.cu_global()
    rng = np.random.default_rng(11)
    rows = np.sort(np.concatenate([rng.choice(w.seqlen, 30, replace=False), [0, w.seqlen - 1]]))
    for r in (0, 5):
        qs, ks = prob.q_heads(r), prob.kv_heads(r)
        ro, rl = oracle.full_attention(q64[:, qs], k64[:, ks], v64[:, ks], cu, rows=rows)
        out, lse = _run(prob, r)
        check_out(out[rows], ro, w.dtype, f"rank{r}")
        check_lse(lse[:, rows], rl, f"rank{r}")


def test_ulysses_and_ring_shares_do_equal_work():
    """Per-rank visible pairs x heads: Ulysses and zig-zag ring both give S(S+1)/2 x Hq / C."""
    from context_blockwise_softmax_ra_amd.ring import RingProblem
    for name in ("mha_8k", "gqa_32k", "varlen_128k"):
        w = synth.WORKLOADS[name]
        z = torch.zeros((w.seqlen, w.hq, 64), dtype=torch.bfloat16, device=DEV)
        zk = torch.zeros((w.seqlen, w.hkv, 64), dtype=torch.bfloat16, device=DEV)
        uly = UlyssesProblem(z, zk, zk, w.cu_global(), w.cp)
        ring = RingProblem(z, zk, zk, w.cu_global(), w.cp)
        for r in (0, w.cp - 1):
            u_pairs = uly.work(r)[0]
            r_pairs = sum(p for p, _, _ in ring.work(r))
            assert u_pairs == r_pairs, (name, r, u_pairs, r_pairs)
            assert u_pairs == oracle.visible_pairs(w.cu_global(), w.cp, r) * w.hq


def test_ulysses_rejects_head_counts_not_divisible():
    w = synth.WORKLOADS["mla_256k"]   # 16 kv heads, C = 32
    z = torch.zeros((64, w.hq, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        UlyssesProblem(z, z, z, np.array([0, 64], np.int32), w.cp)


@pytest.mark.parametrize("lengths", [[513, 300, 7], [1023, 1, 256, 511]])
def test_ulysses_share_odd_lengths_with_half_tiles(lengths, monkeypatch):
    """A cp_size = 1 share may hold odd-length documents.  With half tiles
    forced on the ping-pong kernel, a document's second chunk has one row
    more than its first (len - len/2); e.g. 513 = 256 + 257 needs 1 + 2
    tiles.  Every row must be written and match the oracle."""
    monkeypatch.setenv("RA_FWD_KERNEL", "pp")
    monkeypatch.setenv("RA_FWD_HALF_TILES", "1")
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    g = torch.Generator().manual_seed(sum(lengths))
    q = torch.randn(T, 4, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(T, 2, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(T, 2, 128, generator=g).to(torch.bfloat16)
    prob = UlyssesProblem(q.to(DEV), k.to(DEV), v.to(DEV), cu, 1)
    out, lse, ws = prob.alloc_forward()
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    prob.forward(0, out, lse, ws)
    torch.cuda.synchronize()
    ro, rl = oracle.full_attention(to_np(q), to_np(k), to_np(v), cu)
    check_out(to_np(out), ro, "bf16", f"odd lengths {lengths}")
    check_lse(to_np(lse), rl, f"odd lengths {lengths}")
