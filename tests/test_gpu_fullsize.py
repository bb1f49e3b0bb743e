"""Full-size parity of the paths the benchmark times, compared in full.

* 32K GQA (S=32768, CP=8, 32/8 heads, d 128): rank shares 0 and 7 on the
  default fused path (one ping-pong launch per share, bf16 output written by
  the epilogue), every row and head against the oracle's attention of the
  same global rows.
* 8K MHA (S=8192, CP=4, 8 heads, d 128) backward at full size with the
  automatic work splits, rank-fused and per step: every dQ, dK, dV element
  against the oracle's gradients.
* 32K GQA backward at full size: sampled dQ rows of three ranks, dK/dV of
  the last 256 keys in full, and the sum rules over every key.
* The 16K copy of the 256K MLA workload (S=16384, CP=32: 256-token chunks,
  16 heads, d_qk 192, d_v 128): every rank's forward and backward in full.
* The 128K packed mix (23 documents, CP=16) backward at full size: every
  gradient element of its nine shortest documents, sampled dQ rows of the
  three longest, and the sum rule of dV per document.

The comparison follows the pages' own check of a context-parallel
implementation: run the complete sequence and compare the complete outputs
and gradients ("LLM Context Parallel production guide", 第一步).  The
references are the oracle's functions, called one query head at a time on
a thread pool (gpu_util.oracle_rows / oracle_grads, pinned on the CPU in
test_reference_helpers.py).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (check_lse, check_out, log, make_problem, oracle_grads, oracle_rows,
                      sample_rows, to_np)

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")


def _forward_all(prob, ranks, fuse=2):
    outs, lses = {}, {}
    for r in ranks:
        out, lse, ws = prob.alloc_forward(torch.bfloat16, fuse)
        prob.forward(r, out, lse, ws, fuse_merge=fuse)
        outs[r], lses[r] = out, lse
    torch.cuda.synchronize()
    return outs, lses


def _backward_all(prob):
    """Forward (fused) then backward of every rank; dK/dV added into the owners."""
    outs, lses = _forward_all(prob, range(prob.cp))
    dqs = [torch.zeros((prob.Tl, prob.hq, prob.dqk), device=DEV) for _ in range(prob.cp)]
    dks = [torch.zeros((prob.Tl, prob.hkv, prob.dqk), device=DEV) for _ in range(prob.cp)]
    dvs = [torch.zeros((prob.Tl, prob.hkv, prob.dv), device=DEV) for _ in range(prob.cp)]
    n = L.ra_rank_backward_workspace(prob.backward_desc(0, outs[0], lses[0], dqs[0], dks, dvs,
                                                        None))
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    for r in range(prob.cp):
        prob.backward(r, outs[r], lses[r], dqs[r], dks, dvs, ws)
    torch.cuda.synchronize()
    return outs, lses, dqs, dks, dvs


@pytest.fixture(scope="module")
def gqa_32k():
    w = synth.WORKLOADS["gqa_32k"]
    prob, (q, k, v, do) = make_problem(w, with_dout=True)
    return w, prob, (to_np(q), to_np(k), to_np(v), to_np(do))


@pytest.mark.parametrize("rank", [0, 7])
def test_gqa_32k_rank_share_full_parity(gqa_32k, rank, monkeypatch):
    """The benchmarked path: default kernel choice, fused share, bf16 output."""
    monkeypatch.delenv("RA_FWD_KERNEL", raising=False)
    monkeypatch.delenv("RA_FWD_KV_SPLIT", raising=False)
    w, prob, (q64, k64, v64, _) = gqa_32k
    assert L.ra_forward_kernel(prob.local_desc(rank)) == "attn_fwd_pp"
    log(f"gqa_32k rank {rank}: S={w.seqlen} C={w.cp}, fused share on attn_fwd_pp")
    outs, lses = _forward_all(prob, [rank])
    rows = prob.rows(rank)
    order = np.argsort(rows)
    ro, rl = oracle_rows(q64, k64, v64, w.cu_global(), rows[order])
    ref_o = np.empty_like(ro)
    ref_l = np.empty_like(rl)
    ref_o[order], ref_l[:, order] = ro, rl
    check_out(to_np(outs[rank]), ref_o, "bf16", f"rank{rank} out (all rows)")
    check_lse(to_np(lses[rank]), ref_l, f"rank{rank} lse (all rows)")


@pytest.mark.parametrize("fused", [True, False], ids=["rank_fused", "per_step"])
def test_gqa_32k_backward_sampled_and_sum_rules(fused, gqa_32k, monkeypatch):
    """Full-size backward in both forms with their automatic splits: sampled
    dQ rows of ranks 0, 3 and 7, dK/dV of the last 256 keys (seen only by
    the last 256 rows, which rank 0 holds), and the sum rules over every
    key."""
    for v in ("RA_BWD_RANK_FUSED", "RA_BWD_QSPLIT", "RA_BWD_KSPLIT", "RA_BWD_KV_SPLIT"):
        monkeypatch.delenv(v, raising=False)
    if not fused:
        monkeypatch.setenv("RA_BWD_RANK_FUSED", "0")
    w, prob, (q64, k64, v64, do64) = gqa_32k
    log(f"gqa_32k backward (full size, {'rank-fused' if fused else 'per step'}): "
        f"S={w.seqlen} C={w.cp}")
    _, _, dqs, dks, dvs = _backward_all(prob)
    cu = w.cu_global()
    lay = oracle.ref.Layout(cu)
    grp = w.hq // w.hkv
    sdv = sum(to_np(x).sum(0) for x in dvs)                         # [hkv, dv]
    sdo = do64.sum(0).reshape(w.hkv, grp, w.dv).sum(1)              # query heads of a group
    rel = np.abs(sdv - sdo).max() / np.abs(sdo).max()
    log(f"  sum dV vs sum dO rel={rel:.2e}")
    assert rel <= 1e-3
    sdk = sum(to_np(x).sum(0) for x in dks)
    adk = sum(np.abs(to_np(x)).sum(0) for x in dks)
    rel = np.abs(sdk).max() / adk.max()
    log(f"  |sum dK| / sum|dK| = {rel:.2e}")
    assert rel <= 1e-3
    for r in (0, 3, 7):
        loc = sample_rows(prob, r, 24, seed=3)
        rows = prob.rows(r)[loc]
        o, l = oracle.attention(q64[rows], k64, v64, lay.pos[rows], lay.doc[rows], lay.pos,
                                lay.doc)
        a, _, _ = oracle.attention_bwd(q64[rows], k64, v64, do64[rows], lay.pos[rows],
                                       lay.doc[rows], lay.pos, lay.doc, out=o, lse=l)
        check_out(to_np(dqs[r])[loc], a, "bf16", f"rank{r} dQ rows")
    S = w.seqlen
    rows = np.arange(S - 256, S)
    keys = np.arange(S - 256, S)
    o, l = oracle.attention(q64[rows], k64, v64, lay.pos[rows], lay.doc[rows], lay.pos, lay.doc)
    _, rk, rv = oracle.attention_bwd(q64[rows], k64[keys], v64[keys], do64[rows], lay.pos[rows],
                                     lay.doc[rows], lay.pos[keys], lay.doc[keys], out=o, lse=l,
                                     delta=oracle.bwd_delta(o, do64[rows]))
    r0 = prob.rows(0)
    loc = np.searchsorted(r0, keys)
    assert np.array_equal(r0[loc], keys)
    check_out(to_np(dks[0])[loc], rk, "bf16", "last-256 dK")
    check_out(to_np(dvs[0])[loc], rv, "bf16", "last-256 dV")


def _concat_grads(prob, dqs, dks, dvs):
    gq = np.zeros((prob.T, prob.hq, prob.dqk))
    gk = np.zeros((prob.T, prob.hkv, prob.dqk))
    gv = np.zeros((prob.T, prob.hkv, prob.dv))
    for r in range(prob.cp):
        rows = prob.rows(r)
        gq[rows] = to_np(dqs[r])
        gk[rows] = to_np(dks[r])
        gv[rows] = to_np(dvs[r])
    return gq, gk, gv


def _full_backward(w, monkeypatch, fused=True):
    for v in ("RA_BWD_RANK_FUSED", "RA_BWD_QSPLIT", "RA_BWD_KSPLIT", "RA_BWD_KV_SPLIT"):
        monkeypatch.delenv(v, raising=False)
    if not fused:
        monkeypatch.setenv("RA_BWD_RANK_FUSED", "0")
    log(f"{w.name} backward in full: S={w.seqlen} C={w.cp} hq={w.hq} d={w.dqk}/{w.dv}")
    prob, (q, k, v, do) = make_problem(w, with_dout=True)
    q64, k64, v64, do64 = to_np(q), to_np(k), to_np(v), to_np(do)
    _, _, dqs, dks, dvs = _backward_all(prob)
    rq, rk, rv = oracle_grads(q64, k64, v64, do64, w.cu_global())
    gq, gk, gv = _concat_grads(prob, dqs, dks, dvs)
    check_out(gq, rq, "bf16", "dQ (every element)")
    check_out(gk, rk, "bf16", "dK (every element)")
    check_out(gv, rv, "bf16", "dV (every element)")


@pytest.mark.parametrize("fused", [True, False], ids=["rank_fused", "per_step"])
def test_mha_8k_backward_full_parity(fused, monkeypatch):
    """Both forms of the rank backward, with their automatic splits."""
    _full_backward(synth.WORKLOADS["mha_8k"], monkeypatch, fused)


def _mla_mini():
    return synth.reduced("mla_256k", 16384, 32)


def test_mla_16k_cp32_forward_full_parity(monkeypatch):
    """Every rank share of the 16K / CP=32 MLA copy (256-token chunks) on the
    default fused path, concatenated and compared with full attention."""
    monkeypatch.delenv("RA_FWD_KERNEL", raising=False)
    monkeypatch.delenv("RA_FWD_KV_SPLIT", raising=False)
    w = _mla_mini()
    log(f"{w.name} forward in full: S={w.seqlen} C={w.cp} hq={w.hq} d={w.dqk}/{w.dv}")
    prob, (q, k, v, _) = make_problem(w)
    q64, k64, v64 = to_np(q), to_np(k), to_np(v)
    outs, lses = _forward_all(prob, range(w.cp))
    ro, rl = oracle_rows(q64, k64, v64, w.cu_global(), np.arange(w.seqlen))
    for r in range(w.cp):
        rows = prob.rows(r)
        check_out(to_np(outs[r]), ro[rows], "bf16", f"rank{r} out")
        check_lse(to_np(lses[r]), rl[:, rows], f"rank{r} lse")


@pytest.mark.parametrize("fused", [True, False], ids=["rank_fused", "per_step"])
def test_mla_16k_cp32_backward_full_parity(fused, monkeypatch):
    _full_backward(_mla_mini(), monkeypatch, fused)


def test_varlen_128k_backward_full_size(monkeypatch):
    """The 128K packed mix (23 documents, CP = 16) backward at full size on
    the default path: every dQ, dK, dV element of the nine documents of at
    most 2048 tokens against the oracle's gradients of each document; dQ of
    sampled rows (both chunk ends and random) of the three longest
    documents; and the sum rule of dV over every document (the probabilities
    of a row sum to 1, so the dV of a document's keys sums to its dO).
    Rows of the short documents attend to few keys and reach |dQ| = 6.6 at
    the workload's dO scale, so dO is scaled by 2^-2 (exact in bf16; every
    gradient and its rounding error scale alike) to apply the fixed bars at
    unit magnitude."""
    for v in ("RA_BWD_RANK_FUSED", "RA_BWD_QSPLIT", "RA_BWD_KSPLIT", "RA_BWD_KV_SPLIT",
              "RA_BWD_VAR_SPLIT"):
        monkeypatch.delenv(v, raising=False)
    w = synth.WORKLOADS["varlen_128k"]
    log(f"varlen_128k backward (full size): S={w.seqlen} C={w.cp}")
    prob, (q, k, v, do) = make_problem(w, with_dout=True, dout_scale=0.25)
    q64, k64, v64, do64 = to_np(q), to_np(k), to_np(v), to_np(do)
    _, _, dqs, dks, dvs = _backward_all(prob)
    gq, gk, gv = _concat_grads(prob, dqs, dks, dvs)
    cu = w.cu_global()
    lens = np.diff(cu)
    for d in np.argsort(lens):
        a, b = int(cu[d]), int(cu[d + 1])
        if b - a > 2048:
            break
        rq, rk, rv = oracle_grads(q64[a:b], k64[a:b], v64[a:b], do64[a:b],
                                  np.array([0, b - a], np.int32))
        check_out(gq[a:b], rq, "bf16", f"doc {d} ({b - a} tokens) dQ")
        check_out(gk[a:b], rk, "bf16", f"doc {d} dK")
        check_out(gv[a:b], rv, "bf16", f"doc {d} dV")
    lay = oracle.ref.Layout(cu)
    rng = np.random.default_rng(7)
    for d in np.argsort(lens)[-3:]:
        a, b = int(cu[d]), int(cu[d + 1])
        c = (b - a) // (2 * w.cp)
        ends = [a, a + c - 1, a + c, b - c - 1, b - c, b - 1]
        rows = np.unique(np.concatenate([ends, rng.integers(a, b, 4)]))
        ref = np.zeros((len(rows), w.hq, w.dqk))
        for i, r in enumerate(rows):
            s = slice(a, int(r) + 1)  # the row's visible keys: its document up to itself
            ref[i] = oracle.attention_bwd(q64[r:r + 1], k64[s], v64[s], do64[r:r + 1],
                                          lay.pos[r:r + 1], lay.doc[r:r + 1], lay.pos[s],
                                          lay.doc[s])[0][0]
        check_out(gq[rows], ref, "bf16", f"doc {d} ({b - a} tokens) sampled dQ rows")
    for d in range(len(lens)):
        a, b = int(cu[d]), int(cu[d + 1])
        sdv, sdo = gv[a:b].sum(0), do64[a:b].sum(0)
        rel = np.abs(sdv - sdo).max() / np.abs(sdo).max()
        assert rel <= 1e-3, (d, rel)
