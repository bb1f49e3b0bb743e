"""GPU parity of the backward path (recompute from the saved lse) against the fp64 oracle.

Block level: dQ, dK, dV of one block (segments, halves, causal) with the
oracle's own lse and delta as inputs.  Rank level: every simulated rank's
backward share (its dQ, and dK/dV added into the KV owner's buffers), the
concatenation compared with the un-sharded gradients.  At the 256K MLA
shape: sampled dQ rows, dK/dV of the last 256 keys, and the sum rules
sum_j dV_j = sum_i dO_i and sum_j dK_j = 0.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_lse, check_out, log, make_problem, metrics, sample_rows, to_np

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")


def _part(a, b, part):
    h = (b - a) // 2
    return (a, a + h) if part == 1 else ((a + h, b) if part == 2 else (a, b))


def block_bwd_ref(q, k, v, do, cu_q, cu_k, qp, kp, causal):
    """Oracle gradients of one block treated as the whole attention of its rows."""
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    lse = np.full((q.shape[1], q.shape[0]), -np.inf)
    out = np.zeros((q.shape[0], q.shape[1], v.shape[2]))
    for s in range(len(cu_q) - 1):
        q0, q1 = _part(cu_q[s], cu_q[s + 1], qp)
        k0, k1 = _part(cu_k[s], cu_k[s + 1], kp)
        if q1 <= q0 or k1 <= k0:
            continue
        qpos, kpos = np.arange(q1 - q0), np.arange(k1 - k0)
        z1, z2 = np.zeros_like(qpos), np.zeros_like(kpos)
        o, l = oracle.attention(q[q0:q1], k[k0:k1], v[k0:k1], qpos, z1, kpos, z2, causal=causal)
        a, b, c = oracle.attention_bwd(q[q0:q1], k[k0:k1], v[k0:k1], do[q0:q1], qpos, z1, kpos,
                                       z2, causal=causal, out=o, lse=l)
        dq[q0:q1] += a
        dk[k0:k1] += b
        dv[k0:k1] += c
        out[q0:q1] = o
        lse[:, q0:q1] = l
    return dq, dk, dv, out, lse


CASES = [
    ("ragged_causal", [333], [333], 0, 0, True, 4, 2),
    ("multi_seg_noncausal", [5, 0, 130, 64, 1], [9, 3, 200, 1, 64], 0, 0, False, 2, 2),
    ("causal_tiny_segs", [1, 2, 129, 64, 63, 300], [1, 2, 129, 64, 63, 300], 0, 0, True, 2, 1),
    ("halves_q2_kall", [2, 300, 130, 0], [2, 300, 130, 0], 2, 0, False, 4, 4),
    ("halves_qall_k1", [2, 300, 130, 256], [2, 300, 130, 256], 0, 1, False, 4, 1),
    ("empty_keys", [64, 70], [0, 5], 0, 0, False, 2, 2),
]


@pytest.mark.parametrize("split", ["0", "1"])
@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_bwd_edge_cases(case, dims, split, monkeypatch):
    name, lq, lk, qp, kp, causal, hq, hkv = case
    dqk, dv = dims
    if split == "1" and dqk != 128:
        pytest.skip("the query-split dK/dV form is built for d_qk = 128")
    monkeypatch.setenv("RA_BWD_KV_SPLIT", split)
    log(f"case {name} dims {dims} dK/dV query split {split}")
    cu_q, cu_k = synth.cu_seqlens(lq), synth.cu_seqlens(lk)
    g = torch.Generator().manual_seed(11 + len(name) + dqk)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    q = torch.randn(Tq, hq, dqk, generator=g).to(torch.bfloat16)
    k = torch.randn(Tk, hkv, dqk, generator=g).to(torch.bfloat16)
    v = torch.randn(Tk, hkv, dv, generator=g).to(torch.bfloat16)
    do = torch.randn(Tq, hq, dv, generator=g).to(torch.bfloat16)
    rq, rk, rv, ro, rl = block_bwd_ref(to_np(q), to_np(k), to_np(v), to_np(do), cu_q, cu_k,
                                       qp, kp, causal)
    delta = oracle.bwd_delta(ro, to_np(do))
    dq_d, dk_d, dv_d = (q.to(DEV), k.to(DEV), v.to(DEV))
    cuq = torch.from_numpy(cu_q).to(DEV)
    cuk = torch.from_numpy(cu_k).to(DEV)
    desc = L.attn_desc(dq_d, dk_d, dv_d, cuq, cuk, cu_q, cu_k, q_part=qp, k_part=kp,
                       causal=causal)
    gq = torch.full((Tq, hq, dqk), 0.25, device=DEV)          # accumulators are added to
    gk = torch.full((Tk, hkv, dqk), -0.5, device=DEV)
    gv = torch.full((Tk, hkv, dv), 0.125, device=DEV)
    lse_t = torch.from_numpy(np.ascontiguousarray(rl, dtype=np.float32)).to(DEV)
    delta_t = torch.from_numpy(np.ascontiguousarray(delta, dtype=np.float32)).to(DEV)
    L.ra_block_attn_bwd(desc, do.to(DEV), lse_t, delta_t, gq, gk, gv)
    torch.cuda.synchronize()
    check_out(to_np(gq) - 0.25, rq, "bf16", f"{name} dQ")
    check_out(to_np(gk) + 0.5, rk, "bf16", f"{name} dK")
    check_out(to_np(gv) - 0.125, rv, "bf16", f"{name} dV")


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
def test_block_bwd_softmax_scale_override(dims):
    """Gradients with a caller-given softmax scale (0.5 instead of 1/sqrt(d_qk)).

    A larger scale gives peakier probabilities and larger gradients (|dQ|
    reaches ~25 with unit dO).  The gradients are linear in dO, so dO is
    scaled by a power of two 2^-e (exact in bf16, as are the reference
    gradients scaled by it) chosen so the largest reference gradient is at
    most 1; the fixed bf16 bars then apply unchanged.
    """
    dqk, dv = dims
    scale = 0.5
    cu = synth.cu_seqlens([300, 129])
    g = torch.Generator().manual_seed(23 + dqk)
    T, hq, hkv = int(cu[-1]), 4, 2
    q = torch.randn(T, hq, dqk, generator=g).to(torch.bfloat16)
    k = torch.randn(T, hkv, dqk, generator=g).to(torch.bfloat16)
    v = torch.randn(T, hkv, dv, generator=g).to(torch.bfloat16)
    do = torch.randn(T, hq, dv, generator=g).to(torch.bfloat16)
    q64, k64, v64 = to_np(q), to_np(k), to_np(v)

    def ref_grads(do64):
        rq, rk, rv = np.zeros_like(q64), np.zeros_like(k64), np.zeros_like(v64)
        rl = np.zeros((hq, T))
        ro = np.zeros((T, hq, dv))
        for s0, s1 in zip(cu[:-1], cu[1:]):
            pos = np.arange(s1 - s0)
            z = np.zeros_like(pos)
            o, l = oracle.attention(q64[s0:s1], k64[s0:s1], v64[s0:s1], pos, z, pos, z,
                                    scale=scale)
            a, b, c = oracle.attention_bwd(q64[s0:s1], k64[s0:s1], v64[s0:s1], do64[s0:s1], pos,
                                           z, pos, z, scale=scale, out=o, lse=l)
            rq[s0:s1], rk[s0:s1], rv[s0:s1], ro[s0:s1], rl[:, s0:s1] = a, b, c, o, l
        return rq, rk, rv, ro, rl

    top = max(float(np.abs(x).max()) for x in ref_grads(to_np(do))[:3])
    e = max(0, int(np.ceil(np.log2(top))))
    do = (do.float() * 2.0 ** -e).to(torch.bfloat16)   # exact: a power of two
    do64 = to_np(do)
    rq, rk, rv, ro, rl = ref_grads(do64)
    log(f"  scale 0.5: dO scaled by 2^-{e} (max |grad| {top:.2f} -> "
        f"{max(float(np.abs(x).max()) for x in (rq, rk, rv)):.3f})")
    cud = torch.from_numpy(cu).to(DEV)
    desc = L.attn_desc(q.to(DEV), k.to(DEV), v.to(DEV), cud, cud, cu, cu, causal=True,
                       scale=scale)
    gq = torch.zeros((T, hq, dqk), device=DEV)
    gk = torch.zeros((T, hkv, dqk), device=DEV)
    gv = torch.zeros((T, hkv, dv), device=DEV)
    lse_t = torch.from_numpy(np.ascontiguousarray(rl, dtype=np.float32)).to(DEV)
    delta_t = torch.from_numpy(np.ascontiguousarray(oracle.bwd_delta(ro, do64),
                                                    dtype=np.float32)).to(DEV)
    L.ra_block_attn_bwd(desc, do.to(DEV), lse_t, delta_t, gq, gk, gv)
    torch.cuda.synchronize()
    for got, ref, tag in ((gq, rq, "dQ"), (gk, rk, "dK"), (gv, rv, "dV")):
        check_out(to_np(got), ref, "bf16", f"scale 0.5 {tag}")


def _run_ranks(prob, with_fwd_fuse=True):
    """Forward every rank, then backward every rank; returns dq per rank, dk/dv per owner."""
    outs, lses = [], []
    for r in range(prob.cp):
        out, lse, ws = prob.alloc_forward(torch.bfloat16, with_fwd_fuse)
        prob.forward(r, out, lse, ws, fuse_merge=with_fwd_fuse)
        outs.append(out)
        lses.append(lse)
    dqs = [torch.zeros((prob.Tl, prob.hq, prob.dqk), device=DEV) for _ in range(prob.cp)]
    dks = [torch.zeros((prob.Tl, prob.hkv, prob.dqk), device=DEV) for _ in range(prob.cp)]
    dvs = [torch.zeros((prob.Tl, prob.hkv, prob.dv), device=DEV) for _ in range(prob.cp)]
    n = L.ra_rank_backward_workspace(prob.backward_desc(0, outs[0], lses[0], dqs[0], dks, dvs, None))
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    for r in range(prob.cp):
        prob.backward(r, outs[r], lses[r], dqs[r], dks, dvs, ws)
    torch.cuda.synchronize()
    return outs, lses, dqs, dks, dvs


def _full_bwd_parity(w, dout_scale=1.0):
    log(f"workload {w.name}: S={w.seqlen} C={w.cp} hq={w.hq} hkv={w.hkv} d={w.dqk}/{w.dv}")
    prob, (q, k, v, do) = make_problem(w, with_dout=True, dout_scale=dout_scale)
    q64, k64, v64, do64 = to_np(q), to_np(k), to_np(v), to_np(do)
    cu = w.cu_global()
    lay = oracle.ref.Layout(cu)
    rq, rk, rv = oracle.attention_bwd(q64, k64, v64, do64, lay.pos, lay.doc, lay.pos, lay.doc)
    _, _, dqs, dks, dvs = _run_ranks(prob)
    gq = np.zeros_like(rq)
    gk = np.zeros_like(rk)
    gv = np.zeros_like(rv)
    for r in range(w.cp):
        rows = prob.rows(r)
        gq[rows] = to_np(dqs[r])
        gk[rows] = to_np(dks[r])
        gv[rows] = to_np(dvs[r])
    check_out(gq, rq, "bf16", "dQ")
    check_out(gk, rk, "bf16", "dK")
    check_out(gv, rv, "bf16", "dV")


@pytest.mark.parametrize("odt,ddt", [(torch.bfloat16, torch.bfloat16),
                                     (torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("T,H,dv", [(1000, 3, 128), (77, 5, 64), (33, 2, 192), (5, 1, 8),
                                    (7, 3, 12)])
def test_attn_bwd_delta_parity(T, H, dv, odt, ddt):
    """delta[h, t] = dO[t, h, :] . O[t, h, :] against the oracle's definition,
    on bf16 and float32 inputs (the bf16 pair with d_v a multiple of 8 takes
    16-byte loads, the others the per-element form), ragged sizes."""
    g = torch.Generator().manual_seed(T * 31 + dv)
    out = torch.randn(T, H, dv, generator=g).to(odt)
    do = torch.randn(T, H, dv, generator=g).to(ddt)
    delta = torch.full((H, T), float("nan"), device=DEV)
    L.ra_attn_bwd_delta(out.to(DEV), do.to(DEV), delta)
    torch.cuda.synchronize()
    ref = oracle.bwd_delta(to_np(out), to_np(do))
    scale = np.einsum("thd,thd->ht", np.abs(to_np(do)), np.abs(to_np(out)))
    err = np.abs(to_np(delta) - ref)
    assert not np.isnan(to_np(delta)).any()
    assert (err <= 1e-5 * scale + 1e-30).all(), err.max()


def test_mla_backward_reduced_full_parity():
    _full_bwd_parity(synth.reduced("mla_256k", 4096, 8))


# Forms of the rank backward: (RA_BWD_RANK_FUSED, RA_BWD_QSPLIT,
# RA_BWD_KV_SPLIT, RA_BWD_KSPLIT); "auto" leaves the choice to the library
# (rank-fused).  Rank-fused ("1"): one dK/dV
# launch over every owner's key tiles and one dQ launch walking all blocks,
# ksplit = workgroups sharing a dQ query tile (on a single sequence dealt
# over the tiles by walk length, up to 6 per tile, unless "_uniform").
# Per step ("0"): one pair of
# launches per ring step; qsplit = workgroups sharing a dK/dV key tile,
# ksplit = workgroups sharing a dQ query tile (partials in the workspace,
# added in share order); the query split over a workgroup's waves
# (KV_SPLIT=1) only runs where qsplit is 1.
BWD_SPLITS = {
    "auto": (None, None, None, None),
    "fused_ksplit2_uniform": ("1", None, None, "2", "0"),
    "fused_ksplit4_uniform": ("1", None, None, "4", "0"),
    "fused_ksplit1": ("1", None, None, "1"),
    "fused_ksplit2": ("1", None, None, "2"),
    "fused_ksplit3": ("1", None, None, "3"),
    "fused_ksplit4": ("1", None, None, "4"),
    "fused_auto": ("1", None, None, None),
    "step_auto": ("0", None, None, None),
    "qsplit1": ("0", "1", None, "1"),
    "qsplit1_waves0": ("0", "1", "0", None),
    "qsplit1_waves1": ("0", "1", "1", None),
    "qsplit3": ("0", "3", None, None),
    "qsplit4": ("0", "4", None, None),
    "ksplit2": ("0", None, None, "2"),
    "ksplit3_qsplit3": ("0", "3", None, "3"),
    "ksplit4_qsplit2": ("0", "2", None, "4"),
}


def _set_splits(monkeypatch, mode):
    fused, qs, kv, ks, var = (BWD_SPLITS[mode] + (None,))[:5]
    for name, val in (("RA_BWD_RANK_FUSED", fused), ("RA_BWD_QSPLIT", qs),
                      ("RA_BWD_KV_SPLIT", kv), ("RA_BWD_KSPLIT", ks),
                      ("RA_BWD_VAR_SPLIT", var)):
        if val is None:
            monkeypatch.delenv(name, raising=False)
        else:
            monkeypatch.setenv(name, val)


@pytest.mark.parametrize("mode", list(BWD_SPLITS))
def test_gqa_backward_reduced_full_parity(mode, monkeypatch):
    _set_splits(monkeypatch, mode)
    _full_bwd_parity(synth.reduced("gqa_32k", 4096, 8))


@pytest.mark.parametrize("mode", ["fused_ksplit3", "fused_auto", "qsplit1", "qsplit3",
                                  "ksplit4_qsplit2"])
def test_mla_backward_reduced_split_parity(mode, monkeypatch):
    _set_splits(monkeypatch, mode)
    _full_bwd_parity(synth.reduced("mla_256k", 2048, 4))


@pytest.mark.parametrize("mode", ["fused_ksplit3", "ksplit3_qsplit3"])
def test_varlen_backward_reduced_split3_parity(mode, monkeypatch):
    _set_splits(monkeypatch, mode)
    w = synth.reduced("varlen_128k", 8192, 4)
    w.doc_lengths = synth.doc_lengths_loguniform(4, 8192, 8, 2048, 8)
    _full_bwd_parity(w)


@pytest.mark.parametrize("mode", ["auto", "fused_ksplit2", "step_auto"])
def test_backward_many_documents_parity(mode, monkeypatch):
    """161 packed documents of 4..40 tokens and one of 576 (CP = 2, so
    chunks of 1..10 rows and 144): the rank-fused launches place their
    workgroups on live tiles by scanning the segments 64 at a time, so this
    crosses three scan passes, and every tile is partly masked.

    Rows of such short documents attend to a few keys, so their gradients
    reach |dQ| = 6 at the workload's dO scale (against about 1 on long
    sequences), where the bf16 rounding of the forward output alone moves
    dQ by 0.015 through delta.  dO is scaled by 2^-2, which is exact in
    bf16 and scales every gradient and its rounding error alike, so the
    fixed bars apply at unit magnitude."""
    _set_splits(monkeypatch, mode)
    w = synth.reduced("varlen_128k", 4096, 2)
    w.doc_lengths = [4 * (1 + i % 10) for i in range(160)] + [576]
    assert sum(w.doc_lengths) == 4096 and len(w.doc_lengths) > 128
    _full_bwd_parity(w, dout_scale=0.25)


def _per_document_reference(q64, k64, v64, do64, cu):
    """The oracle's forward and gradients, one document at a time (documents
    are independent, so this equals the whole-stream call)."""
    lay = oracle.ref.Layout(cu)
    ro = np.zeros(q64.shape[:2] + (v64.shape[2],))
    rl = np.zeros((q64.shape[1], q64.shape[0]))
    rq, rk, rv = np.zeros_like(q64), np.zeros_like(k64), np.zeros_like(v64)
    for d in range(len(cu) - 1):
        s = slice(int(cu[d]), int(cu[d + 1]))
        args = (lay.pos[s], lay.doc[s], lay.pos[s], lay.doc[s])
        ro[s], rl[:, s] = oracle.attention(q64[s], k64[s], v64[s], *args)
        rq[s], rk[s], rv[s] = oracle.attention_bwd(q64[s], k64[s], v64[s], do64[s], *args)
    return ro, rl, rq, rk, rv


SMALL_BWD_SHARES = [(520, 2, 2), (1000, 1, 2), (392, 4, 1), (2056, 2, 4)]


@pytest.mark.parametrize("var", ["0", "1"], ids=["uniform", "per_tile"])
@pytest.mark.parametrize("ksplit", [None, "4"], ids=["auto", "ksplit4"])
@pytest.mark.parametrize("shape", SMALL_BWD_SHARES,
                         ids=[f"S{s}_C{c}_h{h}" for s, c, h in SMALL_BWD_SHARES])
def test_small_share_dq_shares(shape, ksplit, var, monkeypatch):
    """Small single-sequence shares in the rank-fused backward with dQ key
    shares, uniform and dealt per tile (tiles whose walk is shorter than
    their shares, tiles with a single share): every gradient element."""
    S, C, H = shape
    _set_splits(monkeypatch, "auto")
    monkeypatch.setenv("RA_BWD_VAR_SPLIT", var)
    if ksplit is not None:
        monkeypatch.setenv("RA_BWD_KSPLIT", ksplit)
    _full_bwd_parity(synth.reduced("mha_8k", S, C, hq=H, hkv=H))


# Packed streams whose tile lists take each ordering of the rank-fused
# grids: heaviest-first by tile (up to 512 tiles), by segment (more tiles,
# at most 512 segments) and the plain list order (more segments).
TILE_ORDER_CASES = {
    # ping-pong forward: 602 half tiles of 300 segments (by segment); 4-wave
    # forward and dQ: 306 tiles (by tile)
    "fwd_by_segment": (2, [8] * 299 + [1704], 16),
    # 600 segments: every launch in list order
    "list_order": (2, [4] * 599 + [1700], 16),
    # one rank (cp 1), 200 documents of 384: dQ and the 4-wave forward 600
    # tiles (by segment), ping-pong forward 400 (by tile)
    "dq_by_segment": (1, [384] * 200, 2),
}


@pytest.mark.parametrize("kernel", ["4w", "pp"])
@pytest.mark.parametrize("case", list(TILE_ORDER_CASES))
def test_packed_tile_orders_parity(case, kernel, monkeypatch):
    """Every output of every rank (forward out/lse, dQ, dK, dV) against the
    oracle, per document, for each ordering of the packed grids."""
    cp, docs, heads = TILE_ORDER_CASES[case]
    _set_splits(monkeypatch, "auto")
    monkeypatch.setenv("RA_FWD_KERNEL", kernel)
    w = synth.reduced("varlen_128k", sum(docs), cp, hq=heads, hkv=heads)
    w.doc_lengths = list(docs)
    log(f"{case} kernel={kernel}: {len(docs)} documents, S={w.seqlen} C={cp} heads={heads}")
    prob, (q, k, v, do) = make_problem(w, with_dout=True, dout_scale=0.25)
    q64, k64, v64, do64 = to_np(q), to_np(k), to_np(v), to_np(do)
    ro, rl, rq, rk, rv = _per_document_reference(q64, k64, v64, do64, w.cu_global())
    outs, lses, dqs, dks, dvs = _run_ranks(prob)
    for r in range(cp):
        rows = prob.rows(r)
        check_out(to_np(outs[r]), ro[rows], "bf16", f"rank{r} out")
        check_lse(to_np(lses[r]), rl[:, rows], f"rank{r} lse")
    gq, gk, gv = np.zeros_like(rq), np.zeros_like(rk), np.zeros_like(rv)
    for r in range(cp):
        rows = prob.rows(r)
        gq[rows], gk[rows], gv[rows] = to_np(dqs[r]), to_np(dks[r]), to_np(dvs[r])
    check_out(gq, rq, "bf16", "dQ")
    check_out(gk, rk, "bf16", "dK")
    check_out(gv, rv, "bf16", "dV")


@pytest.mark.parametrize("mode", ["auto", "fused_ksplit4", "step_auto", "qsplit1",
                                  "ksplit3_qsplit3"])
def test_mha_backward_reduced_full_parity(mode, monkeypatch):
    _set_splits(monkeypatch, mode)
    _full_bwd_parity(synth.reduced("mha_8k", 2048, 4))


@pytest.mark.parametrize("mode", ["auto", "step_auto"])
def test_varlen_backward_reduced_full_parity(mode, monkeypatch):
    _set_splits(monkeypatch, mode)
    w = synth.reduced("varlen_128k", 8192, 4)
    w.doc_lengths = synth.doc_lengths_loguniform(4, 8192, 8, 2048, 8)
    _full_bwd_parity(w)


@pytest.mark.parametrize("mode", ["auto", "fused_ksplit3", "qsplit4", "ksplit3_qsplit3"])
def test_backward_is_deterministic(mode, monkeypatch):
    _set_splits(monkeypatch, mode)
    w = synth.reduced("mla_256k", 2048, 4)
    prob, _ = make_problem(w, with_dout=True)
    a = _run_ranks(prob)
    b = _run_ranks(prob)
    for x, y in zip(a[2] + a[3] + a[4], b[2] + b[3] + b[4]):
        assert torch.equal(x, y)


def test_mla_256k_backward_sampled_and_sum_rules():
    w = synth.WORKLOADS["mla_256k"]
    log(f"workload {w.name} (full size): S={w.seqlen} C={w.cp}")
    prob, (q, k, v, do) = make_problem(w, with_dout=True)
    outs, lses, dqs, dks, dvs = _run_ranks(prob)
    cu = w.cu_global()
    lay = oracle.ref.Layout(cu)
    q64, k64, v64, do64 = to_np(q), to_np(k), to_np(v), to_np(do)
    del q, k, v, do
    # sum rules over the whole sequence
    sdv = sum(to_np(x).sum(0) for x in dvs)                # [hkv, dv]
    sdo = do64.sum(0)                                       # [hq, dv] (hq == hkv here)
    rel = np.abs(sdv - sdo).max() / np.abs(sdo).max()
    log(f"  sum dV vs sum dO rel={rel:.2e}")
    assert rel <= 1e-3
    sdk = sum(to_np(x).sum(0) for x in dks)
    adk = sum(np.abs(to_np(x)).sum(0) for x in dks)
    rel = np.abs(sdk).max() / adk.max()
    log(f"  |sum dK| / sum|dK| = {rel:.2e}")
    assert rel <= 1e-3
    # sampled dQ rows of ranks 0, 15, 31
    for r in (0, 15, 31):
        loc = sample_rows(prob, r, 24, seed=7)
        rows = prob.rows(r)[loc]
        o, l = oracle.attention(q64[rows], k64, v64, lay.pos[rows], lay.doc[rows], lay.pos, lay.doc)
        a, _, _ = oracle.attention_bwd(q64[rows], k64, v64, do64[rows], lay.pos[rows],
                                       lay.doc[rows], lay.pos, lay.doc, out=o, lse=l)
        check_out(to_np(dqs[r])[loc], a, "bf16", f"rank{r} dQ rows")
    # dK, dV of the last 256 keys: only the last 256 rows (rank 0's last chunk) see them
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
