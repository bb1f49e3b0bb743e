"""Plain float64 CPU oracle for one context-parallel rank's share of Ring Attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or
calls this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; its inputs are plain arrays (drawn by the seeded generators in
``synth``) and it uses nothing beyond NumPy.

Everything here is the written-out definition, with no tiling or fusion:
scores are materialised per head (in row blocks only to bound memory), the
mask is built from global token positions and document ids, and the merge,
the shard map and the gradients are the formulas themselves.

Sources (pages of the subject, cited by title and section):
  * "超长序列并行训练技术：Ulysses与Ring-Attention详解" (intelliparadigm),
    section 4.1 (block loop returning (out, lse) per block), section 4.2
    (the log-sum-exp merge formula and the zig-zag head/tail pairing of
    chunks), section 4.3 (backward recomputes the forward quantities),
    section 5.3 (each sequence padded separately to a multiple of
    2 x world size, padding masked).
  * "LLM Context Parallel production guide" (oh-bug), section "核心原理：
    切分 Q，流转 KV" (local Q against every KV shard, exact merge by
    per-row max and exp-sum, not averaging), section "Ring Attention" (KV
    passed round the ring until local Q has seen every block), and the
    correctness-boundary section (varlen cumulative lengths follow the same
    sequence mapping; causal imbalance; zig-zag mapping; skipping dead
    upper-triangle blocks).
  * "超长上下文训练速度翻倍秘籍" (ant-ling), section 2 "踩坑一" (the diagonal
    block is local Q x local KV under the causal mask; received history
    blocks are fully visible and use a non-causal call).
  * "seq_len 从 4K 推到 16K、CP=2 一开就慢了 20%：Ulysses Context
    Parallelism 的工程取舍全记录" (iqiancheng), section 1.1 (KV blocks move
    device 0 -> 1 -> ... -> C-1 -> 0).
  * The oh-bug correctness section on causal rank imbalance also names the
    other placements implemented in ``map_local_tokens`` (striped /
    interleaved tokens, contiguous ranges, and the zig-zag mapping).

Readings where the pages are silent or garbled are listed with each function.
Parity status: every function here is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf
ROW_BLOCK = 1024  # rows materialised at a time (memory bound only)


# ---------------------------------------------------------------------------
# Token layout: documents, global positions, zig-zag shard map
# ---------------------------------------------------------------------------

def doc_of_token(cu_seqlens: Sequence[int]) -> np.ndarray:
    """Document index of every token of a packed stream given its cumulative lengths."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    return np.repeat(np.arange(len(lens), dtype=np.int64), lens)


def zigzag_chunks(cp_size: int, rank: int) -> Tuple[int, int]:
    """Chunks held by ``rank`` when a sequence is cut into 2*cp_size chunks.

    Head/tail pairing of the intelliparadigm page, section 4.2: device i
    holds chunk i and chunk 2C-1-i (C=4: 0+7, 1+6, 2+5, 3+4).  Reading: the
    smaller chunk index comes first in the rank's local order.
    """
    if not (0 <= rank < cp_size):
        raise ValueError("rank out of range")
    return rank, 2 * cp_size - 1 - rank


def zigzag_local_tokens(cp_size: int, rank: int,
                        cu_seqlens_global: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Global token index of every local row of ``rank``, and local cu_seqlens.

    Each document is split on its own (reading of intelliparadigm section
    5.3, which pads *each* sequence to a multiple of 2 x world size, and of
    the oh-bug correctness section, which requires the varlen cumulative
    lengths to follow the same mapping): a document of length L is cut into
    2C chunks of L/(2C) tokens and the rank takes its two zig-zag chunks of
    every document, in document order.  A document whose length is not a
    multiple of 2C must be padded first (``pad_to_multiple``).
    """
    cu = np.asarray(cu_seqlens_global, dtype=np.int64)
    a, b = zigzag_chunks(cp_size, rank)
    rows: List[np.ndarray] = []
    cu_local = [0]
    for d in range(len(cu) - 1):
        g0, g1 = int(cu[d]), int(cu[d + 1])
        L = g1 - g0
        if L % (2 * cp_size):
            raise ValueError(f"document {d} length {L} not divisible by 2*C")
        c = L // (2 * cp_size)
        rows.append(np.arange(g0 + a * c, g0 + (a + 1) * c, dtype=np.int64))
        rows.append(np.arange(g0 + b * c, g0 + (b + 1) * c, dtype=np.int64))
        cu_local.append(cu_local[-1] + 2 * c)
    idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return idx, np.asarray(cu_local, dtype=np.int64)


def pad_to_multiple(length: int, cp_size: int) -> int:
    """Padding a sequence needs so it splits into 2*cp_size equal chunks.

    Reading of the garbled pad formula of intelliparadigm section 5.3: pad
    to the *next* multiple of 2 x world size, and add nothing when the
    length already divides (the printed formula would add a whole 2W).
    """
    m = 2 * cp_size
    return (-length) % m


def ring_owner(rank: int, step: int, cp_size: int) -> int:
    """Rank whose KV block ``rank`` holds at ``step``.

    KV blocks travel device 0 -> 1 -> ... -> C-1 -> 0 (iqiancheng section
    1.1), so at step s a rank holds the block that started s ranks behind.
    Step 0 is the rank's own (diagonal) block.
    """
    return (rank - step) % cp_size


# ---------------------------------------------------------------------------
# Attention over an explicit visibility rule
# ---------------------------------------------------------------------------

def _visible(q_pos, q_doc, k_pos, k_doc, causal: bool) -> np.ndarray:
    """Boolean [len(q), len(k)]: same document and (if causal) key not after query."""
    vis = q_doc[:, None] == k_doc[None, :]
    if causal:
        vis &= k_pos[None, :] <= q_pos[:, None]
    return vis


def _kv_head(h: int, hq: int, hkv: int) -> int:
    """Key/value head read by query head h: contiguous groups of hq/hkv heads.

    Reading: the pages only say grouped-query attention is supported (the
    KV-head count must divide); contiguous grouping is the plain one.
    """
    return h // (hq // hkv)


def softmax_scale(dqk: int) -> float:
    """1/sqrt(head_dim of q,k) (the only scale printed on the pages)."""
    return 1.0 / math.sqrt(dqk)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              q_pos: np.ndarray, q_doc: np.ndarray,
              k_pos: np.ndarray, k_doc: np.ndarray,
              scale: Optional[float] = None, causal: bool = True,
              return_probs: bool = False):
    """Softmax attention of every query row over its visible keys, in float64.

    q [Tq, Hq, dqk], k [Tk, Hkv, dqk], v [Tk, Hkv, dv]; positions/doc ids
    are global.  Returns out [Tq, Hq, dv] and lse [Hq, Tq] (natural log).

    Definition (the exact result the block loop of intelliparadigm section
    4.1 and the exact merge of the oh-bug page reach):
        s_ij = scale * q_i . k_j,   j in V(i)
        lse_i = m_i + ln sum_j exp(s_ij - m_i),   m_i = max_j s_ij
        out_i = sum_j exp(s_ij - lse_i) v_j
    A row with no visible key has lse = -inf and out = 0 (reading: the
    pages never meet such a row; this keeps it neutral in the merge).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, hq, dqk = q.shape
    Tk, hkv, _ = k.shape
    dv = v.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    if scale is None:
        scale = softmax_scale(dqk)
    out = np.zeros((Tq, hq, dv))
    lse = np.full((hq, Tq), NEG_INF)
    probs = np.zeros((hq, Tq, Tk)) if return_probs else None
    if Tq == 0 or Tk == 0:
        return (out, lse, probs) if return_probs else (out, lse)
    for r0 in range(0, Tq, ROW_BLOCK):
        r1 = min(Tq, r0 + ROW_BLOCK)
        vis = _visible(q_pos[r0:r1], q_doc[r0:r1], k_pos, k_doc, causal)
        any_vis = vis.any(axis=1)
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            s = scale * (q[r0:r1, h, :] @ k[:, g, :].T)
            s = np.where(vis, s, NEG_INF)
            m = np.max(s, axis=1)
            m_safe = np.where(any_vis, m, 0.0)
            e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 on masked
            z = e.sum(axis=1)
            with np.errstate(divide="ignore"):
                l = m_safe + np.log(z)               # -inf where nothing visible
            l = np.where(any_vis, l, NEG_INF)
            p = np.where(any_vis[:, None], e / np.where(z > 0, z, 1.0)[:, None], 0.0)
            out[r0:r1, h, :] = p @ v[:, g, :]
            lse[h, r0:r1] = l
            if return_probs:
                probs[h, r0:r1, :] = p
    return (out, lse, probs) if return_probs else (out, lse)


# ---------------------------------------------------------------------------
# Merge of two partial results
# ---------------------------------------------------------------------------

def lse_merge(out_a: np.ndarray, lse_a: np.ndarray,
              out_b: np.ndarray, lse_b: np.ndarray):
    """Merge two partials over disjoint key sets into the partial over their union.

    lse = log(exp(lse_a) + exp(lse_b)) (intelliparadigm section 4.2), computed
    with the larger lse factored out; out = exp(lse_a - lse) out_a +
    exp(lse_b - lse) out_b, which is the per-row max / exp-sum correction of
    the oh-bug page written in terms of lse (reading: the update rule
    itself is not printed).  (0, -inf) is the identity; two empty sides
    give (0, -inf).

    out_* [T, H, dv], lse_* [H, T].
    """
    out_a = np.asarray(out_a, dtype=np.float64)
    out_b = np.asarray(out_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    wa = np.exp(lse_a - m_safe)
    wb = np.exp(lse_b - m_safe)
    tot = wa + wb
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, tot)))
    ca = np.where(empty, 0.0, wa / np.where(empty, 1.0, tot))   # [H, T]
    cb = np.where(empty, 0.0, wb / np.where(empty, 1.0, tot))
    out = ca.T[:, :, None] * out_a + cb.T[:, :, None] * out_b
    return out, lse


# ---------------------------------------------------------------------------
# One rank's share: ring steps, per-step partials, merged result
# ---------------------------------------------------------------------------

class Layout:
    """Global token metadata for a packed stream of documents."""

    def __init__(self, cu_seqlens_global: Sequence[int]):
        self.cu = np.asarray(cu_seqlens_global, dtype=np.int64)
        self.T = int(self.cu[-1])
        self.pos = np.arange(self.T, dtype=np.int64)
        self.doc = doc_of_token(self.cu)


def rank_share(q_glob, k_glob, v_glob, cu_seqlens_global, cp_size: int,
               rank: int, scale: Optional[float] = None,
               order: Optional[Sequence[int]] = None):
    """One rank's share of ring attention, step by step, in float64.

    The rank holds its zig-zag rows of Q; at step s it holds the KV block
    owned by ``ring_owner(rank, s)`` (that owner's zig-zag rows of K and V)
    and computes the partial of its rows against those keys under the
    global document-causal rule; partials are folded with ``lse_merge`` in
    step order (or in ``order``, a permutation of the steps).

    Returns dict with 'rows' (global token of each local row), 'out' [Tl,H,dv],
    'lse' [H,Tl], and 'steps': list of (owner, out_part, lse_part).
    """
    lay = Layout(cu_seqlens_global)
    rows, _ = zigzag_local_tokens(cp_size, rank, lay.cu)
    q = np.asarray(q_glob)[rows]
    steps = []
    out_acc = None
    lse_acc = None
    seq = list(range(cp_size)) if order is None else list(order)
    for s in seq:
        owner = ring_owner(rank, s, cp_size)
        krows, _ = zigzag_local_tokens(cp_size, owner, lay.cu)
        o, l = attention(q, np.asarray(k_glob)[krows], np.asarray(v_glob)[krows],
                         lay.pos[rows], lay.doc[rows], lay.pos[krows], lay.doc[krows],
                         scale=scale, causal=True)
        steps.append((owner, o, l))
        if out_acc is None:
            out_acc, lse_acc = o, l
        else:
            out_acc, lse_acc = lse_merge(out_acc, lse_acc, o, l)
    return {"rows": rows, "out": out_acc, "lse": lse_acc, "steps": steps}


def full_attention(q_glob, k_glob, v_glob, cu_seqlens_global,
                   scale: Optional[float] = None, rows: Optional[np.ndarray] = None):
    """Un-sharded causal attention within each document (optionally for some rows only)."""
    lay = Layout(cu_seqlens_global)
    r = np.arange(lay.T) if rows is None else np.asarray(rows, dtype=np.int64)
    return attention(np.asarray(q_glob)[r], k_glob, v_glob, lay.pos[r], lay.doc[r],
                     lay.pos, lay.doc, scale=scale, causal=True)


def visible_pairs(cu_seqlens_global, cp_size: int, rank: int) -> int:
    """Number of (query, key) pairs a rank's rows can see (per query head)."""
    lay = Layout(cu_seqlens_global)
    rows, _ = zigzag_local_tokens(cp_size, rank, lay.cu)
    tot = 0
    for t in rows:
        tot += int(t - lay.cu[lay.doc[t]] + 1)
    return tot


def step_coverage(cu_seqlens_global, cp_size: int, rank: int, step: int):
    """Which local rows see any key of the step's block, and which keys are seen.

    Returns (row_mask [Tl] bool, key_mask [Tk_owner] bool, all_pairs bool)
    where all_pairs says every covered row sees every covered key of its own
    document (no causal cut inside the step).
    Used to check the integer step plan against the global rule.
    """
    lay = Layout(cu_seqlens_global)
    rows, _ = zigzag_local_tokens(cp_size, rank, lay.cu)
    owner = ring_owner(rank, step, cp_size)
    krows, _ = zigzag_local_tokens(cp_size, owner, lay.cu)
    vis = _visible(lay.pos[rows], lay.doc[rows], lay.pos[krows], lay.doc[krows], True)
    same = _visible(lay.pos[rows], lay.doc[rows], lay.pos[krows], lay.doc[krows], False)
    rm = vis.any(axis=1)
    km = vis.any(axis=0)
    ix = np.ix_(rm, km)
    return rm, km, bool(np.array_equal(vis[ix], same[ix]))


# ---------------------------------------------------------------------------
# Other shard maps (oh-bug, correctness section on causal rank imbalance)
# ---------------------------------------------------------------------------

SHARD_MAPS = ("zigzag", "zigzag_global", "striped", "contiguous")


def map_local_tokens(kind: str, cp_size: int, rank: int,
                     cu_seqlens_global: Sequence[int]) -> np.ndarray:
    """Global token of every local row of ``rank`` under a shard map.

    * ``zigzag``: the per-document zig-zag of ``zigzag_local_tokens``.
    * ``zigzag_global``: the zig-zag applied to the packed stream as if it
      were one sequence: the T tokens are cut into 2C equal chunks regardless
      of document boundaries and the rank takes chunks r and 2C-1-r.  This is
      the mapping the oh-bug page warns about for packed varlen batches
      (static balance breaks once documents differ in length).
    * ``striped``: token t of the packed stream goes to rank t mod C (the
      interleaved / striped placement the oh-bug page lists as a remedy).
    * ``contiguous``: rank r holds tokens [r T/C, (r+1) T/C), the plain split
      whose causal imbalance the oh-bug page describes.
    Every map keeps a rank's tokens in global order.  T must divide by 2C
    (zigzag_global) or C (striped, contiguous).
    """
    cu = np.asarray(cu_seqlens_global, dtype=np.int64)
    T = int(cu[-1])
    C = cp_size
    if not (0 <= rank < C):
        raise ValueError("rank out of range")
    if kind == "zigzag":
        return zigzag_local_tokens(C, rank, cu)[0]
    if kind == "zigzag_global":
        if T % (2 * C):
            raise ValueError("stream length not divisible by 2*C")
        c = T // (2 * C)
        a, b = zigzag_chunks(C, rank)
        return np.concatenate([np.arange(a * c, (a + 1) * c), np.arange(b * c, (b + 1) * c)])
    if kind == "striped":
        if T % C:
            raise ValueError("stream length not divisible by C")
        return np.arange(rank, T, C, dtype=np.int64)
    if kind == "contiguous":
        if T % C:
            raise ValueError("stream length not divisible by C")
        L = T // C
        return np.arange(rank * L, (rank + 1) * L, dtype=np.int64)
    raise ValueError(f"unknown shard map {kind}")


def rank_share_map(kind: str, q_glob, k_glob, v_glob, cu_seqlens_global, cp_size: int,
                   rank: int, scale: Optional[float] = None):
    """``rank_share`` for any shard map: the rank's rows against every owner's
    keys in ring order (owner (r - s) mod C at step s), under the global
    document-causal rule, partials folded with ``lse_merge``."""
    lay = Layout(cu_seqlens_global)
    rows = map_local_tokens(kind, cp_size, rank, lay.cu)
    q = np.asarray(q_glob)[rows]
    out_acc = lse_acc = None
    steps = []
    for s in range(cp_size):
        owner = ring_owner(rank, s, cp_size)
        krows = map_local_tokens(kind, cp_size, owner, lay.cu)
        o, l = attention(q, np.asarray(k_glob)[krows], np.asarray(v_glob)[krows],
                         lay.pos[rows], lay.doc[rows], lay.pos[krows], lay.doc[krows],
                         scale=scale, causal=True)
        steps.append((owner, o, l))
        if out_acc is None:
            out_acc, lse_acc = o, l
        else:
            out_acc, lse_acc = lse_merge(out_acc, lse_acc, o, l)
    return {"rows": rows, "out": out_acc, "lse": lse_acc, "steps": steps}


def map_visible_pairs(kind: str, cu_seqlens_global, cp_size: int, rank: int) -> int:
    """(query, key) pairs a rank's rows see under a shard map (per query head):
    every row sees the keys of its document up to itself."""
    lay = Layout(cu_seqlens_global)
    rows = map_local_tokens(kind, cp_size, rank, lay.cu)
    return int((rows - lay.cu[lay.doc[rows]] + 1).sum())


def step_visible(kind: str, cu_seqlens_global, cp_size: int, rank: int,
                 owner: int) -> np.ndarray:
    """Boolean [rank's local rows, owner's local keys]: which pairs are
    visible when ``rank`` holds ``owner``'s KV block (small inputs only)."""
    lay = Layout(cu_seqlens_global)
    rows = map_local_tokens(kind, cp_size, rank, lay.cu)
    keys = map_local_tokens(kind, cp_size, owner, lay.cu)
    return _visible(lay.pos[rows], lay.doc[rows], lay.pos[keys], lay.doc[keys], True)


# ---------------------------------------------------------------------------
# Backward (gradients recomputed from the saved lse)
# ---------------------------------------------------------------------------

def attention_bwd(q, k, v, dout, q_pos, q_doc, k_pos, k_doc,
                  scale: Optional[float] = None, causal: bool = True,
                  out: Optional[np.ndarray] = None, lse: Optional[np.ndarray] = None,
                  delta: Optional[np.ndarray] = None):
    """Gradients of L = sum(dout * out) with respect to q, k, v, in float64.

    The backward recomputes the probabilities instead of storing them
    (intelliparadigm section 4.3); written out:
        D_i  = dout_i . out_i
        P_ij = exp(s_ij - lse_i)
        dV_j = sum_i P_ij dout_i
        dS_ij = P_ij (dout_i . v_j - D_i)
        dQ_i = scale sum_j dS_ij k_j
        dK_j = scale sum_i dS_ij q_i
    Query heads sharing a kv head add their dK, dV.  ``lse`` (final, over
    all keys the row sees) and ``delta`` may be passed in to compute the
    gradient contribution of a key subset (one ring step); by default they
    come from the full forward over the given keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    Tq, hq, dqk = q.shape
    Tk, hkv, _ = k.shape
    if scale is None:
        scale = softmax_scale(dqk)
    if out is None or lse is None:
        out, lse = attention(q, k, v, q_pos, q_doc, k_pos, k_doc, scale, causal)
    if delta is None:
        delta = np.einsum("thd,thd->ht", dout, out)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, Tq, ROW_BLOCK):
        r1 = min(Tq, r0 + ROW_BLOCK)
        vis = _visible(q_pos[r0:r1], q_doc[r0:r1], k_pos, k_doc, causal)
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            s = scale * (q[r0:r1, h, :] @ k[:, g, :].T)
            l = lse[h, r0:r1]
            l_safe = np.where(np.isneginf(l), 0.0, l)
            p = np.where(vis, np.exp(s - l_safe[:, None]), 0.0)
            do = dout[r0:r1, h, :]
            dv[:, g, :] += p.T @ do
            dp = do @ v[:, g, :].T
            ds = p * (dp - delta[h, r0:r1][:, None])
            dq[r0:r1, h, :] += scale * (ds @ k[:, g, :])
            dk[:, g, :] += scale * (ds.T @ q[r0:r1, h, :])
    return dq, dk, dv


def bwd_delta(out, dout) -> np.ndarray:
    """delta[h, t] = dout[t, h, :] . out[t, h, :]."""
    return np.einsum("thd,thd->ht", np.asarray(dout, np.float64), np.asarray(out, np.float64))


# ---------------------------------------------------------------------------
# bfloat16 rounding (the stored output encoding)
# ---------------------------------------------------------------------------

def bf16_round_bits(x_f32: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round-to-nearest-even.

    The bfloat16 format keeps the top 16 bits of an IEEE binary32 value;
    rounding to nearest with ties to even adds 0x7FFF plus the lowest kept
    bit before truncating.  NaN stays a quiet NaN.
    """
    u = np.asarray(x_f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(np.asarray(x_f32, dtype=np.float32))
    r = np.where(nan, ((u >> 16) | 0x40) & 0xFFFF, r)
    return r.astype(np.uint16)
