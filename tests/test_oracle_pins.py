"""Pins for the fp64 oracle: each check comes from something other than the oracle.

  * brute force: scalar loops with math.fsum on tiny inputs;
  * closed forms (zero queries, a single visible key, constant values,
    scaling of V, shift of K);
  * a library special case: torch's float64 CPU scaled_dot_product_attention
    (the routine the oh-bug page uses to validate CP attention) with
    torch.logsumexp for lse and autograd for gradients;
  * invariants the pages fix: concatenating the un-zig-zagged rank outputs
    gives full causal attention, merge order does not matter, a merged key
    split equals attention on the union, (0, -inf) is the merge identity;
  * the zig-zag map printed on the intelliparadigm page (section 4.2);
  * central finite differences for the backward;
  * planted mistakes in the oracle must fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ref
import synth

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

def brute_attention(q, k, v, q_pos, q_doc, k_pos, k_doc, causal=True, scale=None):
    """Scalar loops with exactly rounded sums (math.fsum)."""
    Tq, hq, d = q.shape
    Tk, hkv, dv = v.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grp = hq // hkv
    out = np.zeros((Tq, hq, dv))
    lse = np.full((hq, Tq), -np.inf)
    for h in range(hq):
        g = h // grp
        for i in range(Tq):
            js = [j for j in range(Tk)
                  if k_doc[j] == q_doc[i] and (not causal or k_pos[j] <= q_pos[i])]
            if not js:
                continue
            s = [scale * math.fsum(q[i, h, x] * k[j, g, x] for x in range(d)) for j in js]
            m = max(s)
            z = math.fsum(math.exp(si - m) for si in s)
            L = m + math.log(z)
            lse[h, i] = L
            for c in range(dv):
                out[i, h, c] = math.fsum(math.exp(si - L) * v[j, g, c] for si, j in zip(s, js))
    return out, lse


def _layout(lengths):
    cu = synth.cu_seqlens(lengths)
    lay = ref.Layout(cu)
    return cu, lay


@pytest.mark.parametrize("lengths,hq,hkv,d,dv,causal", [
    ([12], 1, 1, 4, 3, True),
    ([7, 9, 4], 4, 2, 5, 6, True),
    ([10, 6], 3, 1, 3, 2, True),        # MQA
    ([8, 8], 2, 2, 4, 4, False),        # non-causal within documents
    ([1, 5, 1], 2, 1, 2, 3, True),      # one-token documents
])
def test_attention_vs_brute_force(lengths, hq, hkv, d, dv, causal):
    cu, lay = _layout(lengths)
    T = lay.T
    q, k, v = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv)
    o, l = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc, causal=causal)
    ob, lb = brute_attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc, causal=causal)
    assert np.abs(o - ob).max() <= 1e-12
    assert np.abs(l - lb).max() <= 1e-12


def test_attention_subset_rows_and_keys_vs_brute_force():
    cu, lay = _layout([9, 11])
    T = lay.T
    q, k, v = _rand(T, 2, 4), _rand(T, 1, 4), _rand(T, 1, 5)
    rows = np.array([0, 3, 10, 19])
    keys = np.array([1, 2, 9, 12, 15, 18])
    o, l = oracle.attention(q[rows], k[keys], v[keys], lay.pos[rows], lay.doc[rows],
                            lay.pos[keys], lay.doc[keys])
    ob, lb = brute_attention(q[rows], k[keys], v[keys], lay.pos[rows], lay.doc[rows],
                             lay.pos[keys], lay.doc[keys])
    # row 0 sees nothing among these keys: lse -inf, out 0 on both sides
    assert np.isneginf(l[:, 0]).all() and (o[0] == 0).all()
    assert np.array_equal(np.isneginf(l), np.isneginf(lb))
    fin = np.isfinite(lb)
    assert np.abs(l[fin] - lb[fin]).max() <= 1e-12
    assert np.abs(o - ob).max() <= 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _setup(lengths=(13, 7, 20), hq=4, hkv=2, d=8, dv=6):
    cu, lay = _layout(list(lengths))
    T = lay.T
    return cu, lay, _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv)


def test_zero_queries_give_mean_of_visible_values():
    cu, lay, q, k, v = _setup()
    q[:] = 0.0
    o, l = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc)
    n_vis = lay.pos - cu[lay.doc] + 1                       # keys seen by each row
    for h in range(q.shape[1]):
        g = h // 2
        csum = np.zeros_like(v[:, g, :])
        for dd in range(len(cu) - 1):
            a, b = cu[dd], cu[dd + 1]
            csum[a:b] = np.cumsum(v[a:b, g, :], axis=0)
        assert np.abs(o[:, h, :] - csum / n_vis[:, None]).max() <= 1e-13
        assert np.abs(l[h] - np.log(n_vis)).max() <= 1e-13


def test_first_token_of_each_document_sees_only_itself():
    cu, lay, q, k, v = _setup()
    o, l = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc)
    sc = 1.0 / math.sqrt(q.shape[2])
    for start in cu[:-1]:
        for h in range(q.shape[1]):
            g = h // 2
            assert np.abs(o[start, h] - v[start, g]).max() <= 1e-15
            assert abs(l[h, start] - sc * float(q[start, h] @ k[start, g])) <= 1e-13


def test_constant_values_scaling_and_key_shift():
    cu, lay, q, k, v = _setup()
    o, l = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc)
    vc = np.full_like(v, 2.5)
    oc, _ = oracle.attention(q, k, vc, lay.pos, lay.doc, lay.pos, lay.doc)
    assert np.abs(oc - 2.5).max() <= 1e-13
    oa, la = oracle.attention(q, k, -3.0 * v, lay.pos, lay.doc, lay.pos, lay.doc)
    assert np.abs(oa + 3.0 * o).max() <= 1e-12 and np.abs(la - l).max() == 0
    c = _rand(q.shape[2])
    ok_, lk = oracle.attention(q, k + c, v, lay.pos, lay.doc, lay.pos, lay.doc)
    sc = 1.0 / math.sqrt(q.shape[2])
    assert np.abs(ok_ - o).max() <= 1e-12
    shift = sc * np.einsum("thd,d->ht", q, c)
    assert np.abs(lk - (l + shift)).max() <= 1e-12


def test_probabilities_sum_to_one():
    cu, lay, q, k, v = _setup()
    _, _, p = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc, return_probs=True)
    assert np.abs(p.sum(axis=2) - 1.0).max() <= 1e-13


# ---------------------------------------------------------------------------
# library special case: torch float64 SDPA on the CPU
# ---------------------------------------------------------------------------

def _sdpa(q, k, v, mask, scale):
    hq, hkv = q.shape[1], k.shape[1]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    return tq, tk, tv


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (4, 1)])
def test_oracle_vs_torch_sdpa_causal(hq, hkv):
    T, d, dv = 96, 16, 12
    cu, lay = _layout([T])
    q, k, v = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv)
    o, l = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc)
    tq, tk, tv = _sdpa(q, k, v, None, None)
    ref_o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    s = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    ref_l = torch.logsumexp(s, dim=-1)[0]
    assert np.abs(o - ref_o[0].permute(1, 0, 2).numpy()).max() <= 1e-12
    assert np.abs(l - ref_l.numpy()).max() <= 1e-12


def test_oracle_vs_torch_sdpa_packed_documents_and_grads():
    lengths = [17, 40, 5, 34]
    cu, lay = _layout(lengths)
    T, hq, hkv, d, dv = lay.T, 4, 2, 8, 8
    q, k, v, do = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv), _rand(T, hq, dv)
    o, l = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc)
    dq, dk, dv_ = oracle.attention_bwd(q, k, v, do, lay.pos, lay.doc, lay.pos, lay.doc)
    allowed = torch.from_numpy((lay.doc[:, None] == lay.doc[None, :])
                               & (lay.pos[None, :] <= lay.pos[:, None]))
    tq = torch.from_numpy(q).clone().requires_grad_(True)
    tk = torch.from_numpy(k).clone().requires_grad_(True)
    tv = torch.from_numpy(v).clone().requires_grad_(True)
    qq = tq.permute(1, 0, 2)[None]
    kk = tk.permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    vv = tv.permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=allowed)
    (out * torch.from_numpy(do).permute(1, 0, 2)[None]).sum().backward()
    assert np.abs(o - out[0].detach().permute(1, 0, 2).numpy()).max() <= 1e-12
    s = (qq @ kk.transpose(-1, -2)) / math.sqrt(d)
    ref_l = torch.logsumexp(s.masked_fill(~allowed, float("-inf")), dim=-1)[0]
    assert np.abs(l - ref_l.detach().numpy()).max() <= 1e-12
    assert np.abs(dq - tq.grad.numpy()).max() <= 1e-11
    assert np.abs(dk - tk.grad.numpy()).max() <= 1e-11
    assert np.abs(dv_ - tv.grad.numpy()).max() <= 1e-11


# ---------------------------------------------------------------------------
# zig-zag map, ring order, pairs
# ---------------------------------------------------------------------------

def _golden_zigzag():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "zigzag_cp4.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(tuple(int(x) for x in line.split()))
    return rows


def test_zigzag_map_matches_printed_cp4_example():
    rows = _golden_zigzag()
    assert len(rows) == 4
    for c, r, a, b in rows:
        assert oracle.zigzag_chunks(c, r) == (a, b)
        # token-level map of a 64-token sequence (8 chunks of 8)
        idx, cu_l = oracle.zigzag_local_tokens(c, r, [0, 64])
        assert list(idx) == list(range(8 * a, 8 * a + 8)) + list(range(8 * b, 8 * b + 8))
        assert list(cu_l) == [0, 16]


def test_zigzag_map_is_a_partition_per_document():
    cu = synth.cu_seqlens([32, 96, 8, 64])
    C = 4
    seen = np.concatenate([oracle.zigzag_local_tokens(C, r, cu)[0] for r in range(C)])
    assert sorted(seen.tolist()) == list(range(int(cu[-1])))
    for r in range(C):
        idx, cu_l = oracle.zigzag_local_tokens(C, r, cu)
        assert list(cu_l) == [x // C for x in cu]
    with pytest.raises(ValueError):
        oracle.zigzag_local_tokens(4, 0, [0, 12])


def test_pad_reading():
    assert oracle.pad_to_multiple(64, 4) == 0
    assert oracle.pad_to_multiple(65, 4) == 7
    assert oracle.pad_to_multiple(5, 2) == 3


def test_ring_direction_follows_the_page_arrows():
    # KV blocks move device 0 -> 1 -> 2 -> 3 -> 0: after one step device 1
    # holds device 0's block and device 0 holds device 3's.
    assert oracle.ring_owner(1, 1, 4) == 0
    assert oracle.ring_owner(0, 1, 4) == 3
    assert [oracle.ring_owner(2, s, 4) for s in range(4)] == [2, 1, 0, 3]


@pytest.mark.parametrize("lengths,C", [([256], 4), ([64, 192, 32, 224], 4), ([96, 32], 8 // 4)])
def test_visible_pairs_balanced_per_rank(lengths, C):
    cu = synth.cu_seqlens(lengths)
    per = [oracle.visible_pairs(cu, C, r) for r in range(C)]
    assert len(set(per)) == 1
    assert sum(per) == sum(L * (L + 1) // 2 for L in lengths)
    if len(lengths) == 1:
        S = lengths[0]
        assert per[0] == S * S // (2 * C) + S // (2 * C)


# ---------------------------------------------------------------------------
# ring invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,C,hq,hkv", [([128], 4, 2, 1), ([64, 32, 96], 4, 2, 2),
                                             ([48], 8 // 2, 3, 1), ([16, 16], 8, 1, 1)])
def test_concat_of_rank_shares_equals_full_attention(lengths, C, hq, hkv):
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    q, k, v = _rand(T, hq, 8), _rand(T, hkv, 8), _rand(T, hkv, 4)
    o, l = oracle.full_attention(q, k, v, cu)
    got_o = np.zeros_like(o)
    got_l = np.zeros_like(l)
    for r in range(C):
        res = oracle.rank_share(q, k, v, cu, C, r)
        got_o[res["rows"]] = res["out"]
        got_l[:, res["rows"]] = res["lse"]
    assert np.abs(got_o - o).max() <= 1e-12
    assert np.abs(got_l - l).max() <= 1e-12


def test_merge_order_and_tree_invariance():
    cu = synth.cu_seqlens([256])
    C = 8
    q, k, v = _rand(256, 2, 8), _rand(256, 1, 8), _rand(256, 1, 8)
    base = oracle.rank_share(q, k, v, cu, C, 3)
    perm = list(RNG.permutation(C))
    alt = oracle.rank_share(q, k, v, cu, C, 3, order=perm)
    assert np.abs(base["out"] - alt["out"]).max() <= 1e-13
    assert np.abs(base["lse"] - alt["lse"]).max() <= 1e-13
    parts = base["steps"]
    while len(parts) > 1:                                   # pairwise tree
        nxt = []
        for i in range(0, len(parts) - 1, 2):
            o, l = oracle.lse_merge(parts[i][1], parts[i][2], parts[i + 1][1], parts[i + 1][2])
            nxt.append((None, o, l))
        if len(parts) % 2:
            nxt.append(parts[-1])
        parts = nxt
    assert np.abs(parts[0][1] - base["out"]).max() <= 1e-13


def test_merge_of_key_split_equals_union_and_identity():
    T, hq, d = 40, 2, 6
    q, k, v = _rand(T, hq, d), _rand(T, hq, d), _rand(T, hq, 5)
    pos = np.arange(T)
    doc = np.zeros(T, dtype=np.int64)
    sel = RNG.random(T) < 0.5
    a, b = np.where(sel)[0], np.where(~sel)[0]
    oa, la = oracle.attention(q, k[a], v[a], pos, doc, pos[a], doc[a])
    ob, lb = oracle.attention(q, k[b], v[b], pos, doc, pos[b], doc[b])
    om, lm = oracle.lse_merge(oa, la, ob, lb)
    ou, lu = oracle.attention(q, k, v, pos, doc, pos, doc)
    assert np.abs(om - ou).max() <= 1e-13 and np.abs(lm - lu).max() <= 1e-13
    # commutative; (0, -inf) is the identity; empty + empty stays empty
    om2, lm2 = oracle.lse_merge(ob, lb, oa, la)
    assert np.abs(om2 - om).max() <= 1e-15
    z_o, z_l = np.zeros_like(oa), np.full_like(la, -np.inf)
    oi, li = oracle.lse_merge(oa, la, z_o, z_l)
    assert np.array_equal(np.isneginf(li), np.isneginf(la))
    fin = np.isfinite(la)
    assert np.abs(oi - oa).max() == 0 and np.abs(li[fin] - la[fin]).max() == 0
    oe, le = oracle.lse_merge(z_o, z_l, z_o, z_l)
    assert not np.isnan(oe).any() and np.isneginf(le).all() and (oe == 0).all()


def test_merge_formula_on_printed_lse_rule_and_large_values():
    # lse_new = log(exp(lse_prev) + exp(lse_cur)) with values where the
    # naive form overflows; both sides one row, one head, dv = 1
    la = np.array([[1000.0]]); lb = np.array([[1000.0 + math.log(3.0)]])
    oa = np.array([[[2.0]]]); ob = np.array([[[6.0]]])
    o, l = oracle.lse_merge(oa, la, ob, lb)
    assert abs(l[0, 0] - (1000.0 + math.log(4.0))) <= 1e-12
    assert abs(o[0, 0, 0] - (0.25 * 2.0 + 0.75 * 6.0)) <= 1e-12


def test_step_coverage_matches_part_plan():
    """Step plan derived from the global causal rule: diagonal = all x all causal;
    owner j < r: all rows x first half of the owner's keys, every pair visible;
    owner j > r: second half of the rows x all the owner's keys, every pair visible."""
    for lengths, C in (([64], 4), ([32, 96, 64], 4), ([16, 48], 8)):
        cu = synth.cu_seqlens(lengths)
        for r in range(C):
            _, cu_l = oracle.zigzag_local_tokens(C, r, cu)
            first = np.concatenate([np.arange(cu_l[i], (cu_l[i] + cu_l[i + 1]) // 2)
                                    for i in range(len(cu_l) - 1)])
            Tl = int(cu_l[-1])
            first_mask = np.zeros(Tl, bool)
            first_mask[first] = True
            for s in range(C):
                j = oracle.ring_owner(r, s, C)
                rm, km, allp = oracle.step_coverage(cu, C, r, s)
                if j == r:
                    assert rm.all() and km.all()
                elif j < r:
                    assert rm.all() and np.array_equal(km, first_mask) and allp
                else:
                    assert np.array_equal(rm, ~first_mask) and km.all() and allp


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, lay):
    o, _ = oracle.attention(q, k, v, lay.pos, lay.doc, lay.pos, lay.doc)
    return float(np.sum(o * do))


def test_backward_vs_central_finite_differences():
    cu, lay = _layout([7, 5])
    T, hq, hkv, d, dv = lay.T, 2, 1, 4, 3
    q, k, v, do = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv), _rand(T, hq, dv)
    dq, dk, dvv = oracle.attention_bwd(q, k, v, do, lay.pos, lay.doc, lay.pos, lay.doc)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, lay)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, lay)
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - g).max() <= 1e-8, name


def test_backward_sum_rules():
    cu, lay = _layout([30, 50])
    T, hq, hkv, d, dv = lay.T, 4, 2, 6, 5
    q, k, v, do = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv), _rand(T, hq, dv)
    dq, dk, dvv = oracle.attention_bwd(q, k, v, do, lay.pos, lay.doc, lay.pos, lay.doc)
    # every row sees >= 1 key: sum_j dV_j = sum_i dO_i over the group's heads
    for g in range(hkv):
        assert np.abs(dvv[:, g].sum(0) - do[:, 2 * g:2 * g + 2].sum((0, 1))).max() <= 1e-12
    # softmax is shift invariant in K: sum_j dK_j = 0 per kv head
    assert np.abs(dk.sum(0)).max() <= 1e-12


def test_backward_decomposes_over_ring_steps():
    """Per-step gradients recomputed with the FINAL lse and delta add up to the full ones."""
    cu = synth.cu_seqlens([64, 32])
    C, hq, hkv, d, dv = 4, 2, 1, 6, 4
    lay = ref.Layout(cu)
    T = lay.T
    q, k, v, do = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, dv), _rand(T, hq, dv)
    dq, dk, dvv = oracle.attention_bwd(q, k, v, do, lay.pos, lay.doc, lay.pos, lay.doc)
    o, l = oracle.full_attention(q, k, v, cu)
    gq = np.zeros_like(dq); gk = np.zeros_like(dk); gv = np.zeros_like(dvv)
    for r in range(C):
        rows, _ = oracle.zigzag_local_tokens(C, r, cu)
        delta = oracle.bwd_delta(o[rows], do[rows])
        for s in range(C):
            j = oracle.ring_owner(r, s, C)
            kr, _ = oracle.zigzag_local_tokens(C, j, cu)
            a, b, c = oracle.attention_bwd(q[rows], k[kr], v[kr], do[rows], lay.pos[rows],
                                           lay.doc[rows], lay.pos[kr], lay.doc[kr],
                                           out=o[rows], lse=l[:, rows], delta=delta)
            gq[rows] += a; gk[kr] += b; gv[kr] += c
    assert np.abs(gq - dq).max() <= 1e-12
    assert np.abs(gk - dk).max() <= 1e-12
    assert np.abs(gv - dvv).max() <= 1e-12


# ---------------------------------------------------------------------------
# bfloat16 rounding
# ---------------------------------------------------------------------------

def test_bf16_rounding_hand_values():
    one = 1.0
    cases = {
        one: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,           # tie, kept lsb even -> down
        1.0 + 3 * 2.0 ** -8: 0x3F82,       # tie, kept lsb odd -> up
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,  # above the tie -> up
        -2.0: 0xC000,
        0.0: 0x0000,
        float("inf"): 0x7F80,
    }
    for x, bits in cases.items():
        got = oracle.bf16_round_bits(np.array([x], dtype=np.float32))[0]
        assert int(got) == bits, (x, hex(int(got)))


def test_bf16_rounding_vs_torch_cast():
    x = (RNG.standard_normal(100000) * 10.0 ** RNG.uniform(-30, 30, 100000)).astype(np.float32)
    got = oracle.bf16_round_bits(x)
    exp = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, exp)


# ---------------------------------------------------------------------------
# planted mistakes must be caught
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# other shard maps (oh-bug correctness section on causal imbalance)
# ---------------------------------------------------------------------------

def test_shard_maps_hand_examples():
    cu = [0, 8]
    assert list(oracle.map_local_tokens("striped", 2, 0, cu)) == [0, 2, 4, 6]
    assert list(oracle.map_local_tokens("striped", 2, 1, cu)) == [1, 3, 5, 7]
    assert list(oracle.map_local_tokens("contiguous", 2, 0, cu)) == [0, 1, 2, 3]
    assert list(oracle.map_local_tokens("contiguous", 2, 1, cu)) == [4, 5, 6, 7]
    assert list(oracle.map_local_tokens("zigzag_global", 2, 0, cu)) == [0, 1, 6, 7]
    assert list(oracle.map_local_tokens("zigzag_global", 2, 1, cu)) == [2, 3, 4, 5]
    # documents [0,4) and [4,8): the stream-level zig-zag ignores the boundary,
    # the per-document one splits each document
    assert list(oracle.map_local_tokens("zigzag_global", 2, 0, [0, 4, 8])) == [0, 1, 6, 7]
    assert list(oracle.map_local_tokens("zigzag", 2, 0, [0, 4, 8])) == [0, 3, 4, 7]


@pytest.mark.parametrize("kind", oracle.SHARD_MAPS)
@pytest.mark.parametrize("lengths,C", [([64], 4), ([16, 48, 8, 56], 4), ([32, 96], 8)])
def test_shard_maps_partition_the_stream(kind, lengths, C):
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    parts = [oracle.map_local_tokens(kind, C, r, cu) for r in range(C)]
    for p in parts:
        assert len(p) == T // C and np.all(np.diff(p) > 0)    # equal shares, global order
    assert np.array_equal(np.sort(np.concatenate(parts)), np.arange(T))


def test_single_sequence_stream_zigzag_is_the_zigzag():
    for r in range(4):
        assert np.array_equal(oracle.map_local_tokens("zigzag_global", 4, r, [0, 128]),
                              oracle.map_local_tokens("zigzag", 4, r, [0, 128]))


@pytest.mark.parametrize("kind", oracle.SHARD_MAPS)
def test_concat_of_map_rank_shares_equals_full_attention(kind):
    lengths, C, hq, hkv, d = [16, 48, 8, 56], 4, 2, 1, 8
    cu = synth.cu_seqlens(lengths)
    T = int(cu[-1])
    q, k, v = _rand(T, hq, d), _rand(T, hkv, d), _rand(T, hkv, d)
    full_o, full_l = oracle.full_attention(q, k, v, cu)
    cat_o = np.full_like(full_o, np.nan)
    cat_l = np.full_like(full_l, np.nan)
    for r in range(C):
        res = oracle.rank_share_map(kind, q, k, v, cu, C, r)
        cat_o[res["rows"]] = res["out"]
        cat_l[:, res["rows"]] = res["lse"]
    assert np.abs(cat_o - full_o).max() <= 1e-12
    assert np.abs(cat_l - full_l).max() <= 1e-12


def test_map_pair_counts_closed_forms_and_imbalance():
    S, C = 256, 4
    L = S // C
    cu = [0, S]
    for r in range(C):
        # contiguous: rows rL .. rL+L-1 see t+1 keys each
        assert oracle.map_visible_pairs("contiguous", cu, C, r) == L * (2 * r * L + L + 1) // 2
        # striped: rows iC + r, i < L
        assert oracle.map_visible_pairs("striped", cu, C, r) == C * L * (L - 1) // 2 + L * (r + 1)
        # both zig-zags balance one sequence exactly: (S^2 + S) / (2C)
        for kind in ("zigzag", "zigzag_global"):
            assert oracle.map_visible_pairs(kind, cu, C, r) == (S * S + S) // (2 * C)
    lengths = [16, 48, 8, 56, 8, 120]
    cu = synth.cu_seqlens(lengths)
    total = sum(l * (l + 1) // 2 for l in lengths)
    for kind in oracle.SHARD_MAPS:
        per = [oracle.map_visible_pairs(kind, cu, 4, r) for r in range(4)]
        assert sum(per) == total, kind
        if kind == "zigzag":
            assert len(set(per)) == 1
        if kind == "zigzag_global":
            assert len(set(per)) > 1           # the packed-varlen imbalance


@pytest.mark.parametrize("kind", oracle.SHARD_MAPS)
def test_step_visibility_sums_to_rank_pairs(kind):
    cu = synth.cu_seqlens([16, 48, 8, 56])
    for r in range(4):
        tot = sum(int(oracle.step_visible(kind, cu, 4, r, o).sum()) for o in range(4))
        assert tot == oracle.map_visible_pairs(kind, cu, 4, r)


def _pins_pass():
    """Run a representative subset of the pins; False if any fails."""
    try:
        test_attention_vs_brute_force([7, 9, 4], 4, 2, 5, 6, True)
        test_oracle_vs_torch_sdpa_causal(8, 2)
        test_zigzag_map_matches_printed_cp4_example()
        test_concat_of_rank_shares_equals_full_attention([64, 32, 96], 4, 2, 2)
        test_merge_of_key_split_equals_union_and_identity()
        test_merge_formula_on_printed_lse_rule_and_large_values()
        test_backward_sum_rules()
        test_step_coverage_matches_part_plan()
        test_shard_maps_hand_examples()
        test_concat_of_map_rank_shares_equals_full_attention("striped")
        test_map_pair_counts_closed_forms_and_imbalance()
    except (AssertionError, ValueError, FloatingPointError):
        return False
    return True


MUTANTS = {
    "gqa_mod_mapping": ("_kv_head", lambda h, hq, hkv: h % hkv),
    "mask_strict": ("_visible", lambda qp, qd, kp, kd, causal:
                    (qd[:, None] == kd[None, :]) & ((kp[None, :] < qp[:, None]) if causal else True)),
    "mask_ignores_docs": ("_visible", lambda qp, qd, kp, kd, causal:
                          (kp[None, :] <= qp[:, None]) if causal else np.ones((len(qp), len(kp)), bool)),
    "zigzag_off_by_one": ("zigzag_chunks", lambda c, r: (r, 2 * c - 2 - r) if r < c - 1 else (r, c)),
    "scale_wrong": ("softmax_scale", lambda d: 1.0 / d),
    # a relabelling of ranks still partitions the stream; only the printed /
    # hand examples and closed forms catch it
    "striped_ranks_rotated": ("map_local_tokens", lambda kind, C, r, cu, _f=ref.map_local_tokens:
                              _f(kind, C, (r + 1) % C if kind == "striped" else r, cu)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_oracle_mistakes_fail_a_pin(monkeypatch, name):
    attr, fn = MUTANTS[name]
    assert _pins_pass()
    monkeypatch.setattr(ref, attr, fn)
    assert not _pins_pass(), f"mutant {name} survived every pin"


def test_planted_merge_mistake_fails_a_pin(monkeypatch):
    def bad_merge(oa, la, ob, lb):        # averages instead of weighting by lse
        return 0.5 * (np.asarray(oa) + np.asarray(ob)), np.logaddexp(la, lb)
    monkeypatch.setattr(ref, "lse_merge", bad_merge)
    monkeypatch.setattr(oracle, "lse_merge", bad_merge)
    assert not _pins_pass()
