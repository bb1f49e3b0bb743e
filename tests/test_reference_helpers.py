"""CPU check of the full-size reference helpers of the GPU tests.

``gpu_util.oracle_rows`` and ``gpu_util.oracle_grads`` call the oracle once
per query head (and, for rows, with each run's visible key prefix only),
and ``gpu_util.oracle_attention_by_document`` once per document, so that
whole full-size rank shares can be compared in seconds.  They must give
exactly what one plain call of the oracle gives: packed documents, grouped
heads, rows in several runs per document.
"""
import numpy as np

import oracle
import synth
from gpu_util import oracle_attention_by_document, oracle_grads, oracle_rows


def _inputs(lengths, hq, hkv, dqk, dv, seed):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q = rng.standard_normal((T, hq, dqk))
    k = rng.standard_normal((T, hkv, dqk))
    v = rng.standard_normal((T, hkv, dv))
    do = rng.standard_normal((T, hq, dv))
    return synth.cu_seqlens(lengths), q, k, v, do


def test_oracle_rows_equals_plain_oracle():
    cu, q, k, v, _ = _inputs([40, 1, 96, 63], 6, 2, 16, 8, 1)
    rows = np.array([0, 1, 2, 39, 40, 41, 42, 60, 61, 62, 100, 136, 137, 199], np.int64)
    got_o, got_l = oracle_rows(q, k, v, cu, rows)
    ref_o, ref_l = oracle.full_attention(q, k, v, cu, rows=rows)
    assert np.allclose(got_o, ref_o, rtol=0, atol=1e-13)
    assert np.allclose(got_l, ref_l, rtol=0, atol=1e-13)
    # every row of a zig-zag rank share, in local order sorted
    idx, _ = oracle.zigzag_local_tokens(2, 1, synth.cu_seqlens([64, 128]))
    cu2, q, k, v, _ = _inputs([64, 128], 4, 4, 8, 8, 2)
    got_o, got_l = oracle_rows(q, k, v, cu2, idx)
    ref_o, ref_l = oracle.full_attention(q, k, v, cu2, rows=idx)
    assert np.allclose(got_o, ref_o, rtol=0, atol=1e-13)
    assert np.allclose(got_l, ref_l, rtol=0, atol=1e-13)


def test_oracle_grads_equals_plain_oracle():
    cu, q, k, v, do = _inputs([33, 70, 2], 4, 2, 12, 8, 3)
    lay = oracle.ref.Layout(cu)
    ref = oracle.attention_bwd(q, k, v, do, lay.pos, lay.doc, lay.pos, lay.doc)
    got = oracle_grads(q, k, v, do, cu)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_oracle_by_document_equals_plain_oracle():
    cu, q, k, v, _ = _inputs([40, 1, 96, 63, 2], 6, 2, 16, 8, 3)
    got_o, got_l = oracle_attention_by_document(q, k, v, cu)
    ref_o, ref_l = oracle.full_attention(q, k, v, cu)
    assert np.allclose(got_o, ref_o, rtol=0, atol=1e-13)
    assert np.allclose(got_l, ref_l, rtol=0, atol=1e-13)
