"""GPU parity where element offsets pass 2^31.

One non-causal block of 2^21 query tokens x 16 query heads (4 kv heads) x
128 dims against 400 keys: Q and dO hold 2^32 bf16 elements each (8 GiB),
out and dQ 2^32 float32 (16 GiB).  Sampled rows are checked against the
fp64 oracle on both bf16 forward kernels.  They sit where the element
offset of Q or out, or the byte offset of out, crosses 2^31, plus the last
rows.  For the backward: dQ of the same rows, and over every row the sum
rules sum_j dV_j = sum_i dO_i (per kv head, its query heads added) and
sum_j dK_j = 0.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_lse, check_out, log, to_np

pytestmark = pytest.mark.gpu

R = pytest.importorskip("context_blockwise_softmax_ra_amd")
from context_blockwise_softmax_ra_amd import _lib as L  # noqa: E402

DEV = torch.device("cuda:0")

T, HQ, HKV, D, TK = 1 << 21, 16, 4, 128, 400


def _sample_rows():
    rows = []
    for b in (1 << 18, 1 << 19, 1 << 20):     # out bytes, -, Q/out elements cross 2^31 at 2^20
        rows.extend(range(b - 40, b + 40))
    rows.extend(range(T - 48, T))
    rng = np.random.default_rng(5)
    rows.extend(rng.integers(0, T, 32).tolist())
    return np.unique(np.array(rows, dtype=np.int64))


def _randn(shape, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def test_offsets_past_2_31_forward_and_backward(monkeypatch):
    free, _ = torch.cuda.mem_get_info()
    if free < 64 << 30:
        pytest.skip(f"needs 64 GiB of free device memory, {free >> 30} GiB free")
    log(f"T={T} hq={HQ} hkv={HKV} d={D} keys={TK}")
    q = _randn((T, HQ, D), 101)
    k = _randn((TK, HKV, D), 102)
    v = _randn((TK, HKV, D), 103)
    cu_q = np.array([0, T], np.int32)
    cu_k = np.array([0, TK], np.int32)
    cuq = torch.from_numpy(cu_q).to(DEV)
    cuk = torch.from_numpy(cu_k).to(DEV)
    desc = L.attn_desc(q, k, v, cuq, cuk, cu_q, cu_k, causal=False)
    rows = _sample_rows()
    ridx = torch.from_numpy(rows).to(DEV)
    q64 = to_np(q[ridx])
    k64, v64 = to_np(k), to_np(v)
    z = np.zeros(len(rows), np.int64)
    ro, rl = oracle.attention(q64, k64, v64, z, z, np.zeros(TK, np.int64), np.zeros(TK, np.int64),
                              causal=False)

    out = torch.empty((T, HQ, D), device=DEV, dtype=torch.float32)
    lse = torch.empty((HQ, T), device=DEV, dtype=torch.float32)
    for kernel in ("4w", "pp"):
        monkeypatch.setenv("RA_FWD_KERNEL", kernel)
        log(f"forward, kernel {kernel}")
        out.fill_(7.0)
        lse.fill_(7.0)
        L.ra_block_attn_fwd(desc, out, lse)
        torch.cuda.synchronize()
        check_out(to_np(out[ridx]), ro, "bf16", f"{kernel} sampled rows")
        check_lse(to_np(lse[:, ridx]), rl, f"{kernel} sampled rows")
        assert bool(torch.isfinite(out[-1]).all()) and bool(torch.isfinite(lse[:, -1]).all())
    monkeypatch.delenv("RA_FWD_KERNEL", raising=False)

    log("backward")
    do = _randn((T, HQ, D), 104)
    delta = torch.empty((HQ, T), device=DEV, dtype=torch.float32)
    L.ra_attn_bwd_delta(out, do, delta)
    dq = torch.zeros((T, HQ, D), device=DEV, dtype=torch.float32)
    dk = torch.zeros((TK, HKV, D), device=DEV, dtype=torch.float32)
    dv = torch.zeros((TK, HKV, D), device=DEV, dtype=torch.float32)
    L.ra_block_attn_bwd(desc, do, lse, delta, dq, dk, dv)
    torch.cuda.synchronize()
    do64 = to_np(do[ridx])
    a, _, _ = oracle.attention_bwd(q64, k64, v64, do64, z, z, np.zeros(TK, np.int64),
                                   np.zeros(TK, np.int64), causal=False, out=ro, lse=rl)
    check_out(to_np(dq[ridx]), a, "bf16", "dQ sampled rows")
    # sum rules over every row (dO summed on the device in float64, in chunks)
    sdo = torch.zeros((HQ, D), device=DEV, dtype=torch.float64)
    for t0 in range(0, T, 1 << 18):
        sdo += do[t0:t0 + (1 << 18)].to(torch.float64).sum(0)
    sdo = sdo.cpu().numpy().reshape(HKV, HQ // HKV, D).sum(1)
    sdv = to_np(dv).sum(0)
    rel = np.abs(sdv - sdo).max() / np.abs(sdo).max()
    log(f"  sum dV vs sum dO rel={rel:.2e}")
    assert rel <= 1e-3
    adk = np.abs(to_np(dk)).sum(0)
    rel = np.abs(to_np(dk).sum(0)).max() / adk.max()
    log(f"  |sum dK| / sum|dK| = {rel:.2e}")
    assert rel <= 1e-3
    del q, k, v, out, lse, do, delta, dq, dk, dv, ridx
    gc.collect()
    torch.cuda.empty_cache()
