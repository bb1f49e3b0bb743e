"""Helpers for the GPU parity tests: problem set-up, oracle references, tolerances.

Tolerances (fixed for this path): bfloat16 outputs max-abs <= 2e-2 and
relative RMS <= 1e-2; float32 path <= 1e-5; lse max-abs <= 1e-3 over finite
rows with -inf matching exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 1e-2
F32_MAX_ABS = 1e-5
LSE_MAX_ABS = 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def metrics(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.sqrt((ref ** 2).sum()))
    rel = float(np.sqrt((diff ** 2).sum()) / den) if den > 0 else float(np.sqrt((diff ** 2).sum()))
    return max_abs, rel


def check_out(got, ref, dtype: str, tag: str = ""):
    assert not np.isnan(np.asarray(got, np.float64)).any(), f"{tag}: NaN in output"
    ma, rr = metrics(got, ref)
    log(f"  {tag}: out max_abs={ma:.3e} rel_rms={rr:.3e}")
    if dtype == "fp32":
        assert ma <= F32_MAX_ABS, (tag, ma)
    else:
        assert ma <= BF16_MAX_ABS and rr <= BF16_REL_RMS, (tag, ma, rr)
    return ma, rr


def check_lse(got, ref, tag: str = "", tol: float = LSE_MAX_ABS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert not np.isnan(got).any(), f"{tag}: NaN in lse"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{tag}: -inf pattern differs"
    fin = np.isfinite(ref)
    ma = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    log(f"  {tag}: lse max_abs={ma:.3e}")
    assert ma <= tol, (tag, ma)
    return ma


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def global_inputs(w: synth.Workload, with_dout: bool = False):
    """CPU storage-dtype tensors (bf16/fp32) and their exact float64 copies."""
    q = synth.cast(w.q(), w.dtype)
    k = synth.cast(w.k(), w.dtype)
    v = synth.cast(w.v(), w.dtype)
    do = synth.cast(w.do(), w.dtype) if with_dout else None
    return (q, k, v, do)


def make_problem(w: synth.Workload, with_dout=False, device="cuda:0"):
    from context_blockwise_softmax_ra_amd.ring import RingProblem
    q, k, v, do = global_inputs(w, with_dout)
    dev = torch.device(device)
    prob = RingProblem(q.to(dev), k.to(dev), v.to(dev), w.cu_global(), w.cp,
                       dout_glob=do.to(dev) if do is not None else None)
    return prob, (q, k, v, do)


def sample_rows(prob, r: int, n: int, seed: int = 0) -> np.ndarray:
    """Local rows of rank r: both ends of both halves of the first/last segments, plus random."""
    cl = prob.cu_local
    pick = set()
    for s in (0, len(cl) - 2):
        a, b = int(cl[s]), int(cl[s + 1])
        c = (b - a) // 2
        for x in (a, a + 1, a + c - 1, a + c, a + c + 1, b - 1):
            if a <= x < b:
                pick.add(x)
    rng = np.random.default_rng(seed + r)
    while len(pick) < min(n, prob.Tl):
        pick.add(int(rng.integers(0, prob.Tl)))
    return np.array(sorted(pick), dtype=np.int64)
