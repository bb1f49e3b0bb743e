#!/usr/bin/env python3
"""Throughput of the ring-attention rank shares on one MI355X.

A step is one pass of the whole forward hot path over one batch of the
workload: for every simulated rank r of the CP group, ``ra_rank_forward``
(the diagonal causal block, the C-1 history blocks, the lse merges and the
bf16 finalisation) on the rank's zig-zag shard, all on one stream.  By
default (``--fuse-merge 2``) each rank share is one launch that walks every
block with the online-softmax state in registers; ``--fuse-merge 0`` runs
one launch per block plus ``ra_lse_merge`` per history block.

Default workload: 32K grouped-query causal attention (32 query heads over
8 KV heads, head dim 128, bf16), zig-zag CP=8, N(0,1)*0.5 inputs.

Prints one JSON line.  ``value`` is the effective attention TFLOP/s of the
whole step (causal FLOPs counted once: 2*(dqk+dv) per visible pair per
query head).  ``roofline`` is for the dominant kernel, the bf16 block
attention forward: algorithmic FLOPs over its average launch duration.  In
the default fused form the timed steps consist of nothing but the C
attention launches per step, back to back, so the average launch is the
timed region (two HIP events on the launch stream) over the launch count.
A second, untimed-for-``value`` pass of the same steps records HIP events
around every launch (the library records them on the launch stream) for
the per-launch and per-rank median / min / max in ``stats`` and
``per_rank``; the per-block forms take their launch durations from such
events directly.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_32k")
    ap.add_argument("--fuse-merge", type=int, default=2,
                    help="0: per-step partials + ra_lse_merge; 1: merge in the attention "
                         "epilogue; 2: the whole rank share in one launch")
    ap.add_argument("--mode", default="ring", choices=("ring", "ulysses"),
                    help="ring: zig-zag ring-attention rank shares (the headline); ulysses: "
                         "the Ulysses rank shares of the same workload (all tokens, Hq/C "
                         "heads each) on the same kernels, with the per-rank work of both")
    ap.add_argument("--map", default=None,
                    choices=("zigzag", "zigzag_global", "striped", "contiguous"),
                    help="run the ring shares under this shard map through per-step rectangle "
                         "launches (the same 4-wave kernel for every map) and report the "
                         "per-rank work and time imbalance")
    ap.add_argument("--kernel", default="auto", choices=("auto", "4w", "pp"),
                    help="bf16 forward kernel: chosen by launch size (auto), the 4-wave "
                         "kernel, or the 8-wave ping-pong kernel")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle CPU baseline sample (0 = skip)")
    ap.add_argument("--backward", type=int, default=0,
                    help="1: time the backward shares (after one forward) instead; for the "
                         "256K MLA workload")
    ap.add_argument("--bwd-rank-fused", type=int, default=-1,
                    help="backward: 1 = one dK/dV and one dQ launch per rank share (every owner's "
                         "blocks), 0 = one pair of launches per ring step, -1 = the library's "
                         "choice (rank-fused)")
    ap.add_argument("--merge", type=int, default=0,
                    help="1: time ra_lse_merge alone on the workload's full-row step (every "
                         "local row, every query head, fp32 partials) and report HBM GB/s")
    ap.add_argument("--mfma-ceiling", type=int, default=0,
                    help="1: time a pure v_mfma_f32_32x32x16_bf16 loop on operands drawn like "
                         "the workload's (and on constant ones): the matrix cores' sustained "
                         "rate on this data")
    ap.add_argument("--per-block-steps", type=int, default=5,
                    help="after a fused (--fuse-merge 2) run, time this many steps with one "
                         "launch per ring block to report diagonal vs history launches "
                         "(0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 3 times (the "
                         "reference kernel that scales HBM byte counters), then exit")
    return ap.parse_args()


def bench_merge(a, w, torch, L):
    """ra_lse_merge on one full-row step of a rank share: HBM-bound, in GB/s.

    Cache-cold: the merge's working set (both partials and lses, ~203 MB for
    the 32K workload) fits the 256 MB Infinity Cache, so a 1 GiB buffer is
    read (summed) between merges and every merge is timed alone by HIP events
    on the stream it runs on.  The buffer is read rather than written so that
    no dirty cache lines are left to drain to HBM during the timed merge.
    """
    import numpy as np
    dev = torch.device("cuda:0")
    T = w.seqlen // w.cp                        # local rows of a rank share
    cu = np.array([0, T], np.int32)
    cud = torch.from_numpy(cu).to(dev)
    g = torch.Generator(device=dev).manual_seed(11)
    oa = torch.randn((T, w.hq, w.dv), generator=g, device=dev)
    ob = torch.randn((T, w.hq, w.dv), generator=g, device=dev)
    la = torch.randn((w.hq, T), generator=g, device=dev)
    lb = torch.randn((w.hq, T), generator=g, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        L.ra_lse_merge(oa, la, ob, lb, cud, cu, 0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i in range(a.steps):
        flush.sum()                             # reads 1 GiB: evicts the caches
        ev[i][0].record(stream)
        L.ra_lse_merge(oa, la, ob, lb, cud, cu, 0)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    # the same stream shape without the merge arithmetic, as a practical
    # ceiling of this read/read/write mix: torch's elementwise add of the two
    # partials into a third buffer, cache-cold in the same way
    oc = torch.empty_like(oa)
    for _ in range(a.warmup):
        torch.add(oa, ob, out=oc)
    ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i in range(a.steps):
        flush.sum()
        ev2[i][0].record(stream)
        torch.add(oa, ob, out=oc)
        ev2[i][1].record(stream)
    torch.cuda.synchronize()
    ms_add = sorted(e0.elapsed_time(e1) for e0, e1 in ev2)
    add_bytes = 3 * oa.numel() * 4
    nbytes = T * w.hq * (12 * w.dv + 12)       # read both partials and lses, write acc + lse
    mean = sum(ms) / len(ms)
    med = ms[len(ms) // 2]
    gbs = nbytes / (mean / 1e3) / 1e9
    return {
        "metric": "lse merge HBM GB/s (one full-row step of a rank share, fp32 partials, "
                  "cache-cold), 1 GPU",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(mean, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": f"{w.name}: ra_lse_merge of {T} rows x {w.hq} heads x dv {w.dv}, "
                               f"1 GiB read between merges",
                   "bytes_per_merge": nbytes},
        "stats": {"merge_ms_median": round(med, 5), "merge_ms_min": round(ms[0], 5),
                  "merge_ms_max": round(ms[-1], 5),
                  "gbs_median": round(nbytes / (med / 1e3) / 1e9, 1),
                  "gbs_best": round(nbytes / (ms[0] / 1e3) / 1e9, 1),
                  "reference_torch_add_gbs_median":
                      round(add_bytes / (ms_add[len(ms_add) // 2] / 1e3) / 1e9, 1),
                  "reference_torch_add_bytes": add_bytes},
        "roofline": {"bound": "hbm", "kernel": "lse_merge_kernel", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }


def bench_mfma_ceiling(a, w, torch, L):
    """Sustained v_mfma_f32_32x32x16_bf16 rate of a pure product loop (two
    waves per SIMD, no memory traffic in the loop) on operands drawn like the
    workload's inputs (its Q draw, bf16), and on constant operands: the rate
    the attention kernels are bounded by on this data."""
    import synth
    dev = torch.device("cuda:0")
    ops = synth.cast(w.q(0, 8192), w.dtype).to(dev).contiguous()     # 8192 tokens of Q
    const = torch.full_like(ops, 0.25)
    n_wg, iters = 512, 4000                                          # two workgroups per CU
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    flops = n_wg * 4 * iters * 64 * 2 * 32 * 32 * 16
    stream = torch.cuda.current_stream()
    res = {}
    for name, buf in (("workload_operands", ops), ("constant_operands", const)):
        for _ in range(2):
            L.ra_mfma_ceiling(buf, out, n_wg, iters)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(a.steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            L.ra_mfma_ceiling(buf, out, n_wg, iters)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        med = ms[len(ms) // 2]
        res[name] = {"ms_median": round(med, 4), "ms_min": round(ms[0], 4),
                     "tflops_median": round(flops / (med / 1e3) / 1e12, 1),
                     "tflops_best": round(flops / (ms[0] / 1e3) / 1e12, 1),
                     "frac_median": round(flops / (med / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    v = res["workload_operands"]["tflops_median"]
    return {
        "metric": "MFMA-loop ceiling: sustained v_mfma_f32_32x32x16_bf16 TFLOP/s, 1 GPU",
        "value": v, "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": 2,
        "ms_per_step": res["workload_operands"]["ms_median"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"operands: the first 8192 tokens of the {w.name} Q draw (seeded "
                f"N(0,1)*{w.mult:g}, bf16), or constant 0.25",
        "config": {"workload": f"pure product loop, {n_wg} workgroups x 4 waves (two per SIMD), "
                               f"{iters} x 64 products per wave, 8 accumulator chains",
                   "flop_per_launch": flops},
        "ceiling": res,
        "roofline": {"bound": "mfma", "kernel": "mfma_ceiling_kernel", "achieved": v,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(v / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 3}), flush=True)


def kernel_hash(kernel: str) -> str:
    """Hash of the sources a forward kernel is built from."""
    csrc = os.path.join(ROOT, "context_blockwise_softmax_ra_amd", "csrc")
    h = hashlib.sha256()
    for f in ("mfma_common.h", "fwd_tiles.h", kernel + ".hip"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per attention launch from committed counter runs, if still current."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    if t.get("kernel_sha256_16") != kernel_hash(kernel):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on a bounded sample of rank 0's rows, in effective TFLOP/s."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    cu = w.cu_global()
    rows, _ = oracle.zigzag_local_tokens(w.cp, 0, cu)
    rng = np.random.default_rng(0)
    order = rng.permutation(len(rows))
    q = synth.cast(w.q(), w.dtype).to(__import__("torch").float64).numpy()
    k = synth.cast(w.k(), w.dtype).to(__import__("torch").float64).numpy()
    v = synth.cast(w.v(), w.dtype).to(__import__("torch").float64).numpy()
    lay = oracle.ref.Layout(cu)
    done = 0
    flops = 0.0
    t0 = time.perf_counter()
    blk = 32
    while done < len(rows):
        sel = rows[order[done:done + blk]]
        oracle.full_attention(q, k, v, cu, rows=sel)
        vis = (sel - cu[lay.doc[sel]] + 1).sum()
        flops += float(vis) * w.hq * 2 * (w.dqk + w.dv)
        done += len(sel)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"rank 0 of {w.name}: {done} of {len(rows)} local rows (random), all "
                      f"{w.hq} query heads over every visible key, float64 NumPy, {dt:.1f} s",
            "cpu_model": cpu_model(), "blas": blas_vendor()}


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def blas_vendor() -> str:
    """BLAS library NumPy calls (name, version, threads), as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return (f"{i.get('internal_api')} {i.get('version')} "
                        f"({i.get('threading_layer', '')}, {i.get('num_threads')} threads)")
    except Exception:
        pass
    return "unknown"


def _timed_steps(run_step, ev, a, torch, stream):
    """Warm-up, then a.steps timed steps with no per-launch events (an event
    recorded between two launches leaves a gap of ~10 us before the next),
    then the same number of steps recording ev[i] for the per-launch times.
    Returns the timed steps' ms per step."""
    for e3 in ev:  # recorded once before the timed region
        for e2 in e3:
            for e in e2:
                e.record(stream)
    for _ in range(a.warmup):
        run_step()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(a.steps):
        run_step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / a.steps
    for i in range(a.steps):
        run_step(ev[i])
    torch.cuda.synchronize()
    return ms_step


def bench_backward(a, w, prob, torch, L):
    """Backward step: every rank's ra_rank_backward (delta, then dK/dV over
    every owner's key tiles and dQ over all blocks in one launch each, or
    with --bwd-rank-fused 0 one dQ and one dK/dV launch per ring step)."""
    import synth
    C = w.cp
    if a.bwd_rank_fused in (0, 1):
        os.environ["RA_BWD_RANK_FUSED"] = str(a.bwd_rank_fused)
    else:
        os.environ.pop("RA_BWD_RANK_FUSED", None)
    form = {0: "per ring step", 1: "rank-fused"}.get(a.bwd_rank_fused, "library's choice")
    dev = prob.q[0].device
    do = synth.cast(w.do(), w.dtype).to(dev)
    prob.do = [prob.gather(do, r) for r in range(C)]
    del do
    fwd = []
    for r in range(C):
        out, lse, ws = prob.alloc_forward(torch.bfloat16, True)
        prob.forward(r, out, lse, ws, fuse_merge=True)
        fwd.append((out, lse))
    del ws
    dqs = [torch.zeros((prob.Tl, prob.hq, prob.dqk), device=dev) for _ in range(C)]
    dks = [torch.zeros((prob.Tl, prob.hkv, prob.dqk), device=dev) for _ in range(C)]
    dvs = [torch.zeros((prob.Tl, prob.hkv, prob.dv), device=dev) for _ in range(C)]
    n = L.ra_rank_backward_workspace(prob.backward_desc(0, fwd[0][0], fwd[0][1], dqs[0], dks,
                                                        dvs, None))
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    work = [prob.work(r) for r in range(C)]
    fl_pair = 2 * (3 * w.dqk + 2 * w.dv)
    step_flops = sum(p for r in range(C) for (p, _, _) in work[r]) * fl_pair
    stream = torch.cuda.current_stream()

    def run_step(events=None):
        for r in range(C):
            prob.backward(r, fwd[r][0], fwd[r][1], dqs[r], dks, dvs, ws,
                          events=None if events is None else events[r])

    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2 * C)] for _ in range(C)]
          for _ in range(a.steps)]
    ms_step = _timed_steps(run_step, ev, a, torch, stream)
    # both forms record event 0 before a rank's first launch and event 2C-1
    # after its last: the rank's span
    blk_ms = sum(ev[i][r][0].elapsed_time(ev[i][r][2 * C - 1])
                 for i in range(a.steps) for r in range(C))
    achieved = step_flops * a.steps / (blk_ms / 1e3) / 1e12
    res = {
        "metric": "effective attention backward TFLOP/s per rank-share (bf16), 1 GPU",
        "value": round(step_flops / (ms_step / 1e3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16 RNE)",
        "config": {"workload": f"{w.name}: backward of all {C} rank shares (dQ, dK, dV "
                               f"recomputed from the saved lse), S={w.seqlen}, {w.hq} heads, "
                               f"head dim {w.dqk}/{w.dv}",
                   "step_effective_tflop": round(step_flops / 1e12, 4),
                   "flop_per_pair": fl_pair},
        "roofline": {"bound": "mfma",
                     "kernel": f"attn_bwd_dq + attn_bwd_dkdv ({form})",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def bench_ulysses(a, w, q, k, v, torch, L):
    """Forward step: every rank's Ulysses share (one causal launch over a head slice)."""
    from context_blockwise_softmax_ra_amd.ulysses import UlyssesProblem
    C = w.cp
    uly = UlyssesProblem(q, k, v, w.cu_global(), C)
    bufs = [uly.alloc_forward() for _ in range(C)]
    fl_pair = 2 * (w.dqk + w.dv)
    work = [uly.work(r) for r in range(C)]
    step_flops = sum(wk[0] for wk in work) * fl_pair
    stream = torch.cuda.current_stream()

    def run_step(events=None):
        for r in range(C):
            uly.forward(r, *bufs[r], events=None if events is None else events[r])

    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(C)]
          for _ in range(a.steps)]
    ms_step = _timed_steps(run_step, ev, a, torch, stream)
    per_rank_ms = [sum(ev[i][r][0].elapsed_time(ev[i][r][1]) for i in range(a.steps)) / a.steps
                   for r in range(C)]
    achieved = step_flops / (sum(per_rank_ms) / 1e3) / 1e12
    kname = L.ra_forward_kernel(uly.local_desc(0, causal=True), L.PART_ALL)
    res = {
        "metric": "effective attention TFLOP/s per Ulysses rank-share (bf16), 1 GPU",
        "value": round(step_flops / (ms_step / 1e3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*%g, bf16 RNE)" % w.mult,
        "config": {"workload": f"{w.name}: causal attention, S={w.seqlen}, Ulysses CP={C} (all "
                               f"{C} rank shares, each all tokens x {w.hq // C} q heads / "
                               f"{w.hkv // C} kv heads), head dim {w.dqk}/{w.dv}",
                   "step_effective_tflop": round(step_flops / 1e12, 4)},
        "roofline": {"bound": "mfma", "kernel": kname + " (one causal launch per rank share)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "per_rank": {"ms": [round(x, 4) for x in per_rank_ms],
                     "pairs_x_heads": [int(wk[0]) for wk in work],
                     "tiles_visited": [int(wk[1]) for wk in work],
                     "tiles_skipped": [int(wk[2]) for wk in work]},
        "cpu_baseline": None,
    }
    return res


def bench_map(a, w, q, k, v, torch, L):
    """Forward step under a shard map: every rank's share as C rectangle launches."""
    from context_blockwise_softmax_ra_amd.maps import MapProblem
    C = w.cp
    prob = MapProblem(a.map, q, k, v, w.cu_global(), C)
    bufs = [prob.alloc_forward() for _ in range(C)]
    fl_pair = 2 * (w.dqk + w.dv)
    work = [prob.work(r) for r in range(C)]
    rank_pairs = [sum(p for p, _, _ in wk) for wk in work]
    step_flops = sum(rank_pairs) * fl_pair
    stream = torch.cuda.current_stream()

    def run_step(events=None):
        for r in range(C):
            prob.forward(r, *bufs[r], events=None if events is None else events[r])

    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2 * C)] for _ in range(C)]
          for _ in range(a.steps)]
    ms_step = _timed_steps(run_step, ev, a, torch, stream)
    rank_ms = [sum(ev[i][r][2 * s].elapsed_time(ev[i][r][2 * s + 1])
                   for i in range(a.steps) for s in range(C)) / a.steps for r in range(C)]
    achieved = step_flops / (sum(rank_ms) / 1e3) / 1e12
    mean_ms = sum(rank_ms) / C
    mean_pairs = sum(rank_pairs) / C
    slow = max(range(C), key=lambda r: rank_ms[r])
    return {
        "metric": "effective attention TFLOP/s per rank-share (bf16) under a shard map, 1 GPU",
        "value": round(step_flops / (ms_step / 1e3) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*%g, bf16 RNE)" % w.mult,
        "config": {"workload": f"{w.name}: causal attention, S={w.seqlen}, CP={C}, shard map "
                               f"{a.map} (all {C} rank shares, each C rectangle launches merged "
                               f"in the epilogue), {w.hq} q heads / {w.hkv} kv heads, head dim "
                               f"{w.dqk}/{w.dv}",
                   "map": a.map, "step_effective_tflop": round(step_flops / 1e12, 4)},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16 (rectangle lists)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "per_rank": {"ms": [round(x, 4) for x in rank_ms],
                     "pairs_x_heads": [int(x) for x in rank_pairs],
                     "tiles_visited": [int(sum(t for _, t, _ in wk)) for wk in work],
                     "slowest_rank": slow,
                     "time_max_over_mean": round(rank_ms[slow] / mean_ms, 4),
                     "pairs_max_over_mean": round(max(rank_pairs) / mean_pairs, 4),
                     "concurrent_step_ms": round(rank_ms[slow], 4)},
        "cpu_baseline": None,
    }


def _median(x):
    x = sorted(x)
    n = len(x)
    return x[n // 2] if n % 2 else 0.5 * (x[n // 2 - 1] + x[n // 2])


def launch_stats(ev, work, fl_pair, C, steps, fuse_merge):
    """Median / min / max of the step span (first event of rank 0 to the last
    of rank C-1: the step's launches back to back) and of the attention
    launches, with the effective TFLOP/s they give."""
    step_fl = sum(p for r in range(C) for (p, _, _) in work[r]) * fl_pair
    last = 1 if fuse_merge == 2 else 2 * C - 1     # the fused form records events 0, 1 only
    spans = [ev[i][0][0].elapsed_time(ev[i][C - 1][last]) for i in range(steps)]
    launch = []                                   # (ms, flops) per attention launch
    for i in range(steps):
        for r in range(C):
            if fuse_merge == 2:
                launch.append((ev[i][r][0].elapsed_time(ev[i][r][1]),
                               sum(p for (p, _, _) in work[r]) * fl_pair))
            else:
                for s in range(C):
                    launch.append((ev[i][r][2 * s].elapsed_time(ev[i][r][2 * s + 1]),
                                   work[r][s][0] * fl_pair))
    tf = [f / (d / 1e3) / 1e12 for d, f in launch if d > 0]
    ms = [d for d, _ in launch]
    return {
        "step_span_ms_median": round(_median(spans), 4),
        "step_span_ms_min": round(min(spans), 4),
        "step_span_ms_max": round(max(spans), 4),
        "step_tflops_median": round(step_fl / (_median(spans) / 1e3) / 1e12, 2),
        "step_tflops_best": round(step_fl / (min(spans) / 1e3) / 1e12, 2),
        "launch_ms_median": round(_median(ms), 5),
        "launch_ms_min": round(min(ms), 5),
        "launch_ms_max": round(max(ms), 5),
        "launch_tflops_median": round(_median(tf), 2),
        "launch_tflops_best": round(max(tf), 2),
        "launch_tflops_worst": round(min(tf), 2),
    }


def per_block_pass(a, w, prob, work, fl_pair, torch, L):
    """The same step as one launch per ring block plus ra_lse_merge per history
    block (fuse_merge = 0): effective TFLOP/s of the diagonal (causal) launches
    and of the history (non-causal) launches, FLOP-weighted over all C^2
    launches, after the headline's timed steps."""
    C = w.cp
    bufs = [prob.alloc_forward(torch.bfloat16, 0) for _ in range(C)]
    stream = torch.cuda.current_stream()

    def run(events=None):
        for r in range(C):
            out, lse, ws = bufs[r]
            prob.forward(r, out, lse, ws, fuse_merge=0,
                         events=None if events is None else events[r])

    for _ in range(2):
        run()
    ev = []
    for _ in range(a.per_block_steps):
        e2 = []
        for _ in range(C):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * C)]
            for e in evs:
                e.record(stream)
            e2.append(evs)
        ev.append(e2)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(a.per_block_steps):
        run(ev[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / a.per_block_steps
    d_ms = h_ms = d_fl = h_fl = 0.0
    for i in range(a.per_block_steps):
        for r in range(C):
            for s in range(C):
                d = ev[i][r][2 * s].elapsed_time(ev[i][r][2 * s + 1])
                f = work[r][s][0] * fl_pair
                if s == 0:
                    d_ms += d
                    d_fl += f
                else:
                    h_ms += d
                    h_fl += f
    step_fl = sum(p for r in range(C) for (p, _, _) in work[r]) * fl_pair
    names = {L.ra_forward_kernel(prob.step_desc(0, j, c, qp, kp), qp)
             for (j, c, qp, kp) in prob.step_plan(0)}
    del bufs
    return {
        "fuse_merge": 0, "steps": a.per_block_steps, "kernel": "/".join(sorted(names)),
        "launches": a.per_block_steps * C * C,
        "diag_tflops": round(d_fl / (d_ms / 1e3) / 1e12, 2) if d_ms else None,
        "history_tflops": round(h_fl / (h_ms / 1e3) / 1e12, 2) if h_ms else None,
        "all_launches_tflops": round((d_fl + h_fl) / ((d_ms + h_ms) / 1e3) / 1e12, 2),
        "step_tflops": round(step_fl / (ms_step / 1e3) / 1e12, 2),
        "ms_per_step": round(ms_step, 4),
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU: every rank's share runs in turn "
                                   "on a single MI355X (the ring's KV exchange is not timed); "
                                   "run with --gpus 1"}))
        sys.exit(2)
    if a.copy_calibration_mib:
        copy_calibration(a.copy_calibration_mib)
        return
    if a.kernel != "auto":
        os.environ["RA_FWD_KERNEL"] = a.kernel
    else:
        os.environ.pop("RA_FWD_KERNEL", None)
    import numpy as np
    import torch
    import synth
    from context_blockwise_softmax_ra_amd import _lib as L
    from context_blockwise_softmax_ra_amd.ring import RingProblem

    w = synth.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.merge:
        print(json.dumps(bench_merge(a, w, torch, L)), flush=True)
        return
    if a.mfma_ceiling:
        print(json.dumps(bench_mfma_ceiling(a, w, torch, L)), flush=True)
        return
    print(f"# workload {w.name}: S={w.seqlen} CP={w.cp} hq={w.hq} hkv={w.hkv} "
          f"d={w.dqk}/{w.dv} {w.dtype}", file=sys.stderr, flush=True)
    q = synth.cast(w.q(), w.dtype).to(dev)
    k = synth.cast(w.k(), w.dtype).to(dev)
    v = synth.cast(w.v(), w.dtype).to(dev)
    prob = RingProblem(q, k, v, w.cu_global(), w.cp)
    if a.map is not None:
        res = bench_map(a, w, q, k, v, torch, L)
        print(json.dumps(res), flush=True)
        return
    if a.mode == "ulysses":
        res = bench_ulysses(a, w, q, k, v, torch, L)
        ring_work = [prob.work(r) for r in range(w.cp)]
        res["per_rank"]["ring_pairs_x_heads"] = [int(sum(p for p, _, _ in rw)) for rw in ring_work]
        res["per_rank"]["ring_tiles_visited"] = [int(sum(t for _, t, _ in rw)) for rw in ring_work]
        print(json.dumps(res), flush=True)
        return
    del q, k, v
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    C = w.cp
    if a.backward:
        return bench_backward(a, w, prob, torch, L)
    bufs = [prob.alloc_forward(torch.bfloat16, a.fuse_merge) for _ in range(C)]
    work = [prob.work(r) for r in range(C)]                      # per step (pairs*hq, ...)
    fl_pair = 2 * (w.dqk + w.dv)
    step_flops = sum(p for r in range(C) for (p, _, _) in work[r]) * fl_pair
    stream = torch.cuda.current_stream()

    def make_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)                                     # create the HIP events
        return evs

    def run_step(events=None):
        for r in range(C):
            out, lse, ws = bufs[r]
            prob.forward(r, out, lse, ws, fuse_merge=a.fuse_merge,
                         events=None if events is None else events[r])

    # The per-launch events of the second pass are created first: creating
    # and recording thousands of events idles the GPU for tens of ms, after
    # which the clock takes ~20 launches to settle, and an event recorded
    # between two launches leaves a ~10 us gap before the next one.  So the
    # timed steps run right after the warmup, back to back, bracketed by two
    # events only; every launch then starts as soon as the previous ends.
    ev = [[make_events(2 * C) for _ in range(C)] for _ in range(a.steps)]
    for _ in range(a.warmup):
        run_step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(a.steps):
        run_step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / a.steps
    print(f"# timed {a.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / a.steps:.3f})",
          file=sys.stderr, flush=True)

    # second pass, same steps with events around every attention launch:
    # per-launch and per-rank durations (median / min), diagonal vs history
    for _ in range(2):
        run_step()
    torch.cuda.synchronize()
    for i in range(a.steps):
        run_step(ev[i])
    torch.cuda.synchronize()
    attn_ms = 0.0
    attn_flops = 0.0
    diag_ms = hist_ms = 0.0
    diag_fl = hist_fl = 0.0
    n_launch = 0
    rank_ms = [0.0] * C
    for i in range(a.steps):
        for r in range(C):
            if a.fuse_merge == 2:                                # one launch per rank share
                d = ev[i][r][0].elapsed_time(ev[i][r][1])
                rank_ms[r] += d / a.steps
                attn_ms += d
                attn_flops += sum(p for (p, _, _) in work[r]) * fl_pair
                n_launch += 1
                continue
            for s in range(C):
                d = ev[i][r][2 * s].elapsed_time(ev[i][r][2 * s + 1])
                f = work[r][s][0] * fl_pair
                rank_ms[r] += d / a.steps
                attn_ms += d
                attn_flops += f
                n_launch += 1
                if s == 0:
                    diag_ms += d
                    diag_fl += f
                else:
                    hist_ms += d
                    hist_fl += f
    value = step_flops / (ms_step / 1e3) / 1e12
    if a.fuse_merge == 2:
        # the timed steps hold nothing but the C attention launches of each
        # step, back to back: the average launch takes the timed region over
        # the launch count (their dispatch gaps included)
        avg_launch_ms = ms_total / (a.steps * C)
        achieved = value
        evented_launch_ms = attn_ms / n_launch
    else:
        # per-block steps also run merges and casts: per-launch events
        avg_launch_ms = attn_ms / n_launch
        achieved = attn_flops / (attn_ms / 1e3) / 1e12
        evented_launch_ms = avg_launch_ms
    stats = launch_stats(ev, work, fl_pair, C, a.steps, a.fuse_merge)
    stats["evented_launch_ms_mean"] = round(evented_launch_ms, 5)
    if a.fuse_merge == 2:
        kname = L.ra_forward_kernel(prob.local_desc(0), L.PART_ALL)
    else:
        names = {L.ra_forward_kernel(prob.step_desc(0, j, c, qp, kp), qp)
                 for (j, c, qp, kp) in prob.step_plan(0)}
        kname = "/".join(sorted(names))
    traffic = traffic_for(w.name, kname) if a.fuse_merge == 2 else None

    res = {
        "metric": "effective attention TFLOP/s per rank-share (bf16) + % of MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*%g, bf16 RNE)" % w.mult,
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": f"{w.name}: causal attention, S={w.seqlen}, zig-zag CP={w.cp} "
                        f"(all {w.cp} rank shares forward, one after another), "
                        f"{w.hq} q heads / {w.hkv} kv heads, head dim {w.dqk}/{w.dv}",
            "seq_len": w.seqlen, "cp": w.cp, "hq": w.hq, "hkv": w.hkv, "dqk": w.dqk,
            "dv": w.dv, "fuse_merge": a.fuse_merge,
            "step_effective_tflop": round(step_flops / 1e12, 4),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": kname + (" (whole rank share per launch)" if a.fuse_merge == 2 else ""),
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(avg_launch_ms, 5),
            "launches": a.steps * C if a.fuse_merge == 2 else n_launch,
            "diag_tflops": round(diag_fl / (diag_ms / 1e3) / 1e12, 2) if diag_ms else None,
            "history_tflops": round(hist_fl / (hist_ms / 1e3) / 1e12, 2) if hist_ms else None,
        },
        "stats": stats,
        "per_rank": {
            "ms": [round(x, 4) for x in rank_ms],
            "pairs_x_heads": [int(sum(p for (p, _, _) in work[r])) for r in range(C)],
            "tflops": [round(sum(p for (p, _, _) in work[r]) * fl_pair / (rank_ms[r] / 1e3) / 1e12, 2)
                       for r in range(C)],
            "tiles_visited": [int(sum(t for (_, t, _) in work[r])) for r in range(C)],
            "tiles_skipped": [int(sum(t for (_, _, t) in work[r])) for r in range(C)],
            "slowest_rank": max(range(C), key=lambda r: rank_ms[r]),
            "time_max_over_mean": round(max(rank_ms) / (sum(rank_ms) / C), 4),
        },
        "cpu_baseline": None,
    }
    del bufs
    torch.cuda.empty_cache()
    if a.fuse_merge == 2 and a.per_block_steps > 0:
        res["per_block"] = per_block_pass(a, w, prob, work, fl_pair, torch, L)
    del prob
    torch.cuda.empty_cache()
    if a.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
