"""Build libra.so (HIP kernels for gfx950 + the C-ABI host code) in-tree.

    python -m context_blockwise_softmax_ra_amd.build [-j N]

Every source under csrc/ is compiled by hipcc for gfx950 into _build/ and
linked into context_blockwise_softmax_ra_amd/libra.so.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libra.so")
ARCH = os.environ.get("RA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          # keep the compiler from emitting packed fp32 VALU ops
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") or f.endswith(".cpp"):
            out.append(os.path.join(CSRC, f))
    return out


# Per-file flags.  The attention kernels take row maxima of matrix-core
# outputs; without this, IEEE-mode fmaxf canonicalises every operand first
# (one extra v_max_f32 per score).  NaN inputs still propagate to NaN outputs.
# The backward kernels run one wave per SIMD with large accumulators, which
# live in the AGPR half of the register file (the compiler's default MFMA
# form): with the tiles loaded straight into LDS that measured faster than
# forcing MFMA results into VGPRs.
PER_FILE = {
    "attn_fwd_bf16.hip": ["-fno-honor-nans"],
    "attn_fwd_pp.hip": ["-fno-honor-nans"],
    "attn_bwd_bf16.hip": ["-fno-honor-nans"],
}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + PER_FILE.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return src, obj, r.returncode, "\n".join(lines)


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = []
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for src, obj, rc, log in ex.map(_compile, srcs):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{log}")
            if verbose and log.strip():
                print(log)
            objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.v))
    sys.exit(0)
