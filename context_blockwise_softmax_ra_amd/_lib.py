"""ctypes binding of libra.so: the C-ABI entry points under the same names.

Argument marshalling only: tensors are passed as ``data_ptr()`` device
pointers with torch's current HIP stream; every computation happens in the
library's HIP kernels.  There is no fallback: if libra.so is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_int64,
                    c_size_t, c_void_p)
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP = 0, 1, 2, 3
RA_BF16, RA_FP32 = 0, 1
PART_ALL, PART_FIRST_HALF, PART_SECOND_HALF = 0, 1, 2

_STATUS = {0: "RA_OK", 1: "RA_ERR_INVALID_ARG", 2: "RA_ERR_UNSUPPORTED", 3: "RA_ERR_HIP"}

# Every symbol include/ra.h declares.
EXPORTS = (
    "ra_block_attn_fwd", "ra_block_attn_fwd_merge", "ra_lse_merge", "ra_zigzag_shard_map",
    "ra_zigzag_gather", "ra_zigzag_scatter", "ra_cast_f32_bf16", "ra_rank_forward_workspace",
    "ra_rank_forward", "ra_rank_forward_noalloc", "ra_attn_bwd_delta", "ra_block_attn_bwd", "ra_rank_backward_workspace",
    "ra_rank_backward", "ra_block_attn_work", "ra_forward_kernel", "ra_shard_tokens",
    "ra_step_segments", "ra_gather_tokens", "ra_scatter_tokens", "ra_block_attn_fwd_segments",
    "ra_segments_work", "ra_mfma_ceiling", "ra_last_error", "ra_version",
)

# ra_map values by name (the oracle's names for the same placements)
MAPS = {"zigzag": 0, "zigzag_global": 1, "striped": 2, "contiguous": 3}


class RaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class AttnDesc(Structure):
    _fields_ = [
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p),
        ("dtype", c_int),
        ("hq", c_int32), ("hkv", c_int32), ("dqk", c_int32), ("dv", c_int32),
        ("q_stride_tok", c_int64), ("k_stride_tok", c_int64), ("v_stride_tok", c_int64),
        ("n_seq", c_int32),
        ("cu_seqlens_q", c_void_p), ("cu_seqlens_k", c_void_p),
        ("cu_seqlens_q_host", c_void_p), ("cu_seqlens_k_host", c_void_p),
        ("q_part", c_int), ("k_part", c_int),
        ("causal", c_int32),
        ("softmax_scale", c_float),
    ]


class RankDesc(Structure):
    _fields_ = [
        ("local", AttnDesc),
        ("cp_size", c_int32), ("rank", c_int32),
        ("k_blocks", c_void_p), ("v_blocks", c_void_p),
        ("out", c_void_p), ("out_dtype", c_int),
        ("lse", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("fuse_merge", c_int32),
        ("events", c_void_p),
    ]


class RankBwdDesc(Structure):
    _fields_ = [
        ("local", AttnDesc),
        ("cp_size", c_int32), ("rank", c_int32),
        ("k_blocks", c_void_p), ("v_blocks", c_void_p),
        ("out", c_void_p), ("out_dtype", c_int),
        ("dout", c_void_p),
        ("lse", c_void_p),
        ("dq", c_void_p),
        ("dk_blocks", c_void_p), ("dv_blocks", c_void_p),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
        ("events", c_void_p),
    ]


_lib = None


def lib():
    """The loaded libra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built: run "
                              "`python -m context_blockwise_softmax_ra_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name in EXPORTS:
            getattr(L, name)  # every declared symbol must be exported
        vp = c_void_p
        sig = {
            "ra_block_attn_fwd": [POINTER(AttnDesc), vp, vp, vp],
            "ra_block_attn_fwd_merge": [POINTER(AttnDesc), vp, vp, vp],
            "ra_lse_merge": [vp, vp, vp, vp, c_int32, c_int32, c_int32, c_int32, vp, vp, c_int, vp],
            "ra_zigzag_shard_map": [c_int32, c_int32, c_int32, vp, vp, vp],
            "ra_zigzag_gather": [vp, vp, c_int64, c_int32, vp, vp, vp, vp, c_int32, vp],
            "ra_zigzag_scatter": [vp, vp, c_int64, c_int32, vp, vp, vp, vp, c_int32, vp],
            "ra_cast_f32_bf16": [vp, vp, c_int64, vp],
            "ra_rank_forward_workspace": [POINTER(RankDesc), POINTER(c_size_t)],
            "ra_rank_forward": [POINTER(RankDesc), vp],
            "ra_rank_forward_noalloc": [POINTER(RankDesc), vp],
            "ra_attn_bwd_delta": [vp, c_int, vp, c_int, c_int32, c_int32, c_int32, vp, vp],
            "ra_block_attn_bwd": [POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp],
            "ra_rank_backward_workspace": [POINTER(RankBwdDesc), POINTER(c_size_t)],
            "ra_rank_backward": [POINTER(RankBwdDesc), vp],
            "ra_block_attn_work": [POINTER(AttnDesc), POINTER(c_int64), POINTER(c_int64),
                                   POINTER(c_int64)],
            "ra_shard_tokens": [c_int, c_int32, c_int32, c_int32, vp, vp, c_int32, vp],
            "ra_step_segments": [c_int, c_int32, c_int32, c_int32, c_int32, vp, vp, c_int32, vp],
            "ra_gather_tokens": [vp, vp, c_int64, c_int32, vp, vp, c_int32, vp],
            "ra_scatter_tokens": [vp, vp, c_int64, c_int32, vp, vp, c_int32, vp],
            "ra_block_attn_fwd_segments": [POINTER(AttnDesc), c_int32, vp, vp, vp, vp, c_int32,
                                           vp],
            "ra_segments_work": [vp, c_int32, c_int32, POINTER(c_int64), POINTER(c_int64),
                                 POINTER(c_int64)],
            "ra_mfma_ceiling": [vp, c_int64, vp, c_int64, c_int32, c_int32, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = c_int
        L.ra_forward_kernel.argtypes = [POINTER(AttnDesc), c_int]
        L.ra_forward_kernel.restype = c_char_p
        L.ra_last_error.argtypes = []
        L.ra_last_error.restype = c_char_p
        L.ra_version.argtypes = []
        L.ra_version.restype = c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != RA_OK:
        raise RaError(status, lib().ra_last_error().decode())


def _ptr(t, token_strided: bool = False) -> Optional[int]:
    """Address of a buffer; tensors must be dense (the C ABI takes no strides).

    ``token_strided``: a [tokens, heads, dim] tensor whose token stride is
    passed separately; heads and dim must still be packed.
    """
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("host array must be C-contiguous")
        return t.ctypes.data
    if token_strided:
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"[tokens, heads, dim] tensor needs packed heads/dim, got "
                             f"shape {tuple(t.shape)} strides {t.stride()}")
    elif not t.is_contiguous():
        raise ValueError(f"tensor must be contiguous, got shape {tuple(t.shape)} strides "
                         f"{t.stride()}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def attn_desc(q, k, v, cu_q, cu_k, cu_q_host, cu_k_host, *, q_part=PART_ALL,
              k_part=PART_ALL, causal=False, scale=0.0, dtype=None) -> AttnDesc:
    """Build an ``ra_attn_desc`` from [T, H, D] tensors and int32 cu_seqlens.

    q/k/v may be None (e.g. the k/v of a rank-level descriptor).  cu_*_host
    are copied to int32 NumPy arrays kept alive by the returned object.
    """
    ref = q if q is not None else k
    d = AttnDesc()
    d.q, d.k, d.v = _ptr(q, True), _ptr(k, True), _ptr(v, True)
    d.dtype = _dtype_code(ref) if dtype is None else dtype
    d.hq = q.shape[1] if q is not None else 0
    d.hkv = k.shape[1] if k is not None else d.hq
    d.dqk = q.shape[2] if q is not None else k.shape[2]
    d.dv = v.shape[2] if v is not None else d.dqk
    d.q_stride_tok = q.stride(0) if q is not None else 0
    d.k_stride_tok = k.stride(0) if k is not None else 0
    d.v_stride_tok = v.stride(0) if v is not None else 0
    hq_, hk_ = _host_i32(cu_q_host), _host_i32(cu_k_host)
    d.n_seq = len(hq_) - 1
    d.cu_seqlens_q, d.cu_seqlens_k = _ptr(cu_q), _ptr(cu_k)
    d.cu_seqlens_q_host, d.cu_seqlens_k_host = hq_.ctypes.data, hk_.ctypes.data
    d.q_part, d.k_part = int(q_part), int(k_part)
    d.causal = 1 if causal else 0
    d.softmax_scale = float(scale)
    d._keep = (q, k, v, cu_q, cu_k, hq_, hk_)
    return d


def rank_desc(local: AttnDesc, cp_size: int, rank: int, k_blocks: Sequence, v_blocks: Sequence,
              out, lse, workspace=None, fuse_merge=False, events=None) -> RankDesc:
    # blocks take the local descriptor's token strides (head slices allowed)
    kb = (c_void_p * cp_size)(*[_ptr(t, True) for t in k_blocks])
    vb = (c_void_p * cp_size)(*[_ptr(t, True) for t in v_blocks])
    r = RankDesc()
    r.local = local
    r.cp_size, r.rank = cp_size, rank
    r.k_blocks = ctypes.cast(kb, c_void_p)
    r.v_blocks = ctypes.cast(vb, c_void_p)
    r.out = _ptr(out)
    r.out_dtype = _dtype_code(out)
    r.lse = _ptr(lse)
    r.workspace = _ptr(workspace) if workspace is not None else None
    r.workspace_bytes = (workspace.numel() * workspace.element_size()) if workspace is not None else 0
    r.fuse_merge = int(fuse_merge)
    ev = None
    if events is not None:
        ev = (c_void_p * len(events))(*[e if isinstance(e, int) else (e.cuda_event if e is not None else None)
                                         for e in events])
        r.events = ctypes.cast(ev, c_void_p)
    else:
        r.events = None
    r._keep = (local, k_blocks, v_blocks, kb, vb, out, lse, workspace, ev, events)
    return r


def rank_bwd_desc(local: AttnDesc, cp_size: int, rank: int, k_blocks, v_blocks, out, dout, lse,
                  dq, dk_blocks, dv_blocks, workspace=None, events=None) -> RankBwdDesc:
    # blocks take the local descriptor's token strides (head slices allowed)
    kb = (c_void_p * cp_size)(*[_ptr(t, True) for t in k_blocks])
    vb = (c_void_p * cp_size)(*[_ptr(t, True) for t in v_blocks])
    gk = (c_void_p * cp_size)(*[_ptr(t) for t in dk_blocks])
    gv = (c_void_p * cp_size)(*[_ptr(t) for t in dv_blocks])
    r = RankBwdDesc()
    r.local = local
    r.cp_size, r.rank = cp_size, rank
    r.k_blocks = ctypes.cast(kb, c_void_p)
    r.v_blocks = ctypes.cast(vb, c_void_p)
    r.out = _ptr(out)
    r.out_dtype = _dtype_code(out)
    r.dout = _ptr(dout)
    r.lse = _ptr(lse)
    r.dq = _ptr(dq)
    r.dk_blocks = ctypes.cast(gk, c_void_p)
    r.dv_blocks = ctypes.cast(gv, c_void_p)
    r.workspace = _ptr(workspace) if workspace is not None else None
    r.workspace_bytes = (workspace.numel() * workspace.element_size()) if workspace is not None else 0
    ev = None
    if events is not None:
        ev = (c_void_p * len(events))(*[e.cuda_event if hasattr(e, "cuda_event") else e for e in events])
        r.events = ctypes.cast(ev, c_void_p)
    else:
        r.events = None
    r._keep = (local, k_blocks, v_blocks, kb, vb, gk, gv, out, dout, lse, dq, dk_blocks,
               dv_blocks, workspace, ev, events)
    return r


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def ra_block_attn_fwd(desc: AttnDesc, out, lse, stream=None):
    _check(lib().ra_block_attn_fwd(ctypes.byref(desc), _ptr(out), _ptr(lse), _stream(stream)))


def ra_block_attn_fwd_merge(desc: AttnDesc, out_acc, lse_acc, stream=None):
    _check(lib().ra_block_attn_fwd_merge(ctypes.byref(desc), _ptr(out_acc), _ptr(lse_acc),
                                         _stream(stream)))


def ra_lse_merge(out_acc, lse_acc, out_part, lse_part, cu, cu_host, rows=PART_ALL, stream=None):
    T, H, DV = out_acc.shape
    ch = _host_i32(cu_host)
    _check(lib().ra_lse_merge(_ptr(out_acc), _ptr(lse_acc), _ptr(out_part), _ptr(lse_part),
                              T, H, DV, len(ch) - 1, _ptr(cu), ch.ctypes.data, int(rows),
                              _stream(stream)))


def ra_zigzag_shard_map(cp_size: int, rank: int, cu_global):
    """Host map: (cu_seqlens_local int32[n+1], src_start int32[2n])."""
    cg = _host_i32(cu_global)
    n = len(cg) - 1
    cl = np.zeros(n + 1, dtype=np.int32)
    ss = np.zeros(max(1, 2 * n), dtype=np.int32)
    _check(lib().ra_zigzag_shard_map(cp_size, rank, n, cg.ctypes.data, cl.ctypes.data,
                                     ss.ctypes.data))
    return cl, ss[:2 * n]


def ra_zigzag_gather(global_src, local_dst, cu_local, src_start, cu_local_host, src_start_host,
                     stream=None):
    ch, sh = _host_i32(cu_local_host), _host_i32(src_start_host)
    row_bytes = global_src[0].numel() * global_src.element_size()
    _check(lib().ra_zigzag_gather(_ptr(global_src), _ptr(local_dst), row_bytes, len(ch) - 1,
                                  _ptr(cu_local), _ptr(src_start), ch.ctypes.data, sh.ctypes.data,
                                  global_src.shape[0], _stream(stream)))


def ra_zigzag_scatter(local_src, global_dst, cu_local, src_start, cu_local_host, src_start_host,
                      stream=None):
    ch, sh = _host_i32(cu_local_host), _host_i32(src_start_host)
    row_bytes = global_dst[0].numel() * global_dst.element_size()
    _check(lib().ra_zigzag_scatter(_ptr(local_src), _ptr(global_dst), row_bytes, len(ch) - 1,
                                   _ptr(cu_local), _ptr(src_start), ch.ctypes.data,
                                   sh.ctypes.data, global_dst.shape[0], _stream(stream)))


def ra_cast_f32_bf16(src, dst, stream=None):
    _check(lib().ra_cast_f32_bf16(_ptr(src), _ptr(dst), src.numel(), _stream(stream)))


def ra_rank_forward_workspace(desc: RankDesc) -> int:
    n = c_size_t(0)
    _check(lib().ra_rank_forward_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ra_rank_forward(desc: RankDesc, stream=None):
    _check(lib().ra_rank_forward(ctypes.byref(desc), _stream(stream)))


RA_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/ra.h


def ra_rank_forward_noalloc(desc: RankDesc, stream=None):
    """ra_rank_forward with the library's fixed scratch as workspace (the
    descriptor's workspace fields are ignored)."""
    _check(lib().ra_rank_forward_noalloc(ctypes.byref(desc), _stream(stream)))


def ra_attn_bwd_delta(out, dout, delta, stream=None):
    T, H, DV = out.shape
    _check(lib().ra_attn_bwd_delta(_ptr(out), _dtype_code(out), _ptr(dout), _dtype_code(dout),
                                   T, H, DV, _ptr(delta), _stream(stream)))


def ra_block_attn_bwd(desc: AttnDesc, dout, lse, delta, dq_acc, dk_acc, dv_acc, stream=None):
    _check(lib().ra_block_attn_bwd(ctypes.byref(desc), _ptr(dout), _ptr(lse), _ptr(delta),
                                   _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _stream(stream)))


def ra_rank_backward_workspace(desc: RankBwdDesc) -> int:
    n = c_size_t(0)
    _check(lib().ra_rank_backward_workspace(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ra_rank_backward(desc: RankBwdDesc, stream=None):
    _check(lib().ra_rank_backward(ctypes.byref(desc), _stream(stream)))


def ra_block_attn_work(desc: AttnDesc):
    """(visible_pairs, tiles_visited, tiles_skipped) of one block descriptor."""
    a, b, c = c_int64(0), c_int64(0), c_int64(0)
    _check(lib().ra_block_attn_work(ctypes.byref(desc), ctypes.byref(a), ctypes.byref(b),
                                    ctypes.byref(c)))
    return a.value, b.value, c.value


def _map_code(kind) -> int:
    return MAPS[kind] if isinstance(kind, str) else int(kind)


def ra_shard_tokens(kind, cp_size: int, rank: int, cu_seqlens_global) -> np.ndarray:
    """Global token of each local row of ``rank`` under a shard map (int32)."""
    cu = _host_i32(cu_seqlens_global)
    cap = max(int(cu[-1]) // max(cp_size, 1), 1)
    out = np.zeros(cap, np.int32)
    n = c_int32(0)
    _check(lib().ra_shard_tokens(_map_code(kind), cp_size, rank, len(cu) - 1, cu.ctypes.data,
                                 out.ctypes.data, cap, ctypes.byref(n)))
    return out[:n.value].copy()


def ra_step_segments(kind, cp_size: int, rank: int, owner: int, cu_seqlens_global) -> np.ndarray:
    """Rectangles [n, 5] int32 (q_lo, q_hi, k_lo, k_hi, diag) of one ring step."""
    cu = _host_i32(cu_seqlens_global)
    cap = 2 * (len(cu) - 1) + 2
    out = np.zeros((cap, 5), np.int32)
    n = c_int32(0)
    _check(lib().ra_step_segments(_map_code(kind), cp_size, rank, owner, len(cu) - 1,
                                  cu.ctypes.data, out.ctypes.data, cap, ctypes.byref(n)))
    return out[:n.value].copy()


def ra_gather_tokens(src, dst, tokens_dev, tokens_host, stream=None):
    """dst[i] = src[tokens[i]] for [T, ...] row buffers."""
    th = np.ascontiguousarray(tokens_host, np.int32)
    rb = src[0].numel() * src.element_size()
    _check(lib().ra_gather_tokens(_ptr(src), _ptr(dst), rb, src.shape[0], _ptr(tokens_dev),
                                  th.ctypes.data, len(th), _stream(stream)))


def ra_scatter_tokens(src, dst, tokens_dev, tokens_host, stream=None):
    """dst[tokens[i]] = src[i] for [T, ...] row buffers."""
    th = np.ascontiguousarray(tokens_host, np.int32)
    rb = src[0].numel() * src.element_size()
    _check(lib().ra_scatter_tokens(_ptr(src), _ptr(dst), rb, dst.shape[0], _ptr(tokens_dev),
                                   th.ctypes.data, len(th), _stream(stream)))


def ra_block_attn_fwd_segments(desc: AttnDesc, segs_dev, segs_host, out, lse, merge=False,
                               stream=None):
    sh = np.ascontiguousarray(segs_host, np.int32).reshape(-1, 5)
    _check(lib().ra_block_attn_fwd_segments(ctypes.byref(desc), len(sh), _ptr(segs_dev),
                                            sh.ctypes.data, _ptr(out), _ptr(lse), 1 if merge else 0,
                                            _stream(stream)))


def ra_segments_work(segs_host, hq: int):
    """(visible_pairs, tiles_visited, tiles_skipped) of a rectangle list."""
    sh = np.ascontiguousarray(segs_host, np.int32).reshape(-1, 5)
    a, b, c = c_int64(0), c_int64(0), c_int64(0)
    _check(lib().ra_segments_work(sh.ctypes.data, len(sh), hq, ctypes.byref(a), ctypes.byref(b),
                                  ctypes.byref(c)))
    return a.value, b.value, c.value


def ra_forward_kernel(desc: AttnDesc, q_part: int = PART_ALL) -> str:
    """Name of the forward kernel a launch over q_part of ``desc`` uses."""
    r = lib().ra_forward_kernel(ctypes.byref(desc), q_part)
    if r is None:
        raise RaError(1, lib().ra_last_error().decode())
    return r.decode()


def ra_mfma_ceiling(operands, out, n_workgroups: int, iters: int, stream=None):
    """Pure v_mfma_f32_32x32x16_bf16 loop on the given bf16 operands (a
    measurement helper); out holds n_workgroups x 256 floats."""
    _check(lib().ra_mfma_ceiling(_ptr(operands), operands.numel() * operands.element_size(),
                                 _ptr(out), out.numel(), n_workgroups, iters, _stream(stream)))


def ra_last_error() -> str:
    return lib().ra_last_error().decode()


def ra_version() -> str:
    return lib().ra_version().decode()
