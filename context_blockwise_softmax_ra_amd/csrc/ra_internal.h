// Internal declarations shared by the host API and the HIP kernels of libra.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ra.h"

namespace ra {

// Geometry of the bf16 MFMA forward kernel: 4 waves x 32 query rows per
// workgroup, key tiles of 64.
constexpr int kFwdWaves = 4;
constexpr int kFwdRowsPerWave = 32;
constexpr int kFwdBlockM = kFwdWaves * kFwdRowsPerWave;  // 128
constexpr int kFwdBlockN = 64;

// fp32 forward kernel: one query row per lane, one wave per workgroup.
constexpr int kF32BlockM = 64;
constexpr int kF32BlockN = 32;

// Arguments of every attention kernel (forward and backward).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_stride, k_stride, v_stride;  // elements between tokens
  int32_t hq, hkv, group;                // group = hq / hkv
  int32_t n_seq;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const ra_segment* segs;  // rectangle list (segment-list launches), else NULL
  int32_t q_part, k_part;
  int32_t n_qtiles;       // query tiles per segment (max over segments)
  int32_t n_ktiles;       // key tiles per segment (max over segments; backward)
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
  int32_t total_q;        // lse / delta row stride
  // forward outputs (fp32): out [total_q, hq, dv], lse [hq, total_q]
  float* out;
  float* lse;
  // backward
  const void* dout;       // [total_q, hq, dv], same dtype as q
  const float* lse_in;    // final lse [hq, total_q]
  const float* delta;     // [hq, total_q]
  float* dq;              // [total_q, hq, dqk] fp32 accumulate
  float* dk;              // [total_k, hkv, dqk] fp32 accumulate
  float* dv;              // [total_k, hkv, dv] fp32 accumulate
  // dK/dV query split: qsplit workgroups share each key tile, each taking a
  // contiguous share of its (query head, query tile) iterations.  Share 0
  // adds into dk/dv; share s > 0 stores its scaled partial at dk_part /
  // dv_part + (s - 1) * part_keys rows (same row layout as dk/dv), which
  // bwd_qsplit_reduce then adds in share order.
  int32_t qsplit;
  int32_t part_keys;
  float* dk_part;
  float* dv_part;
  // dQ key split: ksplit workgroups share each query tile, dealing its key
  // tiles round-robin; share 0 adds into dq, share s > 0 stores its scaled
  // partial at dq_part + (s - 1) * total_q rows, which bwd_ksplit_reduce
  // adds in share order.
  int32_t ksplit;
  float* dq_part;
  // fused rank share on the ping-pong kernel: tile the two halves (zig-zag
  // chunks) of every segment separately, n_qtiles_half 256-row tiles per
  // segment at most
  int32_t half_tiles;
  int32_t n_qtiles_half;
};

// KV blocks of every owner for a rank's fused forward (one launch per rank).
constexpr int kMaxCp = 64;
constexpr int kMaxTileOrder = 512;  // tiles a packed share can order (kernel arguments)
struct RankKV {
  const void* k[kMaxCp];
  const void* v[kMaxCp];
  int32_t cp, rank;
  // KV split of a rank share (4-wave kernel): part p of `split` takes the
  // key tiles p, p + split, ... of the share's walk (all blocks in ring
  // order) and writes its float32 partial (out, lse) at out + p *
  // part_out_stride, lse + p * part_lse_stride (elements)
  int32_t split;
  int64_t part_out_stride, part_lse_stride;
  // rank-fused dK/dV launch: kv_tile_off[o] counts the 128-key tiles (with
  // a row that sees them) of the owners of ring steps before o, over all
  // segments; kv_tile_off[cp] tiles per kv head make up the grid, so no
  // workgroup lands past a short segment's keys
  int32_t kv_tile_off[kMaxCp + 1];
  // rank-fused dQ launch: 128-row query tiles of the local rows, segment by
  // segment (the grid per kv head, times the group and the key shares);
  // over packed segments taken in tile_order as the forward's tiles are.
  // The rank-fused dK/dV launch takes its live key tiles (kv_tile_off) in
  // tile_order if tile_ordered.
  int32_t q_tiles;
  // rank-fused forward over packed segments: fwd_tiles query tiles (256
  // rows on the ping-pong kernel, half tiles if AttnArgs::half_tiles; 128
  // on the 4-wave kernel) of all segments, listed segment by segment with
  // each segment's heaviest tile first.  tile_ordered 1: workgroup unit u
  // (all kv heads of one tile) takes tile tile_order[u] of that list (the
  // host's heaviest-first order); 2: the list takes the segments in the
  // order tile_order[0], tile_order[1], ... (heaviest first, for lists of
  // more tiles than the order holds); 0: unit u takes tile u
  int32_t fwd_tiles;
  int32_t tile_ordered;
  // Per-tile parts of a single sequence, tile_order[u] = query tile << 6 |
  // part << 3 | parts - 1 for unit u, heaviest part first:
  //  - forward KV split (4-wave kernel): fwd_tiles units per head; split is
  //    then the number of partial slots, and part 0 of a tile sets
  //    lse = -inf in the slots past its tile's parts;
  //  - rank-fused dQ key shares: q_tiles units per head; the share
  //    reduction takes each tile's count from TileShares.
  int32_t var_split;
  uint16_t tile_order[kMaxTileOrder];
};

// dK / dV accumulators of every owner for a rank's fused backward (one
// dK/dV launch over all owners' key tiles).
struct RankGrad {
  float* dk[kMaxCp];
  float* dv[kMaxCp];
};

// The block of `owner` in `rank`'s share of a ring of the zig-zag placement:
// its own block is causal over all rows and keys; an earlier owner's block
// is seen whole by every row through its first key half only; a later
// owner's block is seen by the second row half only, over all its keys.
// (Derived from the global causal rule: the owner's first chunk precedes
// both of the rank's chunks, its second chunk follows both, and both chunks
// of a later owner lie between the rank's two.)
__host__ __device__ inline void owner_plan(int rank, int owner, int* causal, int* q_part,
                                           int* k_part) {
  if (owner == rank) {
    *causal = 1;
    *q_part = RA_PART_ALL;
    *k_part = RA_PART_ALL;
  } else if (owner < rank) {
    *causal = 0;
    *q_part = RA_PART_ALL;
    *k_part = RA_PART_FIRST_HALF;
  } else {
    *causal = 0;
    *q_part = RA_PART_SECOND_HALF;
    *k_part = RA_PART_ALL;
  }
}

// Segment part [lo, hi) after applying a zig-zag half selector.
__host__ __device__ inline void part_range(int32_t s0, int32_t s1, int32_t part, int32_t* lo,
                                           int32_t* hi) {
  int32_t half = (s1 - s0) >> 1;
  if (part == RA_PART_FIRST_HALF) {
    *lo = s0;
    *hi = s0 + half;
  } else if (part == RA_PART_SECOND_HALF) {
    *lo = s0 + half;
    *hi = s1;
  } else {
    *lo = s0;
    *hi = s1;
  }
}

// Launchers (return hipError_t of the launch).
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                                hipStream_t st);
hipError_t launch_rank_fwd_bf16(const AttnArgs& a, const RankKV& rk, int dqk, int dv,
                                bool out_bf16, hipStream_t st);
hipError_t launch_attn_fwd_segments(const AttnArgs& a, int dqk, int dv, bool merge,
                                    hipStream_t st);
hipError_t launch_gather_tokens(const void* src, void* dst, int64_t row_bytes,
                                const int32_t* tokens, int32_t n, bool gather, hipStream_t st);
hipError_t launch_attn_fwd_pp(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                              hipStream_t st);
hipError_t launch_rank_fwd_pp(const AttnArgs& a, const RankKV& rk, int dqk, int dv,
                              bool out_bf16, hipStream_t st);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                               hipStream_t st);
hipError_t launch_lse_merge(float* out_acc, float* lse_acc, const float* out_part,
                            const float* lse_part, int32_t total_t, int32_t h, int32_t dv,
                            int32_t n_seq, const int32_t* cu, int32_t part, int32_t max_rows,
                            hipStream_t st);
hipError_t launch_cast_f32_bf16(const float* src, void* dst, int64_t n, hipStream_t st);
// out/lse of a row-head = lse-weighted sum of `split` float32 partials
// (part p at part_out + p * part_out_stride, part_lse + p * part_lse_stride,
// elements); out has out_dtype.
hipError_t launch_split_combine(const float* part_out, const float* part_lse, int split,
                                int64_t part_out_stride, int64_t part_lse_stride, void* out,
                                ra_dtype out_dtype, float* lse, int32_t total_t, int32_t h,
                                int32_t dv, hipStream_t st);
hipError_t launch_zigzag_copy(const void* src, void* dst, int64_t row_bytes, int32_t n_seq,
                              const int32_t* cu_local, const int32_t* src_start,
                              int32_t max_half, bool gather, hipStream_t st);
hipError_t launch_bwd_delta(const void* out, int out_dtype, const void* dout, int dout_dtype,
                            int32_t total_t, int32_t hq, int32_t dv, float* delta,
                            hipStream_t st);
hipError_t launch_attn_bwd_bf16(const AttnArgs& a, int dqk, int dv, bool causal, bool kv_split,
                                int total_k, hipStream_t st);
// A rank's whole backward share in two launches: dK/dV over every owner's
// key tiles (each with the owner's plan, into rg's accumulators), and dQ
// with every query tile walking all owners' key tiles in ring order (dealt
// over a.ksplit workgroups, partials reduced in share order).  a describes
// the rank's local rows (q, dout, lse, delta, dq; parts ALL); rk the
// owners' K/V blocks.
// Key shares per 128-row query tile of a single-sequence rank-fused dQ
// launch (var = 1): the reduction adds shares 1 .. n[tile] - 1.
struct TileShares {
  int32_t var;
  uint8_t n[kMaxTileOrder];
};

hipError_t launch_rank_bwd_bf16(const AttnArgs& a, const RankKV& rk_kv, const RankKV& rk_q,
                                const RankGrad& rg, const TileShares& ts, int dqk, int dv,
                                hipStream_t st);

// Sets the thread-local message ra_last_error() returns and passes st back.
ra_status set_error(ra_status st, const char* fmt, ...);

}  // namespace ra
