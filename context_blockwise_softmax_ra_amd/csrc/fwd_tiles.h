// K/V tile geometry, LDS layouts and direct global->LDS tile loads shared by
// the bf16 forward attention kernels.
//
// A key tile holds BN = 64 keys.  K and V go from global memory straight into
// LDS (global_load_lds_dwordx4: each wave instruction fills 1 KiB of LDS,
// lane i writing bytes 16i..16i+15).  Because the LDS destination of a lane is
// fixed, bank spreading is done by choosing which global 16-byte chunk each
// lane fetches (an XOR swizzle), with 64 banks x 4 bytes in mind:
//   K: 64-dim panels of 128-byte rows, chunk slot = chunk ^ ((row>>1)&7);
//      the 16 rows a 128-bit read serves at once land on 16 distinct slots.
//   V: 256-byte rows, chunk slot = chunk ^ (((row&3)<<2)|((row>>2)&3)); the
//      4 rows x 64 bytes of one transposing read land on 16 distinct slots.
#pragma once

#include "mfma_common.h"

namespace ra {
namespace fwd {

using namespace mfma;

constexpr int BN = kFwdBlockN;

template <int DQK, int DV>
struct Geo {
  static constexpr int KPANELS = DQK / 64;               // 64-dim panels of K
  static constexpr int KPANEL_BYTES = BN * 128;
  static constexpr int K_BYTES = KPANELS * KPANEL_BYTES;
  static constexpr int VROWB = DV * 2;                   // 256 (DV=128) or 128 (DV=64)
  static constexpr int V_BYTES = BN * VROWB;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int K_INST = K_BYTES / 1024;          // wave instructions per K tile
  static constexpr int V_INST = V_BYTES / 1024;
  static constexpr int KK = DQK / 16;                    // MFMA k-steps for S
  static constexpr int OT = DV / 32;                     // output tiles per wave
  static_assert(DV == 128 || DV == 64, "V layouts");
};

__device__ __forceinline__ int k_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

// V chunk slot: 256-byte rows use the dual swizzle; 128-byte rows flip the
// 64-byte half on alternate row pairs.
template <int VROWB>
__device__ __forceinline__ int v_slot(int row, int c) {
  return VROWB == 256 ? (c ^ swz(row)) : (c ^ (((row >> 1) & 1) << 2));
}

template <int VROWB>
__device__ __forceinline__ int v_off(int row, int byte) {
  return row * VROWB + (v_slot<VROWB>(row, byte >> 4) << 4) + (byte & 15);
}

// One wave's share (of NW waves) of the direct global->LDS loads of a K/V
// tile: per instruction a per-lane byte offset (fixed for the whole launch)
// from the tile's first key row, and a wave-uniform LDS destination.  K and V
// may go to separate LDS buffers.
template <int DQK, int DV, int NW>
struct TileLoader {
  using G = Geo<DQK, DV>;
  static_assert(G::K_INST % NW == 0 && G::V_INST % NW == 0, "tile load split");
  static constexpr int KI = G::K_INST / NW, VI = G::V_INST / NW;
  static constexpr int VCH = G::VROWB / 16, RPI = 1024 / G::VROWB;
  uint32_t koff[KI], voff[VI];  // byte offsets from the tile's first key row
  int wave, lane;

  __device__ __forceinline__ int krow(int jj) const { return ((wave + NW * jj) % (BN / 8)) * 8 + (lane >> 3); }
  __device__ __forceinline__ int kcol(int jj) const {
    return ((wave + NW * jj) / (BN / 8) * 64 + k_slot(krow(jj), lane & 7) * 8) * 2;  // XOR involution
  }
  __device__ __forceinline__ int kdst(int jj) const {
    const int j = wave + NW * jj;
    return j / (BN / 8) * G::KPANEL_BYTES + (j % (BN / 8)) * 1024;
  }
  __device__ __forceinline__ int vrow(int jj) const { return (wave + NW * jj) * RPI + lane / VCH; }
  __device__ __forceinline__ int vcol(int jj) const { return v_slot<G::VROWB>(vrow(jj), lane % VCH) * 16; }
  __device__ __forceinline__ int vdst(int jj) const { return (wave + NW * jj) * 1024; }

  __device__ __forceinline__ void init(int64_t ks_bytes, int64_t vs_bytes, int w, int l) {
    wave = w;
    lane = l;
#pragma unroll
    for (int jj = 0; jj < KI; ++jj) koff[jj] = (uint32_t)(krow(jj) * ks_bytes + kcol(jj));
#pragma unroll
    for (int jj = 0; jj < VI; ++jj) voff[jj] = (uint32_t)(vrow(jj) * vs_bytes + vcol(jj));
  }

  // rows_left: key rows available from the tile's first row on (only the
  // last tile of a block is clamped)
  __device__ __forceinline__ void issue_k(const char* kt, int64_t ks_bytes, int rows_left,
                                          char* kdst_base) const {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(kt);
    if (rows_left >= BN) {
#pragma unroll
      for (int jj = 0; jj < KI; ++jj) g2lds(r, koff[jj], kdst_base + kdst(jj));
    } else {
#pragma unroll
      for (int jj = 0; jj < KI; ++jj)
        g2lds(r, (uint32_t)(min(krow(jj), rows_left - 1) * ks_bytes + kcol(jj)), kdst_base + kdst(jj));
    }
  }
  __device__ __forceinline__ void issue_v(const char* vt, int64_t vs_bytes, int rows_left,
                                          char* vdst_base) const {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(vt);
    if (rows_left >= BN) {
#pragma unroll
      for (int jj = 0; jj < VI; ++jj) g2lds(r, voff[jj], vdst_base + vdst(jj));
    } else {
#pragma unroll
      for (int jj = 0; jj < VI; ++jj)
        g2lds(r, (uint32_t)(min(vrow(jj), rows_left - 1) * vs_bytes + vcol(jj)), vdst_base + vdst(jj));
    }
  }
};

// Masks the 32 scores of a lane in a 64-key S tile: entry i of C tile hh is
// key offset e = 32*hh + 16*(i/8) + (i%8) past the lane's first key (the
// tile's first key plus 8*(lane/32)), and is kept iff e <= lim.  The caller
// folds every masking rule of the lane's row into the one limit, so each
// score costs a compare against an inline constant and a select.
__device__ __forceinline__ void mask_scores(mfma::f32x16& s0, mfma::f32x16& s1, int lim) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = ((i >> 3) << 4) + (i & 7);
    s0[i] = e <= lim ? s0[i] : -INFINITY;
    s1[i] = e + 32 <= lim ? s1[i] : -INFINITY;
  }
}

// In-lane maximum of the 32 scores a lane holds of a 64-key S tile (the
// lane's query row, one half of the keys), as two left-folded fmaxf chains:
// the backend fuses those into v_max3_f32 (two scores per instruction),
// while a chain of three-way maxima gets re-associated into pairwise
// v_max_f32 (three instructions per four scores).  The softmax shares its
// SIMD's vector issue with the matrix-core products of the other wave
// there, so the instruction count matters.
__device__ __forceinline__ float lane_max32(const mfma::f32x16& s0, const mfma::f32x16& s1) {
  float a = __builtin_fmaxf(s0[0], s0[1]);
  float b = __builtin_fmaxf(s1[0], s1[1]);
#pragma unroll
  for (int i = 2; i < 16; ++i) {
    a = __builtin_fmaxf(a, s0[i]);
    b = __builtin_fmaxf(b, s1[i]);
  }
  return __builtin_fmaxf(a, b);
}

// P operand of a lane's 32 scores against the offset mc (the running max
// times c2): p = 2^(c2 * s - mc), rounded to bf16 into p[4] (key order of
// the P^T operand: entries 8bb..8bb+7 of the pair (s0, s1) make p[bb]).
// Returns the float32 sum of the unrounded values; s is left intact.
__device__ __forceinline__ float exp2_pack_sum(const mfma::f32x16& s0, const mfma::f32x16& s1,
                                               float c2, float mc, mfma::bf16x8 (&p)[4]) {
  float a = 0.f, b = 0.f;
  mfma::u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    const float x0 = __builtin_amdgcn_exp2f(fmaf(i < 16 ? s0[i & 15] : s1[i & 15], c2, -mc));
    const float x1 = __builtin_amdgcn_exp2f(fmaf(i < 16 ? s0[(i & 15) + 1] : s1[(i & 15) + 1], c2, -mc));
    a = i == 0 ? x0 : a + x0;
    b = i == 0 ? x1 : b + x1;
    w[i >> 3][(i >> 1) & 3] = mfma::pack_bf16x2(x0, x1);
  }
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) p[bb] = mfma::as_bf16x8(w[bb]);
  return a + b;
}

// Online softmax of one 64-key S tile for the lane's query row (log2
// domain; scores s, c2 = softmax scale * log2(e)).  The running max m_run
// is raised lazily: only when a score exceeds it by more than 2^8 in
// probability.  The numerator, the row sum l_run and the lse all use the
// same (possibly stale) max, so the result is exact.
//
// The probabilities are first taken against the running max.  A lane whose
// 32 of them sum to at most 2^8 has none above 2^8, so no raise is due for
// it; only when some lane exceeds that (or has no finite max yet, as on a
// row's first tile) are the row maximum and the raise worked out, and P
// recomputed if the max moved.  This keeps the row-max reduction out of
// the common tile and reaches the same state as testing the max first.
template <int OT>
__device__ __forceinline__ void online_softmax_tile(const mfma::f32x16& s0, const mfma::f32x16& s1,
                                                    float c2, float& m_run, float& l_run,
                                                    mfma::f32x16 (&o)[OT], mfma::bf16x8 (&p)[4]) {
  constexpr float kRescaleLog2 = 8.0f;
  constexpr float kSumBound = 256.0f;  // 2^kRescaleLog2
  const bool all_finite = !__builtin_amdgcn_ballot_w64(m_run == -INFINITY);
  float ts = 0.f;
  if (all_finite) ts = exp2_pack_sum(s0, s1, c2, m_run * c2, p);
  if (!all_finite || __builtin_amdgcn_ballot_w64(!(ts <= kSumBound))) {
    const float mx = mfma::xhalf_max(lane_max32(s0, s1));
    const bool raise = (mx - m_run) * c2 > kRescaleLog2;  // true on a row's first live tile
    const bool any_raise = __builtin_amdgcn_ballot_w64(raise) != 0;
    if (any_raise) {
      const float m_new = raise ? mx : m_run;
      const float m_use_new = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_use_new) * c2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int tt = 0; tt < OT; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[tt][i] *= alpha;
    }
    if (any_raise || !all_finite) {
      const float mc = ((m_run == -INFINITY) ? 0.f : m_run) * c2;
      ts = exp2_pack_sum(s0, s1, c2, mc, p);
    }
  }
  l_run += ts;
}

// How a KV block meets the rows of a workgroup.
enum BlockKind {
  KIND_CAUSAL = 0,     // key j visible to row i iff j <= i + diag (part-relative)
  KIND_ALL = 1,        // every key visible
  KIND_LATE_ROWS = 2,  // every key visible to rows of the segment's second half only
};

struct Block {
  const char* kb;  // K of the block's first key (this kv head)
  const char* vb;
  int klen;
  int kind;
  int diag;        // KIND_CAUSAL: diagonal offset (0 except for rectangle lists)
  int ntiles;
};

}  // namespace fwd
}  // namespace ra
