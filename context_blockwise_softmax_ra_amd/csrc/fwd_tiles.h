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

__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
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
