// Device helpers shared by the bf16 attention kernels (forward and backward).
//
// Matrix-core layout used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand (M x K = 32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B operand (K x N = 16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   C/D (32 x 32 fp32, 16 per lane): lane l holds column l%32 and rows
//       8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
#pragma once

#include "ra_internal.h"

namespace ra {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x4 lds16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// Two floats -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// 8 accumulator entries [i0, i0+8) of a C tile as a bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int i0) {
  u32x4 u;
  u[0] = pack_bf16x2(c[i0 + 0], c[i0 + 1]);
  u[1] = pack_bf16x2(c[i0 + 2], c[i0 + 3]);
  u[2] = pack_bf16x2(c[i0 + 4], c[i0 + 5]);
  u[3] = pack_bf16x2(c[i0 + 6], c[i0 + 7]);
  return as_bf16x8(u);
}

// Value exchange with lane l^32 (v_permlane32_swap).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row fed as A-operand row mm so that C entries 8j..8j+7 of a lane are 8
// consecutive rows of that operand: entry i of lane l is row
// 16*(i/8) + 8*(l/32) + i%8.
__device__ __forceinline__ int sigma(int mm) {
  const int g = (mm >> 2) & 1;
  const int i = ((mm >> 3) << 2) | (mm & 3);
  return ((i >> 3) << 4) | (g << 3) | (i & 7);
}

// Item r (0-based) of a list in which segment s = 0, 1, ... holds count(s)
// items, for grids that list only the live tiles of packed segments.  Each
// wave scans 64 segments at a time (a prefix sum over its lanes, then the
// first lane past r); the results are wave-uniform: the segment, the item's
// index in it and the segment's count.  Returns false if r is past the end.
template <class Count>
__device__ __forceinline__ bool locate_in_segments(int n_seq, int r, Count count, int* seg,
                                                   int* idx, int* cnt) {
  const int lane = threadIdx.x & 63;
  for (int base = 0; base < n_seq; base += 64) {
    const int s = base + lane;
    const int t = s < n_seq ? count(s) : 0;
    int inc = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(inc, d, 64);
      if (lane >= d) inc += u;
    }
    const unsigned long long hit = __ballot(inc > r);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      *seg = __builtin_amdgcn_readfirstlane(base + f);
      *idx = __builtin_amdgcn_readfirstlane(r - __shfl(inc - t, f, 64));
      *cnt = __builtin_amdgcn_readfirstlane(__shfl(t, f, 64));
      return true;
    }
    r = __builtin_amdgcn_readfirstlane(r - __shfl(inc, 63, 64));
  }
  return false;
}

// Blocks are dispatched round-robin over the 8 XCDs (b % 8); give each XCD
// a contiguous range of logical tiles so neighbours share its L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Causal launches: query tiles differ in work (later rows see more keys), so
// contiguous ranges per XCD would leave one XCD with all the heavy tiles.
// Deal units of g consecutive logical tiles (the query heads of one kv
// group, which read the same K/V) round-robin over the 8 XCDs instead; each
// XCD then runs light and heavy units alike, in logical (heaviest-first)
// order.  The last partial round of 8*g blocks keeps the identity.
__device__ __forceinline__ int xcd_deal(int b, int nb, int g) {
  const int round = 8 * g;
  const int full = nb / round * round;
  if (b >= full) return b;
  const int x = b & 7, j = b >> 3;
  return (j / g) * round + x * g + (j % g);
}

// Buffer resource over the rows of one tile (gfx9 descriptor word 3).  The
// record count is never the limit: every offset stays within one tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

// 16 (or 4) bytes per lane from the tile at byte offset voff into LDS (lane i
// writes lds + 16i, or lds + 4i).  The buffer form (buffer_load ... lds) is
// used rather than global_load_lds: the compiler treats an outstanding
// global (FLAT) load into LDS as an out-of-order LDS access and then drains
// every LDS read before its first use, which serialises the operand reads.
__device__ __forceinline__ void g2lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           0, 0, 0);
}
__device__ __forceinline__ void g2lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff,
                                           0, 0, 0);
}

// Orders the instructions of a block of NM matrix-core products, each fed by
// RPM LDS reads, so that the reads run AHEAD products ahead of the products
// that consume them (the machine scheduler otherwise tends to issue each
// read right before its product and wait for it).  Call after the code of
// the block, inside the same basic block.
template <int NM, int RPM, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma() {
  static_assert(AHEAD <= NM, "read-ahead beyond the block");
  __builtin_amdgcn_sched_group_barrier(0x100, RPM * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < NM - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// The same for a block of N1 products fed by R1 reads each followed by N2
// products fed by R2 reads each.
template <int N1, int R1, int N2, int R2, int AHEAD>
__device__ __forceinline__ void pipeline_lds_mfma_n() {
  static_assert(AHEAD <= N1 && AHEAD <= N2, "read-ahead beyond the block");
  __builtin_amdgcn_sched_group_barrier(0x100, R1 * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N1 - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R1, 0);
  }
#pragma unroll
  for (int i = 0; i < N2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// As pipeline_lds_mfma, with up to VPM vector-ALU instructions placed after
// each product: independent vector work of the same wave (a softmax the
// products do not feed) then issues while the matrix core runs.
template <int NM, int RPM, int AHEAD, int VPM>
__device__ __forceinline__ void pipeline_lds_mfma_valu() {
  static_assert(AHEAD <= NM, "read-ahead beyond the block");
  __builtin_amdgcn_sched_group_barrier(0x100, RPM * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NM - AHEAD) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
  }
}

// Keeps the computation of v ahead of this point: an empty asm statement
// that reads it.  Without it the compiler sinks work whose result is used
// only after a branch into the block past the branch, away from the
// products it was scheduled beside.
__device__ __forceinline__ void keep_here(const bf16x8& v) { asm volatile("" : : "v"(v)); }

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane i receives element i%4 of the 8 bytes addressed by lane 4r + i/4,
// r = 0..3.
__device__ __forceinline__ s16x4 lds_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ bf16x8 cat_tr(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// "Dual" LDS tile layout for tiles read both by 128-bit row reads (16 rows
// at one 16-byte chunk) and by transposing reads (4 consecutive rows x 64
// bytes): rows of ROWB = 256 or 512 bytes, 16-byte chunks XOR-swizzled by
// swz(row) within each 256-byte half.  Both patterns then touch 16
// distinct chunk slots of the 64 banks.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <int ROWB>
__device__ __forceinline__ int dual_off(int row, int byte) {
  return row * ROWB + ((((byte >> 4) ^ swz(row))) << 4) + (byte & 15);
}

// One wave's share (of NW waves) of the direct global->LDS loads of a
// [ROWS x DIM] bf16 tile into the dual layout with ROWB-byte rows.
// Instruction j fills LDS bytes [1024 j, 1024 j + 1024); lane i writes the 16
// bytes at 1024 j + 16 i, i.e. row (1024 j + 16 i) / ROWB at slot s, and
// fetches the global chunk the swizzle maps to slot s (s ^ swz(row), an
// involution within each 256-byte half).  Chunks past DIM (row padding up to
// ROWB) fetch a chunk of the first half instead; they are never read.
template <int ROWS, int DIM, int ROWB, int NW>
struct DualLoader {
  static constexpr int INST = ROWS * ROWB / 1024;
  static_assert(INST % NW == 0 && DIM >= 128, "tile load split");
  static constexpr int PER = INST / NW;
  uint32_t off[PER];  // byte offset of the fetched chunk from the tile's first row
  int wave, lane;

  __device__ __forceinline__ int row(int jj) const { return ((wave + NW * jj) * 1024 + 16 * lane) / ROWB; }
  __device__ __forceinline__ int colb(int jj) const {
    const int slot = (((wave + NW * jj) * 1024 + 16 * lane) % ROWB) >> 4;
    const int c = slot ^ swz(row(jj));
    return (c * 16 < DIM * 2 ? c : (c & 15)) * 16;
  }
  __device__ __forceinline__ void init(int64_t row_stride_bytes, int w, int l) {
    wave = w;
    lane = l;
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) off[jj] = (uint32_t)(row(jj) * row_stride_bytes + colb(jj));
  }
  // rows_left: rows available from the tile's first row on (the last tile of
  // a range is clamped to its last row)
  __device__ __forceinline__ void issue(const void* base, int64_t row_stride_bytes, int rows_left,
                                        char* lds) const {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base);
    if (rows_left >= ROWS) {
#pragma unroll
      for (int jj = 0; jj < PER; ++jj) g2lds(r, off[jj], lds + (wave + NW * jj) * 1024);
    } else {
#pragma unroll
      for (int jj = 0; jj < PER; ++jj)
        g2lds(r, (uint32_t)(min(row(jj), rows_left - 1) * row_stride_bytes + colb(jj)),
              lds + (wave + NW * jj) * 1024);
    }
  }
};

// Byte column, within a 32-column tile of 16-bit elements, that lane
// addresses in a transposing read: 16*((lane/16)%2) + 4*(lane%4) elements.
__device__ __forceinline__ int tr_col_bytes(int lane) {
  return (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
}
// Row, within the 16-row k-step, that lane addresses in a transposing read
// for k = 8*(lane/32) .. +3 (add 4 for the next 4).
__device__ __forceinline__ int tr_row(int lane) { return 8 * (lane >> 5) + ((lane & 15) >> 2); }

}  // namespace mfma
}  // namespace ra
