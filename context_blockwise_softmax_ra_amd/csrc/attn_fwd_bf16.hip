// Block attention forward, bfloat16 inputs, float32 accumulation, on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// What one launch computes (the per-block (out, lse) of the block loop in
// "超长序列并行训练技术：Ulysses与Ring-Attention详解", section 4.1): for every
// segment, query head and query row of the selected part, softmax attention
// over the keys of the selected part of the same segment (all of them, or
// j <= i when causal), written either as a partial (out, lse) or merged
// into a running (out, lse) with the lse rule of section 4.2.
//
// Work decomposition
//   workgroup = (segment, query tile of 128 rows, query head); 4 waves, each
//   owning 32 query rows; the key loop walks 64-key tiles of the segment
//   part, skipping tiles that are entirely masked (causal upper triangle,
//   beyond the part) -- they are never loaded.
//
// Per wave and key tile (all on the matrix cores, fp32 accumulate):
//   S^T[64 keys x 32 rows] = K_tile * Q^T        (A = K rows from LDS,
//                                                 B = Q held in registers)
//   O^T[dv x 32 rows]     += V_tile^T * P^T      (A = V^T from LDS,
//                                                 B = P straight from the
//                                                 S^T accumulator)
// The 32x32 accumulator gives lane l the column l%32, i.e. one query row,
// and 16 of the 32 keys (the other 16 sit in lane l^32).  Row max and row
// sum are therefore in-lane reductions plus one exchange with lane l^32,
// and the running output rescale is a per-lane scalar multiply.
//
// K rows are fed to the S^T product in a permuted order sigma so that the
// 8 accumulator values a lane feeds as one B operand of the P*V product are
// 8 consecutive keys.  V stays row-major in LDS and the V^T operand is read
// with the gfx950 transposing LDS read (ds_read_b64_tr_b16): within each
// 16-lane group, lane i receives element i%4 of the 8 bytes addressed by
// lanes 4r + i/4, r = 0..3, so lanes pointing at 4 consecutive key rows
// hand every lane 4 consecutive keys of one dim.
//
// LDS banking (64 banks x 4 bytes; a 128-bit access serves 16 lanes at a
// time, a 64-bit access 32): K rows are padded to an odd number of 16-byte
// slots, so the 16 rows read together land on 16 distinct slots; V rows
// are padded to a stride of 64 mod 256 bytes, so the 4 rows x 64 bytes one
// transposing read touches cover all 64 banks once.
//
// Blocks are remapped so that each of the 8 XCDs gets a contiguous range of
// tiles ordered (segment, kv head, query tile, head in group): the query
// heads sharing a kv head, and neighbouring query tiles, read the same K/V
// through the same L2.  Causal launches order query tiles heaviest first.

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kFwdBlockM;
constexpr int BN = kFwdBlockN;
constexpr int NT = kFwdWaves * 64;

__device__ __forceinline__ int xcd_remap(int b, int nb) {
  // Hardware places block b on XCD b % 8.  Hand XCD x the logical range
  // [x*q + min(x, r), ...) so consecutive logical tiles share an L2.
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Key row fed by accumulator row mm so that accumulator entries
// 8j..8j+7 of a lane hold 8 consecutive keys (see file comment).
__device__ __forceinline__ int sigma(int mm) {
  const int g = (mm >> 2) & 1;
  const int i = ((mm >> 3) << 2) | (mm & 3);
  return ((i >> 3) << 4) | (g << 3) | (i & 7);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// max / sum of a value and its copy in lane l^32 (v_permlane32_swap).
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

// Rescale threshold (log2 units): the running max used for the exponent is
// only raised when a row's max grows by more than this, so the output
// rescale is skipped on most tiles.  Exact: numerator, row sum and lse all
// use the same (possibly stale) max; p stays <= 2^8.
constexpr float kRescaleLog2 = 8.0f;

template <int DQK, int DV>
struct Geo {
  static constexpr int KCH = DQK / 8;                 // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;                  // 16-byte chunks per V row
  static constexpr int KSTR = DQK * 2 + 16;           // odd number of 16-byte slots
  static constexpr int VSTR = DV * 2 + 64;            // 64 mod 256 bytes
  static constexpr int K_BYTES = BN * KSTR;
  static constexpr int V_BYTES = BN * VSTR;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int NBUF = (2 * STAGE <= 81920) ? 2 : 1;
  static constexpr int K_LD = (BN * KCH) / NT;        // K chunks per thread
  static constexpr int V_LD = (BN * VCH) / NT;        // V chunks per thread
  static constexpr int KK = DQK / 16;                 // MFMA k-steps for S
  static constexpr int OT = DV / 32;                  // output tiles per wave
  static_assert((BN * KCH) % NT == 0 && (BN * VCH) % NT == 0, "tile load split");
  static_assert(((KSTR / 16) & 1) == 1 && (VSTR % 256) == 64 || (DV == 64 && VSTR == 192),
                "bank spread");
};

template <int DQK, int DV>
struct Prefetch {
  u32x4 k[Geo<DQK, DV>::K_LD];
  u32x4 v[Geo<DQK, DV>::V_LD];
};

template <int DQK, int DV>
__device__ __forceinline__ void load_tile(Prefetch<DQK, DV>& pf, const __bf16* __restrict__ kb,
                                          const __bf16* __restrict__ vb, int64_t ks, int64_t vs,
                                          int key0, int k_last, int tid) {
  using G = Geo<DQK, DV>;
#pragma unroll
  for (int i = 0; i < G::K_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::KCH, c = idx % G::KCH;
    const int tok = min(key0 + row, k_last);
    pf.k[i] = ldg16(kb + (int64_t)tok * ks + c * 8);
  }
#pragma unroll
  for (int i = 0; i < G::V_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::VCH, c = idx % G::VCH;
    const int tok = min(key0 + row, k_last);
    pf.v[i] = ldg16(vb + (int64_t)tok * vs + c * 8);
  }
}

template <int DQK, int DV>
__device__ __forceinline__ void store_tile(const Prefetch<DQK, DV>& pf, char* stage, int tid) {
  using G = Geo<DQK, DV>;
  char* ks = stage;
  char* vs = stage + G::K_BYTES;
#pragma unroll
  for (int i = 0; i < G::K_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::KCH, c = idx % G::KCH;
    *reinterpret_cast<u32x4*>(ks + row * G::KSTR + (c << 4)) = pf.k[i];
  }
#pragma unroll
  for (int i = 0; i < G::V_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::VCH, c = idx % G::VCH;
    *reinterpret_cast<u32x4*>(vs + row * G::VSTR + (c << 4)) = pf.v[i];
  }
}

template <int DQK, int DV, bool CAUSAL, bool MERGE>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  using G = Geo<DQK, DV>;
  __shared__ __attribute__((aligned(16))) char smem[G::NBUF * G::STAGE];

  const int nb = gridDim.x;
  int b = xcd_remap(blockIdx.x, nb);
  const int group = a.group;
  const int hg = b % group;
  b /= group;
  const int qt_rev = b % a.n_qtiles;
  b /= a.n_qtiles;
  const int kvh = b % a.hkv;
  const int seg = b / a.hkv;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - qt_rev) : qt_rev;
  const int h = kvh * group + hg;

  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], a.q_part, &q_lo, &q_hi);
  part_range(a.cu_k[seg], a.cu_k[seg + 1], a.k_part, &k_lo, &k_hi);
  const int q0 = q_lo + qt * BM;
  if (q0 >= q_hi) return;
  const int klen = k_hi - k_lo;
  if (klen <= 0 && MERGE) return;  // merging an empty block is the identity

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // key range of the whole workgroup
  const int qrel_last_wg = min(q0 + BM, q_hi) - 1 - q_lo;
  const int kend = CAUSAL ? min(klen, qrel_last_wg + 1) : klen;
  const int ntiles = (kend + BN - 1) / BN;

  // this wave's rows
  const int wq0 = q0 + wave * kFwdRowsPerWave;        // first row of the wave
  const bool wave_live = wq0 < q_hi;
  const int wq_first_rel = wq0 - q_lo;
  const int wq_last_rel = min(wq0 + kFwdRowsPerWave, q_hi) - 1 - q_lo;
  const int wave_kend = CAUSAL ? min(klen, wq_last_rel + 1) : klen;
  const int my_row = wq0 + l32;                        // query token of this lane
  const int my_row_rel = my_row - q_lo;

  const __bf16* __restrict__ qb = reinterpret_cast<const __bf16*>(a.q) + (int64_t)h * DQK;
  const __bf16* __restrict__ kb = reinterpret_cast<const __bf16*>(a.k) + (int64_t)kvh * DQK;
  const __bf16* __restrict__ vb = reinterpret_cast<const __bf16*>(a.v) + (int64_t)kvh * DV;

  // Q^T operand: lane holds row my_row, dims 16*kk + 8*g .. +7
  bf16x8 qf[G::KK];
  {
    const int row = min(my_row, q_hi - 1);
    const __bf16* qp = qb + (int64_t)row * a.q_stride + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) qf[kk] = as_bf16x8(ldg16(qp + 16 * kk));
  }

  f32x16 o[G::OT];
#pragma unroll
  for (int t = 0; t < G::OT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  float m_run = -INFINITY;  // running max of raw scores
  float l_run = 0.f;        // running sum of this lane's 16-key halves
  const float c2 = a.scale_log2;

  const int k_last = k_hi - 1;
  const int krow_a = sigma(l32);
  // transposing-read address of this lane: key row 8g + (lane%16)/4, dims
  // 16*((lane/16)%2) + 4*(lane%4) (+32 per output tile, +4 rows for keys 4..7)
  const int v_row = 8 * g + ((lane & 15) >> 2);
  const int v_col = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  Prefetch<DQK, DV> pf;
  if (ntiles > 0) {
    load_tile<DQK, DV>(pf, kb, vb, a.k_stride, a.v_stride, k_lo, k_last, tid);
    store_tile<DQK, DV>(pf, smem, tid);
    if (ntiles > 1)
      load_tile<DQK, DV>(pf, kb, vb, a.k_stride, a.v_stride, k_lo + BN, k_last, tid);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const char* stage = smem + (G::NBUF == 2 ? (t & 1) * G::STAGE : 0);
    const int kt0 = t * BN;  // relative to k_lo
    if (wave_live && kt0 < wave_kend) {
      const char* ks = stage;
      const char* vsm = stage + G::K_BYTES;
      // ---- S^T = K * Q^T : two 32-key halves
      f32x16 s[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[hh][i] = 0.f;
        const char* rp = ks + (krow_a + 32 * hh) * G::KSTR + (g << 4);
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
          const u32x4 kv = *reinterpret_cast<const u32x4*>(rp + (kk << 5));
          s[hh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qf[kk], s[hh], 0, 0, 0);
        }
      }
      // ---- mask (only tiles that cross the causal diagonal or the part end)
      const bool need_mask = (kt0 + BN > wave_kend) || (CAUSAL && kt0 + BN - 1 > wq_first_rel);
      if (need_mask) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kr = kt0 + 32 * hh + ((i >> 3) << 4) + (g << 3) + (i & 7);
            const bool ok = (kr < klen) && (!CAUSAL || kr <= my_row_rel);
            if (!ok) s[hh][i] = -INFINITY;
          }
      }
      // ---- online softmax (log2 domain, lazily rescaled)
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[0][i], s[0][i + 1]));
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(s[1][i], s[1][i + 1]));
      mx = xhalf_max(mx);
      // raise the running max only if it grew by more than the threshold
      const bool raise = (mx - m_run) * c2 > kRescaleLog2;   // true on the first live tile
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float m_new = raise ? mx : m_run;
        const float m_use_new = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use_new) * c2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int tt = 0; tt < G::OT; ++tt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[tt][i] *= alpha;
      }
      const float mc = ((m_run == -INFINITY) ? 0.f : m_run) * c2;
      float rs = 0.f;
      unsigned pk[16];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[hh][i], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[hh][i + 1], c2, -mc));
          rs += p0 + p1;
          pk[hh * 8 + (i >> 1)] = pack_bf16x2(p0, p1);
        }
      l_run += rs;
      // ---- O^T += V^T * P^T : 4 k-steps of 16 keys
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        u32x4 pv;
        pv[0] = pk[4 * bb + 0];
        pv[1] = pk[4 * bb + 1];
        pv[2] = pk[4 * bb + 2];
        pv[3] = pk[4 * bb + 3];
        const bf16x8 pb = as_bf16x8(pv);
        // V^T operand: keys 16bb + 8g + 0..7 of dim 32tt + l32, two transposing reads
        const char* vp = vsm + (16 * bb + v_row) * G::VSTR + v_col;
#pragma unroll
        for (int tt = 0; tt < G::OT; ++tt) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 64 * tt));
          const s16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 4 * G::VSTR + 64 * tt));
          const bf16x8 va = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[tt], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) {
      if (G::NBUF == 1) __syncthreads();
      store_tile<DQK, DV>(pf, smem + (G::NBUF == 2 ? ((t + 1) & 1) * G::STAGE : 0), tid);
      __syncthreads();
      if (t + 2 < ntiles)
        load_tile<DQK, DV>(pf, kb, vb, a.k_stride, a.v_stride, k_lo + (t + 2) * BN, k_last, tid);
    }
  }

  if (!wave_live || my_row >= q_hi) return;

  // ---- epilogue: lanes l and l^32 hold the two key halves of the same row
  const float l_tot = xhalf_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
  const float lse = empty ? -INFINITY : (m_fin * a.scale + __builtin_amdgcn_logf(l_tot) * 0.69314718055994531f);

  float* orow = a.out + ((int64_t)my_row * a.hq + h) * DV;
  float* lrow = a.lse + (int64_t)h * a.total_q + my_row;
  if (!MERGE) {
#pragma unroll
    for (int tt = 0; tt < G::OT; ++tt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 val;
        val.x = o[tt][4 * q4 + 0] * inv;
        val.y = o[tt][4 * q4 + 1] * inv;
        val.z = o[tt][4 * q4 + 2] * inv;
        val.w = o[tt][4 * q4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + 32 * tt + 8 * q4 + 4 * g) = val;
      }
    if (g == 0) *lrow = lse;
  } else {
    const float la = *lrow;
    const float mm = fmaxf(la, lse);
    const bool both_empty = (mm == -INFINITY);
    const float ms = both_empty ? 0.f : mm;
    const float wa = __expf(la - ms), wb = __expf(lse - ms);
    const float tot = wa + wb;
    const float ca = both_empty ? 0.f : wa / tot;
    const float cb = both_empty ? 0.f : wb / tot * inv;
    const float lnew = both_empty ? -INFINITY : ms + __logf(tot);
#pragma unroll
    for (int tt = 0; tt < G::OT; ++tt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4* p = reinterpret_cast<float4*>(orow + 32 * tt + 8 * q4 + 4 * g);
        float4 acc = *p;
        acc.x = ca * acc.x + cb * o[tt][4 * q4 + 0];
        acc.y = ca * acc.y + cb * o[tt][4 * q4 + 1];
        acc.z = ca * acc.z + cb * o[tt][4 * q4 + 2];
        acc.w = ca * acc.w + cb * o[tt][4 * q4 + 3];
        *p = acc;
      }
    if (g == 0) *lrow = lnew;
  }
}

template <int DQK, int DV>
hipError_t launch_t(const AttnArgs& a, bool causal, bool merge, hipStream_t st) {
  const long long nblk = (long long)a.n_seq * a.hkv * a.n_qtiles * a.group;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nblk), block(NT);
  if (causal) {
    if (merge) hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, true, false>), grid, block, 0, st, a);
  } else {
    if (merge) hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                                hipStream_t st) {
  if (dqk == 128 && dv == 128) return launch_t<128, 128>(a, causal, merge, st);
  if (dqk == 192 && dv == 128) return launch_t<192, 128>(a, causal, merge, st);
  if (dqk == 64 && dv == 64) return launch_t<64, 64>(a, causal, merge, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
