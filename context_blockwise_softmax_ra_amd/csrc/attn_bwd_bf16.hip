// Block attention backward, bfloat16 inputs, float32 accumulation, on the
// gfx950 matrix cores.  The probabilities are recomputed from the saved
// final lse instead of being stored ("超长序列并行训练技术：Ulysses与
// Ring-Attention详解", section 4.3):
//   P_ij = exp(scale q_i.k_j - lse_i)        (final lse over every key i sees)
//   dV_j += sum_i P_ij dout_i
//   dS_ij = P_ij (dout_i . v_j - delta_i)     delta_i = dout_i . out_i
//   dQ_i += scale sum_j dS_ij k_j
//   dK_j += scale sum_i dS_ij q_i
// over the visible pairs of one block (segments, halves and the causal rule
// exactly as in the forward).  Two launches, no atomics, deterministic:
//
// dK/dV kernel -- workgroup = 128 keys of one kv head (4 waves x 32 keys).
//   K and V of the wave's keys stay in registers; the loop walks every
//   query head of the kv group and every 32-row query tile of the segment
//   part (causal: only tiles at or below the keys).  Per tile, with lane l
//   owning key column l%32 of the 32x32 accumulators:
//     S  = Q K^T, dP = dO V^T        A = Q / dO rows from LDS, B = K / V regs
//     dV += P^T dO, dK += dS^T Q     A = P^T / dS^T straight from the S / dP
//                                    accumulators (query rows fed in the
//                                    permuted order sigma so 8 consecutive
//                                    entries are 8 consecutive rows),
//                                    B = dO / Q via transposing LDS reads.
// dQ kernel -- workgroup = 128 query rows of one head (4 waves x 32 rows),
//   the forward's shape: lane l owns query row l%32; per 64-key tile
//     S^T = K Q^T, dP^T = V dO^T     A = K / V rows from LDS (sigma order),
//                                    B = Q / dO held in registers
//     dQ^T += K^T dS^T               A = K via transposing LDS reads.
// Q, dO and K tiles are read both by 128-bit row reads and by transposing
// reads, so they use the XOR-swizzled "dual" LDS layout (conflict-free for
// both, see mfma_common.h).

#include "mfma_common.h"

namespace ra {
namespace {

using namespace mfma;

constexpr int NT = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float lse_log2(const float* lse, int64_t i, bool valid) {
  // rows outside the part (or that see nothing) contribute P = 0
  if (!valid) return INFINITY;
  const float l = lse[i];
  return l == -INFINITY ? INFINITY : l * kLog2e;
}

// ===========================================================================
// dK / dV
// ===========================================================================
constexpr int KV_BN = 128;  // keys per workgroup
constexpr int KV_BQ = 32;   // query rows per iteration

template <int DQK, int DV>
struct GeoKV {
  static constexpr int QROWB = DQK <= 128 ? 256 : 512;
  static constexpr int OROWB = 256;
  static constexpr int Q_BYTES = KV_BQ * QROWB;
  static constexpr int O_BYTES = KV_BQ * OROWB;
  static constexpr int STAGE = Q_BYTES + O_BYTES + 2 * KV_BQ * 4;
  static constexpr int QCH = DQK / 8, OCH = DV / 8;
  static constexpr int Q_LD = KV_BQ * QCH / NT;
  static constexpr int O_LD = KV_BQ * OCH / NT;
  static constexpr int KK = DQK / 16, VK = DV / 16;
  static constexpr int NQT = DQK / 32, NVT = DV / 32;
  static_assert(KV_BQ * QCH % NT == 0 && KV_BQ * OCH % NT == 0, "tile split");
  static_assert(DV == 128, "dO rows are 256 bytes");
};

template <int DQK, int DV>
struct PfKV {
  u32x4 q[GeoKV<DQK, DV>::Q_LD];
  u32x4 o[GeoKV<DQK, DV>::O_LD];
  float ld;  // lse*log2e (threads 0..31) or delta (threads 32..63)
};

template <int DQK, int DV>
__device__ __forceinline__ void kv_load(PfKV<DQK, DV>& pf, const AttnArgs& a, int h, int q0,
                                        int q_hi, int tid) {
  using G = GeoKV<DQK, DV>;
  const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + (int64_t)h * DQK;
  const __bf16* ob = reinterpret_cast<const __bf16*>(a.dout) + (int64_t)h * DV;
#pragma unroll
  for (int i = 0; i < G::Q_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::QCH, c = idx % G::QCH;
    const int tok = min(q0 + row, q_hi - 1);
    pf.q[i] = ldg16(qb + (int64_t)tok * a.q_stride + c * 8);
  }
#pragma unroll
  for (int i = 0; i < G::O_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::OCH, c = idx % G::OCH;
    const int tok = min(q0 + row, q_hi - 1);
    pf.o[i] = ldg16(ob + (int64_t)tok * ((int64_t)a.hq * DV) + c * 8);
  }
  if (tid < 2 * KV_BQ) {
    const int row = tid & (KV_BQ - 1);
    const int tok = q0 + row;
    const bool valid = tok < q_hi;
    const int64_t i = (int64_t)h * a.total_q + (valid ? tok : 0);
    pf.ld = tid < KV_BQ ? lse_log2(a.lse_in, i, valid) : (valid ? a.delta[i] : 0.f);
  }
}

template <int DQK, int DV>
__device__ __forceinline__ void kv_store(const PfKV<DQK, DV>& pf, char* st, int tid) {
  using G = GeoKV<DQK, DV>;
#pragma unroll
  for (int i = 0; i < G::Q_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::QCH, c = idx % G::QCH;
    *reinterpret_cast<u32x4*>(st + dual_off<G::QROWB>(row, c * 16)) = pf.q[i];
  }
#pragma unroll
  for (int i = 0; i < G::O_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::OCH, c = idx % G::OCH;
    *reinterpret_cast<u32x4*>(st + G::Q_BYTES + dual_off<G::OROWB>(row, c * 16)) = pf.o[i];
  }
  if (tid < 2 * KV_BQ) reinterpret_cast<float*>(st + G::Q_BYTES + G::O_BYTES)[tid] = pf.ld;
}

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(NT, 1) void attn_bwd_dkdv_kernel(AttnArgs a) {
  using G = GeoKV<DQK, DV>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE];

  int b = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = b % a.n_ktiles;
  b /= a.n_ktiles;
  const int kvh = b % a.hkv;
  const int seg = b / a.hkv;

  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], a.q_part, &q_lo, &q_hi);
  part_range(a.cu_k[seg], a.cu_k[seg + 1], a.k_part, &k_lo, &k_hi);
  const int k0 = k_lo + kt * KV_BN;
  const int qlen = q_hi - q_lo, klen = k_hi - k_lo;
  if (k0 >= k_hi || qlen <= 0) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wk_rel = kt * KV_BN + wave * 32;        // first key of the wave (part-relative)
  const bool wave_live = wk_rel < klen;
  const int my_key_rel = wk_rel + l32;               // this lane's key column
  const int my_key = min(k_lo + my_key_rel, k_hi - 1);

  // K, V of this lane's key as B operands (k = dims 16kk + 8g .. +7)
  bf16x8 kf[G::KK], vf[G::VK];
  {
    const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + (int64_t)my_key * a.k_stride +
                       (int64_t)kvh * DQK + 8 * g;
    const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + (int64_t)my_key * a.v_stride +
                       (int64_t)kvh * DV + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) kf[kk] = as_bf16x8(ldg16(kp + 16 * kk));
#pragma unroll
    for (int kk = 0; kk < G::VK; ++kk) vf[kk] = as_bf16x8(ldg16(vp + 16 * kk));
  }
  f32x16 dk[G::NQT], dv[G::NVT];
#pragma unroll
  for (int t = 0; t < G::NQT; ++t) dk[t] = zero16();
#pragma unroll
  for (int t = 0; t < G::NVT; ++t) dv[t] = zero16();

  const int n_qt = (qlen + KV_BQ - 1) / KV_BQ;
  const int qt_begin = CAUSAL ? (kt * KV_BN) / KV_BQ : 0;
  const int per_head = n_qt - qt_begin;
  const int n_it = per_head > 0 ? per_head * a.group : 0;
  const float c2 = a.scale_log2;
  const int arow = sigma(l32);  // A-operand row of this lane (query row in the tile)
  const int trr = tr_row(lane), trc = tr_col_bytes(lane);

  PfKV<DQK, DV> pf;
  auto it_head = [&](int it) { return kvh * a.group + it / per_head; };
  auto it_q0 = [&](int it) { return q_lo + (qt_begin + it % per_head) * KV_BQ; };
  if (n_it > 0) {
    kv_load<DQK, DV>(pf, a, it_head(0), it_q0(0), q_hi, tid);
    kv_store<DQK, DV>(pf, smem, tid);
    if (n_it > 1) kv_load<DQK, DV>(pf, a, it_head(1), it_q0(1), q_hi, tid);
  }
  __syncthreads();

  for (int it = 0; it < n_it; ++it) {
    const char* st = smem + (it & 1) * G::STAGE;
    const int qt_rel = (qt_begin + it % per_head) * KV_BQ;  // first query row (part-relative)
    const bool live = wave_live && (!CAUSAL || qt_rel + KV_BQ - 1 >= wk_rel);
    if (live) {
      const char* qs = st;
      const char* os = st + G::Q_BYTES;
      const float* lsd = reinterpret_cast<const float*>(st + G::Q_BYTES + G::O_BYTES);
      // S = Q K^T and dP = dO V^T, lane = key column, entry i = query row
      // 16*(i/8) + 8g + i%8 of the tile
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < G::KK; ++kk)
        s = mma(as_bf16x8(lds16(qs + dual_off<G::QROWB>(arow, (16 * kk + 8 * g) * 2))), kf[kk], s);
#pragma unroll
      for (int kk = 0; kk < G::VK; ++kk)
        dp = mma(as_bf16x8(lds16(os + dual_off<G::OROWB>(arow, (16 * kk + 8 * g) * 2))), vf[kk],
                 dp);
      const bool need_mask =
          (my_key_rel >= klen) || (wk_rel + 31 >= klen) || (CAUSAL && qt_rel < wk_rel + 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * (i >> 3) + 8 * g + (i & 7);
        const float l2 = lsd[r];
        const float dl = lsd[KV_BQ + r];
        float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -l2));
        if (need_mask) {
          const bool ok = (my_key_rel < klen) && (!CAUSAL || my_key_rel <= qt_rel + r);
          p = ok ? p : 0.f;
        }
        s[i] = p;
        dp[i] = p * (dp[i] - dl);
      }
      const bf16x8 pp0 = pack8(s, 0), pp1 = pack8(s, 8);
      const bf16x8 ds0 = pack8(dp, 0), ds1 = pack8(dp, 8);
      // dV += P^T dO,  dK += dS^T Q   (B via transposing reads)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int row = 16 * bb + trr;
#pragma unroll
        for (int nt = 0; nt < G::NVT; ++nt) {
          const int col = 64 * nt + trc;
          const bf16x8 bo = cat_tr(lds_tr(os + dual_off<G::OROWB>(row, col)),
                                   lds_tr(os + dual_off<G::OROWB>(row + 4, col)));
          dv[nt] = mma(bb ? pp1 : pp0, bo, dv[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < G::NQT; ++nt) {
          const int col = 64 * nt + trc;
          const bf16x8 bq = cat_tr(lds_tr(qs + dual_off<G::QROWB>(row, col)),
                                   lds_tr(qs + dual_off<G::QROWB>(row + 4, col)));
          dk[nt] = mma(bb ? ds1 : ds0, bq, dk[nt]);
        }
      }
    }
    if (it + 1 < n_it) {
      kv_store<DQK, DV>(pf, smem + ((it + 1) & 1) * G::STAGE, tid);
      __syncthreads();
      if (it + 2 < n_it) kv_load<DQK, DV>(pf, a, it_head(it + 2), it_q0(it + 2), q_hi, tid);
    }
  }
  if (!wave_live) return;

  // C rows = keys 8*(i/4) + 4g + i%4 of the wave, column = dim 32*nt + l32
  const float scale = a.scale;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = wk_rel + 8 * (i >> 2) + 4 * g + (i & 3);
    if (kr >= klen) continue;
    const int64_t key = k_lo + kr;
    float* dkp = a.dk + (key * a.hkv + kvh) * DQK + l32;
    float* dvp = a.dv + (key * a.hkv + kvh) * DV + l32;
#pragma unroll
    for (int nt = 0; nt < G::NQT; ++nt) dkp[32 * nt] += scale * dk[nt][i];
#pragma unroll
    for (int nt = 0; nt < G::NVT; ++nt) dvp[32 * nt] += dv[nt][i];
  }
}

// ===========================================================================
// dQ
// ===========================================================================
constexpr int Q_BM = 128;  // query rows per workgroup
constexpr int Q_BN = 64;   // keys per tile

template <int DQK, int DV>
struct GeoQ {
  static constexpr int KROWB = DQK <= 128 ? 256 : 512;
  static constexpr int VROWB = 256;
  static constexpr int K_BYTES = Q_BN * KROWB;
  static constexpr int V_BYTES = Q_BN * VROWB;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int KCH = DQK / 8, VCH = DV / 8;
  static constexpr int K_LD = Q_BN * KCH / NT;
  static constexpr int V_LD = Q_BN * VCH / NT;
  static constexpr int KK = DQK / 16, VK = DV / 16;
  static constexpr int NQT = DQK / 32;
  static_assert(DV == 128, "V rows are 256 bytes");
};

template <int DQK, int DV>
struct PfQ {
  u32x4 k[GeoQ<DQK, DV>::K_LD];
  u32x4 v[GeoQ<DQK, DV>::V_LD];
};

template <int DQK, int DV>
__device__ __forceinline__ void q_load(PfQ<DQK, DV>& pf, const __bf16* kb, const __bf16* vb,
                                       int64_t ks, int64_t vs, int key0, int k_last, int tid) {
  using G = GeoQ<DQK, DV>;
#pragma unroll
  for (int i = 0; i < G::K_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::KCH, c = idx % G::KCH;
    pf.k[i] = ldg16(kb + (int64_t)min(key0 + row, k_last) * ks + c * 8);
  }
#pragma unroll
  for (int i = 0; i < G::V_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::VCH, c = idx % G::VCH;
    pf.v[i] = ldg16(vb + (int64_t)min(key0 + row, k_last) * vs + c * 8);
  }
}

template <int DQK, int DV>
__device__ __forceinline__ void q_store(const PfQ<DQK, DV>& pf, char* st, int tid) {
  using G = GeoQ<DQK, DV>;
#pragma unroll
  for (int i = 0; i < G::K_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::KCH, c = idx % G::KCH;
    *reinterpret_cast<u32x4*>(st + dual_off<G::KROWB>(row, c * 16)) = pf.k[i];
  }
#pragma unroll
  for (int i = 0; i < G::V_LD; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / G::VCH, c = idx % G::VCH;
    *reinterpret_cast<u32x4*>(st + G::K_BYTES + dual_off<G::VROWB>(row, c * 16)) = pf.v[i];
  }
}

template <int DQK, int DV, bool CAUSAL>
__global__ __launch_bounds__(NT, 1) void attn_bwd_dq_kernel(AttnArgs a) {
  using G = GeoQ<DQK, DV>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::STAGE];

  int b = xcd_remap(blockIdx.x, gridDim.x);
  const int hg = b % a.group;
  b /= a.group;
  const int qt_rev = b % a.n_qtiles;
  b /= a.n_qtiles;
  const int kvh = b % a.hkv;
  const int seg = b / a.hkv;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - qt_rev) : qt_rev;
  const int h = kvh * a.group + hg;

  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], a.q_part, &q_lo, &q_hi);
  part_range(a.cu_k[seg], a.cu_k[seg + 1], a.k_part, &k_lo, &k_hi);
  const int q0 = q_lo + qt * Q_BM;
  if (q0 >= q_hi) return;
  const int klen = k_hi - k_lo;
  if (klen <= 0) return;  // nothing to add

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < q_hi;
  const int my_row = wq0 + l32;
  const bool row_ok = my_row < q_hi;
  const int my_row_rel = my_row - q_lo;
  const int wq_first_rel = wq0 - q_lo;
  const int wq_last_rel = min(wq0 + 32, q_hi) - 1 - q_lo;
  const int qrel_last_wg = min(q0 + Q_BM, q_hi) - 1 - q_lo;
  const int kend = CAUSAL ? min(klen, qrel_last_wg + 1) : klen;
  const int wave_kend = CAUSAL ? min(klen, wq_last_rel + 1) : klen;
  const int ntiles = (kend + Q_BN - 1) / Q_BN;

  const int row = min(my_row, q_hi - 1);
  bf16x8 qf[G::KK], of[G::VK];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (int64_t)row * a.q_stride +
                       (int64_t)h * DQK + 8 * g;
    const __bf16* op = reinterpret_cast<const __bf16*>(a.dout) + ((int64_t)row * a.hq + h) * DV +
                       8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) qf[kk] = as_bf16x8(ldg16(qp + 16 * kk));
#pragma unroll
    for (int kk = 0; kk < G::VK; ++kk) of[kk] = as_bf16x8(ldg16(op + 16 * kk));
  }
  const int64_t li = (int64_t)h * a.total_q + row;
  const float l2 = lse_log2(a.lse_in, li, row_ok);
  const float dl = row_ok ? a.delta[li] : 0.f;
  const float c2 = a.scale_log2;

  f32x16 dq[G::NQT];
#pragma unroll
  for (int t = 0; t < G::NQT; ++t) dq[t] = zero16();

  const __bf16* kb = reinterpret_cast<const __bf16*>(a.k) + (int64_t)kvh * DQK;
  const __bf16* vb = reinterpret_cast<const __bf16*>(a.v) + (int64_t)kvh * DV;
  const int k_last = k_hi - 1;
  const int arow = sigma(l32);
  const int trr = tr_row(lane), trc = tr_col_bytes(lane);

  PfQ<DQK, DV> pf;
  if (ntiles > 0) {
    q_load<DQK, DV>(pf, kb, vb, a.k_stride, a.v_stride, k_lo, k_last, tid);
    q_store<DQK, DV>(pf, smem, tid);
    if (ntiles > 1) q_load<DQK, DV>(pf, kb, vb, a.k_stride, a.v_stride, k_lo + Q_BN, k_last, tid);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const char* st = smem + (t & 1) * G::STAGE;
    const int kt0 = t * Q_BN;
    if (wave_live && kt0 < wave_kend) {
      const char* ks = st;
      const char* vs = st + G::K_BYTES;
      const bool need_mask = (kt0 + Q_BN > wave_kend) || (CAUSAL && kt0 + Q_BN - 1 > wq_first_rel);
      bf16x8 dsp[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x16 s = zero16(), dp = zero16();
        const int kr = arow + 32 * hh;
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk)
          s = mma(as_bf16x8(lds16(ks + dual_off<G::KROWB>(kr, (16 * kk + 8 * g) * 2))), qf[kk], s);
#pragma unroll
        for (int kk = 0; kk < G::VK; ++kk)
          dp = mma(as_bf16x8(lds16(vs + dual_off<G::VROWB>(kr, (16 * kk + 8 * g) * 2))), of[kk],
                   dp);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -l2));
          if (need_mask) {
            const int key = kt0 + 32 * hh + 16 * (i >> 3) + 8 * g + (i & 7);
            const bool ok = key < klen && (!CAUSAL || key <= my_row_rel);
            p = ok ? p : 0.f;
          }
          dp[i] = p * (dp[i] - dl);
        }
        dsp[2 * hh] = pack8(dp, 0);
        dsp[2 * hh + 1] = pack8(dp, 8);
      }
      // dQ^T += K^T dS^T, A = K^T by transposing reads of the K tile
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int r = 16 * bb + trr;
#pragma unroll
        for (int nt = 0; nt < G::NQT; ++nt) {
          const int col = 64 * nt + trc;
          const bf16x8 ka = cat_tr(lds_tr(ks + dual_off<G::KROWB>(r, col)),
                                   lds_tr(ks + dual_off<G::KROWB>(r + 4, col)));
          dq[nt] = mma(ka, dsp[bb], dq[nt]);
        }
      }
    }
    if (t + 1 < ntiles) {
      q_store<DQK, DV>(pf, smem + ((t + 1) & 1) * G::STAGE, tid);
      __syncthreads();
      if (t + 2 < ntiles)
        q_load<DQK, DV>(pf, kb, vb, a.k_stride, a.v_stride, k_lo + (t + 2) * Q_BN, k_last, tid);
    }
  }
  if (!wave_live || !row_ok) return;

  // C: column = query row (this lane), rows = dims 32*nt + 8*(i/4) + 4g + i%4
  float* dqp = a.dq + ((int64_t)my_row * a.hq + h) * DQK;
  const float scale = a.scale;
#pragma unroll
  for (int nt = 0; nt < G::NQT; ++nt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4* p = reinterpret_cast<float4*>(dqp + 32 * nt + 8 * q4 + 4 * g);
      float4 x = *p;
      x.x += scale * dq[nt][4 * q4 + 0];
      x.y += scale * dq[nt][4 * q4 + 1];
      x.z += scale * dq[nt][4 * q4 + 2];
      x.w += scale * dq[nt][4 * q4 + 3];
      *p = x;
    }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnArgs& a0, int dqk, int dv, bool causal,
                                hipStream_t st) {
  // a0.n_qtiles counts 128-row query tiles, a0.n_ktiles 128-key tiles
  AttnArgs a = a0;
  const long long nq = (long long)a.n_seq * a.hkv * a.n_qtiles * a.group;
  const long long nk = (long long)a.n_seq * a.hkv * a.n_ktiles;
  if (nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define RA_BWD_LAUNCH(DQ, DVV, C)                                                              \
  do {                                                                                         \
    if (nq > 0)                                                                                \
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQ, DVV, C>), dim3((unsigned)nq), dim3(NT), 0, st, \
                         a);                                                                   \
    if (nk > 0)                                                                                \
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQ, DVV, C>), dim3((unsigned)nk), dim3(NT), 0,   \
                         st, a);                                                               \
  } while (0)
  if (dqk == 128 && dv == 128) {
    if (causal) RA_BWD_LAUNCH(128, 128, true);
    else RA_BWD_LAUNCH(128, 128, false);
  } else if (dqk == 192 && dv == 128) {
    if (causal) RA_BWD_LAUNCH(192, 128, true);
    else RA_BWD_LAUNCH(192, 128, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef RA_BWD_LAUNCH
  return hipGetLastError();
}

}  // namespace ra
