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
//   K and (at d_qk = 128) V of the wave's keys stay in registers, V
//   otherwise in LDS (loaded once); the loop walks every query head of the
//   kv group and every 32-row query tile of the segment part (causal: only
//   tiles at or below the keys).  Per tile, with lane l owning key column
//   l%32 of the 32x32 accumulators:
//     S  = Q K^T, dP = dO V^T        A = Q / dO rows from LDS, B = K / V
//                                    in registers (V in LDS at d_qk = 192)
//     dV += P^T dO, dK += dS^T Q     A = P^T / dS^T straight from the S / dP
//                                    accumulators (query rows fed in the
//                                    permuted order sigma so 8 consecutive
//                                    entries are 8 consecutive rows),
//                                    B = dO / Q via transposing LDS reads.
// dQ kernel -- workgroup = 128 query rows of one head (4 waves x 32 rows),
//   the forward's shape: lane l owns query row l%32; per 64-key tile
//     S^T = K Q^T, dP^T = V dO^T     A = K / V rows from LDS (sigma order),
//                                    B = Q / dO of the lane's row, held in
//                                    registers (dO of the workgroup's rows
//                                    in LDS at d_qk = 192)
//     dQ^T += K^T dS^T               A = K via transposing LDS reads.
// Q, dO and K tiles are read both by 128-bit row reads and by transposing
// reads, so they use the XOR-swizzled "dual" LDS layout (conflict-free for
// both, see mfma_common.h).  Every tile goes from global memory straight
// into LDS (buffer_load ... lds, DualLoader), double-buffered in separate LDS
// objects: tile t+1 streams in while tile t is computed, and no registers
// stage the prefetch.  The lse and delta of a query tile come along (4 bytes
// per lane).  Each kernel runs one wave per SIMD (large accumulators), so
// the LDS operand reads of a block of products are scheduled a few products
// ahead (pipeline_lds_mfma).  Only tiles that cross a part end or the
// diagonal evaluate the mask, on a branch of their own.  At d_qk = 128 the
// dQ kernel issues the softmax of one 32-key half between products it does
// not feed (pipeline_lds_mfma_valu).

#include <cstring>

#include "mfma_common.h"

namespace ra {
namespace {

using namespace mfma;

constexpr int NT = 256;
constexpr float kLog2e = 1.4426950408889634f;
// matrix-core products the LDS operand reads run ahead of (one wave per
// SIMD here, so nothing else hides the read latency)
#ifndef RA_BWD_AHEAD
#define RA_BWD_AHEAD 4
#endif
constexpr int kBwdAhead = RA_BWD_AHEAD;
// vector instructions of the softmax of one 32-key half in the dQ kernel
// (per score: two accumulator reads, fma, exp, sub, mul; one pack per two),
// spread over the products it is interleaved with
constexpr int kSoftmaxValu = 16 * 6 + 8;

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
  static constexpr int KK = DQK / 16, VK = DV / 16;
  static constexpr int NQT = DQK / 32, NVT = DV / 32;
  static_assert(DV == 128, "dO rows are 256 bytes");
};

// Tile r of the live 128-key (BY_KEYS) or 128-row tiles of a block in the
// rank-fused grids: a segment contributes ceil(length / 128) tiles along
// that axis if some row of its query part sees some key of its key part.
// seg_at(i) is the segment the grid takes i-th.  (A functor that reads the
// kernel argument directly: a pointer into a by-value kernel argument makes
// the compiler copy the whole argument to scratch memory.)
template <bool BY_KEYS, class SegAt>
__device__ __forceinline__ bool locate_tile(const int32_t* cu_q, const int32_t* cu_k, int n_seq,
                                            int qp, int kp, int r, int* seg, int* idx, int* cnt,
                                            SegAt seg_at) {
  auto count = [&](int s) {
    s = seg_at(s);
    int ql, qh, kl, kh;
    part_range(cu_q[s], cu_q[s + 1], qp, &ql, &qh);
    part_range(cu_k[s], cu_k[s + 1], kp, &kl, &kh);
    return (qh > ql && kh > kl) ? ((BY_KEYS ? kh - kl : qh - ql) + 127) / 128 : 0;
  };
  if (!locate_in_segments(n_seq, r, count, seg, idx, cnt)) return false;
  *seg = seg_at(*seg);
  return true;
}

// QS ("query split"): a workgroup covers 32 keys and its 4 waves split the
// (query head, query tile) iterations among themselves, each with its own
// two LDS stages and no barrier in the loop; the waves' dK/dV are added in
// a fixed order (wave 0 + 1 + 2 + 3) through LDS at the end, so the result
// stays deterministic.  It gives 4x the workgroups of the 128-key form, for
// launches with few key tiles (GQA/MHA history blocks at d_qk = 128).
// RANK: a rank's whole backward share in one launch; the slowest index of
// the grid is the ring step o (owner (rank - o) mod C, the diagonal block
// first), and every workgroup takes its owner's K/V, dK/dV accumulators,
// parts and causal rule (owner_plan); CAUSAL is then ignored.
template <int DQK, int DV, bool CAUSAL, bool QS, bool RANK = false>
__global__ __launch_bounds__(NT, 1) void attn_bwd_dkdv_kernel(AttnArgs a, RankKV rk, RankGrad rg) {
  using G = GeoKV<DQK, DV>;
  constexpr int KBN = QS ? 32 : KV_BN;  // keys per workgroup
  constexpr int NS = QS ? NT / 64 : 1;  // stage sets (one per wave with QS)
  static_assert(!QS || (G::Q_BYTES == 8192 && G::O_BYTES == 8192), "QS reduction buffers");
  // per stage: Q tile, dO tile, lse (rows 0..31) and delta (32..63)
  __shared__ __attribute__((aligned(1024))) char qs0[NS][G::Q_BYTES];
  __shared__ __attribute__((aligned(1024))) char qs1[NS][G::Q_BYTES];
  __shared__ __attribute__((aligned(1024))) char os0[NS][G::O_BYTES];
  __shared__ __attribute__((aligned(1024))) char os1[NS][G::O_BYTES];
  __shared__ __attribute__((aligned(256))) float ld0[NS][2 * KV_BQ];
  __shared__ __attribute__((aligned(256))) float ld1[NS][2 * KV_BQ];
  // V of the wave's keys as B operands of dP: held in registers at d_qk =
  // 128 (re-read from LDS every tile it had been a fifth of the tile's LDS
  // operand bytes); at d_qk = 192 the registers are nearly full (holding it
  // there cost the MLA backward 9%), so V of the workgroup's keys sits in
  // LDS (dual layout)
  constexpr bool VREG = DQK <= 128;
  __shared__ __attribute__((aligned(1024))) char vsm[VREG ? 16 : KBN * G::OROWB];

  const int nsp = QS || RANK ? 1 : a.qsplit;  // workgroups sharing a key tile
  // One block: packed documents deal key tiles (with their query shares)
  // over the XCDs, since one document's tiles follow another's in logical
  // order; otherwise contiguous ranges per XCD (neighbours share K/V in L2).
  // A rank share: the kv head is the slowest index and every XCD takes a
  // contiguous range, i.e. the key tiles of one kv head over all owners and
  // documents: they all read that head's Q and dO tiles, which then stay in
  // the XCD's L2 (dealt over the XCDs, every L2 fetched every head's tiles;
  // 32K GQA backward 478 -> 284 TFLOP/s).  The diagonal block comes first.
  // A rank share's grid holds only live tiles: per kv head, the ring steps
  // in order, each with its owner's live tiles segment by segment, taken in
  // the host's heaviest-first order when it fits the kernel arguments.
  int b = (!RANK && a.n_seq > 1) ? xcd_deal(blockIdx.x, gridDim.x, nsp)
                                 : xcd_remap(blockIdx.x, gridDim.x);
  const int sp = b % nsp;
  b /= nsp;
  int kt, kvh, seg, step_o = 0;
  int own_causal = CAUSAL ? 1 : 0, own_qp = a.q_part, own_kp = a.k_part;
  if (RANK) {
    const int per_head = rk.kv_tile_off[rk.cp];
    kvh = b / per_head;
    int r = b - kvh * per_head;
    if (rk.tile_ordered == 1) r = rk.tile_order[r];  // the host's heaviest-first order
    while (step_o + 1 < rk.cp && r >= rk.kv_tile_off[step_o + 1]) ++step_o;
    r -= rk.kv_tile_off[step_o];
    owner_plan(rk.rank, (rk.rank - step_o + rk.cp) % rk.cp, &own_causal, &own_qp, &own_kp);
    if (a.n_seq == 1) {
      seg = 0;
      kt = r;
    } else {
      int cnt;
      if (!locate_tile<true>(a.cu_q, a.cu_k, a.n_seq, own_qp, own_kp, r, &seg, &kt, &cnt,
                             [](int i) { return i; }))
        return;
    }
  } else {
    kt = b % a.n_ktiles;
    b /= a.n_ktiles;
    kvh = b % a.hkv;
    seg = b / a.hkv;
  }
  const int owner = RANK ? (rk.rank - step_o + rk.cp) % rk.cp : 0;
  const bool causal = RANK ? own_causal != 0 : CAUSAL;
  const void* kptr = RANK ? rk.k[owner] : a.k;
  const void* vptr = RANK ? rk.v[owner] : a.v;
  float* dkptr = RANK ? rg.dk[owner] : a.dk;
  float* dvptr = RANK ? rg.dv[owner] : a.dv;

  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], own_qp, &q_lo, &q_hi);
  part_range(a.cu_k[seg], a.cu_k[seg + 1], own_kp, &k_lo, &k_hi);
  const int k0 = k_lo + kt * KBN;
  const int qlen = q_hi - q_lo, klen = k_hi - k_lo;
  if (k0 >= k_hi || qlen <= 0) return;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int ws = QS ? wave : 0;                      // this wave's stage set
  const int wk_rel = kt * KBN + (QS ? 0 : wave * 32);  // first key of the wave (part-relative)
  const bool wave_live = wk_rel < klen;
  const int my_key_rel = wk_rel + l32;               // this lane's key column
  const int my_key = min(k_lo + my_key_rel, k_hi - 1);

  // K (and V) of this lane's key as B operands (k = dims 16kk + 8g .. +7;
  // keys past the block re-read the last one)
  bf16x8 kf[G::KK], vf[VREG ? G::VK : 1];
  {
    const __bf16* kp = reinterpret_cast<const __bf16*>(kptr) + (int64_t)my_key * a.k_stride +
                       (int64_t)kvh * DQK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) kf[kk] = as_bf16x8(ldg16(kp + 16 * kk));
    if constexpr (VREG) {
      const __bf16* vp = reinterpret_cast<const __bf16*>(vptr) + (int64_t)my_key * a.v_stride +
                         (int64_t)kvh * DV + 8 * g;
#pragma unroll
      for (int kk = 0; kk < G::VK; ++kk) vf[kk] = as_bf16x8(ldg16(vp + 16 * kk));
    } else {
      DualLoader<KBN, DV, G::OROWB, NT / 64> lvk;
      const int64_t vsb = a.v_stride * 2;
      lvk.init(vsb, wave, lane);
      lvk.issue(reinterpret_cast<const char*>(vptr) + ((int64_t)k0 * a.v_stride + (int64_t)kvh * DV) * 2,
                vsb, k_hi - k0, vsm);
    }
  }
  const int vrow = (QS ? 0 : wave * 32) + l32;  // this lane's key row in vsm
  f32x16 dk[G::NQT], dv[G::NVT];
#pragma unroll
  for (int t = 0; t < G::NQT; ++t) dk[t] = zero16();
#pragma unroll
  for (int t = 0; t < G::NVT; ++t) dv[t] = zero16();

  const int n_qt = (qlen + KV_BQ - 1) / KV_BQ;
  const int qt_begin = causal ? (kt * KBN) / KV_BQ : 0;
  const int per_head = n_qt - qt_begin;
  const int n_all = per_head > 0 ? per_head * a.group : 0;
  // this workgroup's share of the iterations: [it_lo, n_it)
  const int it_lo = (int)((int64_t)n_all * sp / nsp);
  const int n_it = (int)((int64_t)n_all * (sp + 1) / nsp);
  const float c2 = a.scale_log2;
  const int arow = sigma(l32);  // A-operand row of this lane (query row in the tile)
  const int trr = tr_row(lane), trc = tr_col_bytes(lane);

  // Iteration it is query head it / per_head of the group and query tile
  // qt_begin + it % per_head; the loop steps a (head, tile) cursor instead
  // of dividing by the runtime per_head twice per iteration (a software
  // division is some 40 scalar instructions, on the only wave of the SIMD).
  struct ItPos {
    int h, qt;  // head within the group, tile index from qt_begin
  };
  auto it_pos = [&](int it) {
    ItPos c;
    c.h = per_head > 0 ? it / per_head : 0;
    c.qt = per_head > 0 ? it - c.h * per_head : 0;
    return c;
  };
  auto it_next = [&](ItPos c, int n) {
    c.qt += n;
    while (c.qt >= per_head) {
      c.qt -= per_head;
      ++c.h;
    }
    return c;
  };
  // with QS each wave loads its own tiles alone
  DualLoader<KV_BQ, DQK, G::QROWB, QS ? 1 : NT / 64> lq;
  DualLoader<KV_BQ, DV, G::OROWB, QS ? 1 : NT / 64> lo;
  const int64_t qsb = a.q_stride * 2, osb = (int64_t)a.hq * DV * 2;
  lq.init(qsb, QS ? 0 : wave, lane);
  lo.init(osb, QS ? 0 : wave, lane);
  // tile it's Q, dO, lse and delta into one stage (rows past the part are
  // clamped to its last row here and masked in the products)
  auto issue = [&](ItPos c, char* qd, char* od, float* ldd) __attribute__((always_inline)) {
    const int h = kvh * a.group + c.h, q0 = q_lo + (qt_begin + c.qt) * KV_BQ;
    const int rows_left = q_hi - q0;
    lq.issue(reinterpret_cast<const char*>(a.q) + ((int64_t)q0 * a.q_stride + (int64_t)h * DQK) * 2,
             qsb, rows_left, qd);
    lo.issue(reinterpret_cast<const char*>(a.dout) + ((int64_t)q0 * a.hq + h) * DV * 2, osb,
             rows_left, od);
    if (QS || wave == 0) {
      const uint32_t r4 = (uint32_t)min(lane & (KV_BQ - 1), rows_left - 1) * 4;
      const int64_t i0 = (int64_t)h * a.total_q + q0;
      if (lane < KV_BQ) g2lds4(tile_rsrc(a.lse_in + i0), r4, ldd);
      else g2lds4(tile_rsrc(a.delta + i0), r4, ldd);
    }
  };

  // products of tile it from one stage
  auto tile = [&](ItPos c, const char* qs, const char* os, const float* lsd)
      __attribute__((always_inline)) {
    const int qt_rel = (qt_begin + c.qt) * KV_BQ;  // first query row (part-relative)
    const bool live = wave_live && (!causal || qt_rel + KV_BQ - 1 >= wk_rel);
    if (!live) return;
    // lse and delta of the lane's 16 rows (entry i below is row 16(i/8) +
    // 8g + i%8), read before the products so their latency hides there
    float4 lr[4], dr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * (j >> 1) + 8 * g + 4 * (j & 1);
      lr[j] = *reinterpret_cast<const float4*>(lsd + r);
      dr[j] = *reinterpret_cast<const float4*>(lsd + KV_BQ + r);
    }
    __builtin_amdgcn_sched_barrier(0);
    // S = Q K^T and dP = dO V^T, lane = key column, entry i = query row
    // 16*(i/8) + 8g + i%8 of the tile
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk)
      s = mma(as_bf16x8(lds16(qs + dual_off<G::QROWB>(arow, (16 * kk + 8 * g) * 2))), kf[kk], s);
    if constexpr (VREG) {
#pragma unroll
      for (int kk = 0; kk < G::VK; ++kk)
        dp = mma(as_bf16x8(lds16(os + dual_off<G::OROWB>(arow, (16 * kk + 8 * g) * 2))), vf[kk], dp);
      pipeline_lds_mfma<G::KK + G::VK, 1, kBwdAhead>();
    } else {
#pragma unroll
      for (int kk = 0; kk < G::VK; ++kk)
        dp = mma(as_bf16x8(lds16(os + dual_off<G::OROWB>(arow, (16 * kk + 8 * g) * 2))),
                 as_bf16x8(lds16(vsm + dual_off<G::OROWB>(vrow, (16 * kk + 8 * g) * 2))), dp);
      pipeline_lds_mfma_n<G::KK, 1, G::VK, 2, kBwdAhead>();
    }
    __builtin_amdgcn_sched_barrier(0);
    // wave-uniform: some pair of the tile is hidden (the wave's last key past
    // the part covers every lane's key past it)
    const bool need_mask = (wk_rel + 31 >= klen) || (causal && qt_rel < wk_rel + 31) ||
                           (qt_rel + KV_BQ > qlen);
    float nl2[16], dl[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      nl2[i] = -lr[i >> 2][i & 3] * kLog2e;
      dl[i] = dr[i >> 2][i & 3];
    }
    if (need_mask) {
      // Hidden pairs get score -inf, so P = 0.  A row that sees nothing
      // (lse -inf, which only a masked tile holds: every pair of an
      // unmasked tile is visible) gets offset -inf instead of +inf.  Entry i
      // is row 8g + e of the tile, e = 16(i/8) + i%8; it is visible iff
      // lo <= e < hi.
      const int r0 = qt_rel + 8 * g;
      const int hi = my_key_rel < klen ? qlen - r0 : -1;
      const int lo = causal ? my_key_rel - r0 : -KV_BQ;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = 16 * (i >> 3) + (i & 7);
        s[i] = (e >= lo && e < hi) ? s[i] : -INFINITY;
        nl2[i] = nl2[i] == INFINITY ? -INFINITY : nl2[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, nl2[i]));
      s[i] = p;
      dp[i] = p * (dp[i] - dl[i]);
    }
    const bf16x8 pp0 = pack8(s, 0), pp1 = pack8(s, 8);
    const bf16x8 ds0 = pack8(dp, 0), ds1 = pack8(dp, 8);
    __builtin_amdgcn_sched_barrier(0);
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
    pipeline_lds_mfma<2 * (G::NVT + G::NQT), 2, kBwdAhead>();
  };

  // iterations of this wave: all (it += 1), or with QS every 4th from the
  // wave's index
  const int it0 = it_lo + (QS ? wave : 0), istep = QS ? NT / 64 : 1;
  ItPos pos = it_pos(it0);  // of iteration it
  if (it0 < n_it) issue(pos, qs0[ws], os0[ws], ld0[ws]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // K, V and (without QS) the first tile in place
  auto step = [&](int it, const char* qs, const char* os, const float* lsd, char* qn, char* on,
                  float* ln) __attribute__((always_inline)) {
    const ItPos next = it_next(pos, istep);
    if (it + istep < n_it) issue(next, qn, on, ln);
    tile(pos, qs, os, lsd);
    pos = next;
    // next tile landed (own loads); without QS also every wave is done with
    // this one (with QS the stages are the wave's own, and its reads of
    // them complete before it issues the next load into them)
    __builtin_amdgcn_s_waitcnt(0);
    if (!QS) __syncthreads();
  };
  for (int it = it0; it < n_it; it += 2 * istep) {
    step(it, qs0[ws], os0[ws], ld0[ws], qs1[ws], os1[ws], ld1[ws]);
    if (it + istep < n_it) step(it + istep, qs1[ws], os1[ws], ld1[ws], qs0[ws], os0[ws], ld0[ws]);
  }
  if (QS) {
    // add the waves' dK/dV in a fixed order: waves 1..3 park theirs in their
    // own (now idle) stage buffers, wave 0 adds them one by one
    __syncthreads();
    if (wave > 0) {
      float* pk0 = reinterpret_cast<float*>(qs0[wave]);
      float* pk1 = reinterpret_cast<float*>(qs1[wave]);
      float* pv0 = reinterpret_cast<float*>(os0[wave]);
      float* pv1 = reinterpret_cast<float*>(os1[wave]);
#pragma unroll
      for (int nt = 0; nt < G::NQT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = nt * 16 + i;  // 64 floats per lane, lane-major
          (e < 32 ? pk0 : pk1)[(e & 31) * 64 + lane] = dk[nt][i];
        }
#pragma unroll
      for (int nt = 0; nt < G::NVT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = nt * 16 + i;
          (e < 32 ? pv0 : pv1)[(e & 31) * 64 + lane] = dv[nt][i];
        }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
      const float* pk0 = reinterpret_cast<const float*>(qs0[w]);
      const float* pk1 = reinterpret_cast<const float*>(qs1[w]);
      const float* pv0 = reinterpret_cast<const float*>(os0[w]);
      const float* pv1 = reinterpret_cast<const float*>(os1[w]);
#pragma unroll
      for (int nt = 0; nt < G::NQT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = nt * 16 + i;
          dk[nt][i] += (e < 32 ? pk0 : pk1)[(e & 31) * 64 + lane];
        }
#pragma unroll
      for (int nt = 0; nt < G::NVT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = nt * 16 + i;
          dv[nt][i] += (e < 32 ? pv0 : pv1)[(e & 31) * 64 + lane];
        }
    }
  }
  if (!wave_live) return;

  // C rows = keys 8*(i/4) + 4g + i%4 of the wave, column = dim 32*nt + l32
  const float scale = a.scale;
  if (sp == 0 && QS) {
    // (the query-split form keeps one load-add-store per key row: its
    // waves' reduction leaves no registers for a batch)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = wk_rel + 8 * (i >> 2) + 4 * g + (i & 3);
      if (kr >= klen) continue;
      const int64_t key = k_lo + kr;
      float* dkp = dkptr + (key * a.hkv + kvh) * DQK + l32;
      float* dvp = dvptr + (key * a.hkv + kvh) * DV + l32;
#pragma unroll
      for (int nt = 0; nt < G::NQT; ++nt) dkp[32 * nt] += scale * dk[nt][i];
#pragma unroll
      for (int nt = 0; nt < G::NVT; ++nt) dvp[32 * nt] += dv[nt][i];
    }
  } else if (sp == 0) {
    // Add into the owner's float32 dK, then dV, each as one batch: every
    // old value is loaded before the first store.  Written as a
    // load-add-store per key row, the compiler cannot tell the rows'
    // addresses apart and waits a full memory round trip per row (32 per
    // wave), which dominated workgroups with few query iterations.  Rows
    // past the block load the last key's values and store nothing.
    auto row_of = [&](int i) { return wk_rel + 8 * (i >> 2) + 4 * g + (i & 3); };
    {
      float old[16][G::NQT];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = k_lo + min(row_of(i), klen - 1);
        const float* p = dkptr + (key * a.hkv + kvh) * DQK + l32;
#pragma unroll
        for (int nt = 0; nt < G::NQT; ++nt) old[i][nt] = p[32 * nt];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (row_of(i) >= klen) continue;
        float* p = dkptr + ((k_lo + row_of(i)) * (int64_t)a.hkv + kvh) * DQK + l32;
#pragma unroll
        for (int nt = 0; nt < G::NQT; ++nt) p[32 * nt] = old[i][nt] + scale * dk[nt][i];
      }
    }
    {
      float old[16][G::NVT];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t key = k_lo + min(row_of(i), klen - 1);
        const float* p = dvptr + (key * a.hkv + kvh) * DV + l32;
#pragma unroll
        for (int nt = 0; nt < G::NVT; ++nt) old[i][nt] = p[32 * nt];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (row_of(i) >= klen) continue;
        float* p = dvptr + ((k_lo + row_of(i)) * (int64_t)a.hkv + kvh) * DV + l32;
#pragma unroll
        for (int nt = 0; nt < G::NVT; ++nt) p[32 * nt] = old[i][nt] + dv[nt][i];
      }
    }
  } else {
    const int64_t row0 = (int64_t)(sp - 1) * a.part_keys;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = wk_rel + 8 * (i >> 2) + 4 * g + (i & 3);
      if (kr >= klen) continue;
      const int64_t key = row0 + k_lo + kr;
      float* dkp = a.dk_part + (key * a.hkv + kvh) * DQK + l32;
      float* dvp = a.dv_part + (key * a.hkv + kvh) * DV + l32;
#pragma unroll
      for (int nt = 0; nt < G::NQT; ++nt) dkp[32 * nt] = scale * dk[nt][i];
#pragma unroll
      for (int nt = 0; nt < G::NVT; ++nt) dvp[32 * nt] = dv[nt][i];
    }
  }
}

// dk/dv += the stored partials of query shares 1 .. qsplit-1, in share
// order, for every key the dK/dV launch covered (keys inside the k part of
// a segment whose q part is not empty).  One thread per 4 floats of a key's
// [hkv, dqk] + [hkv, dv] gradient rows; HBM-bound.
__global__ __launch_bounds__(256) void bwd_qsplit_reduce_kernel(AttnArgs a, int dqk, int dv,
                                                                int total_k) {
  const int nk4 = a.hkv * dqk / 4, row4 = nk4 + a.hkv * dv / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)total_k * row4) return;
  const int key = (int)(idx / row4), c = (int)(idx % row4);
  int lo = 0, hi = a.n_seq;  // segment of the key: cu_k[seg] <= key < cu_k[seg + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_k[mid] <= key) lo = mid; else hi = mid;
  }
  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[lo], a.cu_q[lo + 1], a.q_part, &q_lo, &q_hi);
  part_range(a.cu_k[lo], a.cu_k[lo + 1], a.k_part, &k_lo, &k_hi);
  if (q_hi <= q_lo || key < k_lo || key >= k_hi) return;
  float* dst;
  const float* src;
  int64_t stride;
  if (c < nk4) {
    dst = a.dk + (int64_t)key * a.hkv * dqk + 4 * c;
    src = a.dk_part + (int64_t)key * a.hkv * dqk + 4 * c;
    stride = (int64_t)a.part_keys * a.hkv * dqk;
  } else {
    dst = a.dv + (int64_t)key * a.hkv * dv + 4 * (c - nk4);
    src = a.dv_part + (int64_t)key * a.hkv * dv + 4 * (c - nk4);
    stride = (int64_t)a.part_keys * a.hkv * dv;
  }
  float4 acc = *reinterpret_cast<const float4*>(dst);
  for (int s = 1; s < a.qsplit; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(src + (s - 1) * stride);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  *reinterpret_cast<float4*>(dst) = acc;
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
  static constexpr int KK = DQK / 16, VK = DV / 16;
  static constexpr int NQT = DQK / 32;
  static_assert(DV == 128, "V rows are 256 bytes");
};

// How a KV block meets the query rows of a dQ workgroup (as in the forward).
enum QKind {
  QK_CAUSAL = 0,     // key j visible to row i iff j <= i (part-relative)
  QK_ALL = 1,        // every key visible
  QK_LATE_ROWS = 2,  // every key visible to the segment's second-half rows only
};

// RANK: a rank's whole backward share; every query tile walks the key tiles
// of all C owners' blocks in ring order (the diagonal block first) with dQ
// in registers, each block with its owner's K/V and rule (owner_plan).
// Otherwise one block as described by the AttnArgs parts and CAUSAL.  With
// a.ksplit > 1 the tiles of the walk are dealt round-robin over that many
// workgroups of the same query tile.
template <int DQK, int DV, bool CAUSAL, bool RANK = false>
__global__ __launch_bounds__(NT, 1) void attn_bwd_dq_kernel(AttnArgs a, RankKV rk) {
  using G = GeoQ<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) char ks0[G::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char ks1[G::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs0[G::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs1[G::V_BYTES];
  // dO of the lane's row as B operands of dP^T: held in registers at d_qk
  // = 128 (re-read from LDS every tile it had been a quarter of the tile's
  // LDS operand bytes); at d_qk = 192 the registers are nearly full (holding
  // it there cost the MLA backward 5%), so dO of the workgroup's 128 rows
  // sits in LDS (dual layout)
  constexpr bool OREG = DQK <= 128;
  __shared__ __attribute__((aligned(1024))) char osm[OREG ? 16 : Q_BM * G::VROWB];

  // One block of packed documents: deal query tiles (a kv group's heads and
  // their key shares together) over the XCDs; otherwise contiguous ranges
  // per XCD.  A rank share: the kv head is the slowest index, so an XCD's
  // contiguous range is one kv head's query tiles over all documents, which
  // all walk that head's K/V tiles of every block (kept in the XCD's L2).
  // Per-tile key shares of a single sequence (rk.var_split): units of
  // (query tile, share, shares), heaviest first, the kv heads of a unit
  // next to each other and dealt over the XCDs (an XCD then keeps to one kv
  // head's K/V when there are 8).
  const bool var = RANK && rk.var_split;
  int nks = max(a.ksplit, 1);  // workgroups sharing a query tile
  int b = ((!RANK && a.n_seq > 1) || var)
              ? xcd_deal(blockIdx.x, gridDim.x, var ? a.group : a.group * nks)
              : xcd_remap(blockIdx.x, gridDim.x);
  int kshare = 0;  // this workgroup takes tiles kshare, kshare + nks, ... of the walk
  if (!var) {
    kshare = b % nks;
    b /= nks;
  }
  const int hg = b % a.group;
  b /= a.group;
  int kvh, seg, qt;
  if (var) {
    kvh = b % a.hkv;
    const int e = rk.tile_order[b / a.hkv];
    seg = 0;
    qt = e >> 6;
    kshare = (e >> 3) & 7;
    nks = (e & 7) + 1;
  } else if (RANK) {
    // only live tiles: per kv head, each segment's query tiles, the
    // heaviest (last rows) first; packed segments in the host's
    // heaviest-first order of those tiles
    kvh = b / rk.q_tiles;
    const int r = b - kvh * rk.q_tiles;
    int idx, cnt;
    if (a.n_seq == 1) {
      seg = 0;
      idx = r;
      cnt = a.n_qtiles;
    } else if (!locate_tile<false>(
                   a.cu_q, a.cu_k, a.n_seq, RA_PART_ALL, RA_PART_ALL,
                   rk.tile_ordered == 1 ? (int)rk.tile_order[r] : r, &seg, &idx, &cnt,
                   [&](int i) { return rk.tile_ordered == 2 ? (int)rk.tile_order[i] : i; })) {
      return;
    }
    qt = cnt - 1 - idx;
  } else {
    const int qt_rev = b % a.n_qtiles;
    b /= a.n_qtiles;
    kvh = b % a.hkv;
    seg = b / a.hkv;
    qt = CAUSAL ? (a.n_qtiles - 1 - qt_rev) : qt_rev;  // heaviest first
  }
  const int h = kvh * a.group + hg;

  int q_lo, q_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], RANK ? RA_PART_ALL : a.q_part, &q_lo, &q_hi);
  const int q0 = q_lo + qt * Q_BM;
  if (q0 >= q_hi) return;
  const int qhalf = (q_hi - q_lo) >> 1;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wq0 = q0 + wave * 32;
  const bool wave_live = wq0 < q_hi;
  const int my_row = wq0 + l32;
  const bool row_ok = my_row < q_hi;
  const int my_row_rel = my_row - q_lo;
  const int wq_first_rel = wq0 - q_lo;
  const int wq_last_rel = min(wq0 + 32, q_hi) - 1 - q_lo;
  const int qrel_last_wg = min(q0 + Q_BM, q_hi) - 1 - q_lo;
  const int64_t ksb = a.k_stride * 2, vsb = a.v_stride * 2;
  const int kseg0 = a.cu_k[seg], kseg1 = a.cu_k[seg + 1];
  const int nblocks = RANK ? rk.cp : 1;

  struct QBlock {
    const char* kb;
    const char* vb;
    int klen, kind, ntiles;
  };
  auto get_block = [&](int bi) -> QBlock {
    QBlock blk;
    const void* kp;
    const void* vp;
    int kpart;
    if (RANK) {
      const int owner = (rk.rank - bi + rk.cp) % rk.cp;
      kp = rk.k[owner];
      vp = rk.v[owner];
      blk.kind = bi == 0 ? QK_CAUSAL : (owner < rk.rank ? QK_ALL : QK_LATE_ROWS);
      kpart = (bi != 0 && owner < rk.rank) ? RA_PART_FIRST_HALF : RA_PART_ALL;
    } else {
      kp = a.k;
      vp = a.v;
      blk.kind = CAUSAL ? QK_CAUSAL : QK_ALL;
      kpart = a.k_part;
    }
    int k_lo, k_hi;
    part_range(kseg0, kseg1, kpart, &k_lo, &k_hi);
    blk.klen = k_hi - k_lo;
    blk.kb = reinterpret_cast<const char*>(kp) + ((int64_t)k_lo * a.k_stride + (int64_t)kvh * DQK) * 2;
    blk.vb = reinterpret_cast<const char*>(vp) + ((int64_t)k_lo * a.v_stride + (int64_t)kvh * DV) * 2;
    int kend = blk.klen;
    if (blk.kind == QK_CAUSAL) kend = min(blk.klen, qrel_last_wg + 1);
    if (blk.kind == QK_LATE_ROWS && qrel_last_wg < qhalf) kend = 0;
    blk.ntiles = kend > 0 ? (kend + Q_BN - 1) / Q_BN : 0;
    return blk;
  };
  struct Cursor {
    int bi, t;
    QBlock blk;
  };
  // step a cursor by n tiles of the walk (past the end it stays put)
  auto advance = [&](Cursor& c, int n) {
    for (int i = 0; i < n; ++i) {
      if (++c.t < c.blk.ntiles) continue;
      c.t = 0;
      do {
        if (++c.bi >= nblocks) return;
        c.blk = get_block(c.bi);
      } while (c.blk.ntiles == 0);
    }
  };
  int total = 0;
  for (int bi = 0; bi < nblocks; ++bi) total += get_block(bi).ntiles;
  if (total == 0) return;  // whole workgroup: nothing to add
  Cursor cc;               // tile to compute
  cc.bi = 0;
  cc.t = 0;
  cc.blk = get_block(0);
  while (cc.blk.ntiles == 0 && cc.bi + 1 < nblocks) cc.blk = get_block(++cc.bi);
  cc.t = -1;
  advance(cc, kshare + 1);
  Cursor lc = cc;          // tile to load

  const int row = min(my_row, q_hi - 1);
  // Q (and dO) of this lane's row as B operands (k = dims 16kk + 8g .. +7;
  // rows past the part re-read the last one)
  bf16x8 qf[G::KK], of[OREG ? G::VK : 1];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + (int64_t)row * a.q_stride +
                       (int64_t)h * DQK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) qf[kk] = as_bf16x8(ldg16(qp + 16 * kk));
    if constexpr (OREG) {
      const __bf16* op =
          reinterpret_cast<const __bf16*>(a.dout) + ((int64_t)row * a.hq + h) * DV + 8 * g;
#pragma unroll
      for (int kk = 0; kk < G::VK; ++kk) of[kk] = as_bf16x8(ldg16(op + 16 * kk));
    } else {
      DualLoader<Q_BM, DV, G::VROWB, NT / 64> lod;
      const int64_t osb = (int64_t)a.hq * DV * 2;
      lod.init(osb, wave, lane);
      lod.issue(reinterpret_cast<const char*>(a.dout) + ((int64_t)q0 * a.hq + h) * DV * 2, osb,
                q_hi - q0, osm);
    }
  }
  const int orow = wave * 32 + l32;  // this lane's query row in osm
  const int64_t li = (int64_t)h * a.total_q + row;
  const float l2 = lse_log2(a.lse_in, li, row_ok);
  const float dl = row_ok ? a.delta[li] : 0.f;
  const float c2 = a.scale_log2;

  f32x16 dq[G::NQT];
#pragma unroll
  for (int t = 0; t < G::NQT; ++t) dq[t] = zero16();

  const int arow = sigma(l32);
  const int trr = tr_row(lane), trc = tr_col_bytes(lane);
  DualLoader<Q_BN, DQK, G::KROWB, NT / 64> lk;
  DualLoader<Q_BN, DV, G::VROWB, NT / 64> lv;
  lk.init(ksb, wave, lane);
  lv.init(vsb, wave, lane);
  auto issue = [&](const Cursor& c, char* kd, char* vd) __attribute__((always_inline)) {
    const int rows_left = c.blk.klen - c.t * Q_BN;
    lk.issue(c.blk.kb + (int64_t)c.t * Q_BN * ksb, ksb, rows_left, kd);
    lv.issue(c.blk.vb + (int64_t)c.t * Q_BN * vsb, vsb, rows_left, vd);
  };

  auto tile = [&](const Cursor& c, const char* ks, const char* vs) __attribute__((always_inline)) {
    const int kt0 = c.t * Q_BN, klen = c.blk.klen, kind = c.blk.kind;
    bool live = wave_live, need_mask;
    int wave_kend = klen;
    if (kind == QK_CAUSAL) {
      wave_kend = min(klen, wq_last_rel + 1);
      live = live && kt0 < wave_kend;
      need_mask = (kt0 + Q_BN > wave_kend) || (kt0 + Q_BN - 1 > wq_first_rel);
    } else if (kind == QK_LATE_ROWS) {
      live = live && wq_last_rel >= qhalf && kt0 < klen;
      need_mask = (kt0 + Q_BN > klen) || (wq_first_rel < qhalf);
    } else {
      live = live && kt0 < klen;
      need_mask = kt0 + Q_BN > klen;
    }
    if (!live) return;
    // Two 32-key halves of the tile: S^T, dP^T products of half hh, its
    // mask and softmax (dS^T packed into dsp[2hh], dsp[2hh + 1]), then the
    // dQ products of key blocks bb (16 keys each, half bb / 2).
    f32x16 s[2], dp[2];
    bf16x8 dsp[4];
    auto sdp_products = [&](int hh) __attribute__((always_inline)) {
      s[hh] = zero16();
      dp[hh] = zero16();
      const int kr = arow + 32 * hh;
#pragma unroll
      for (int kk = 0; kk < G::KK; ++kk)
        s[hh] = mma(as_bf16x8(lds16(ks + dual_off<G::KROWB>(kr, (16 * kk + 8 * g) * 2))), qf[kk], s[hh]);
#pragma unroll
      for (int kk = 0; kk < G::VK; ++kk) {
        const bf16x8 ob = OREG ? of[OREG ? kk : 0]
                               : as_bf16x8(lds16(osm + dual_off<G::VROWB>(orow, (16 * kk + 8 * g) * 2)));
        dp[hh] = mma(as_bf16x8(lds16(vs + dual_off<G::VROWB>(kr, (16 * kk + 8 * g) * 2))), ob, dp[hh]);
      }
    };
    auto mask_half = [&](int hh) __attribute__((always_inline)) {
      if (!need_mask) return;
      // hidden pairs get score -inf (P = 0; a row outside the part already
      // has offset -inf).  Entry i is key base + e of the block, e =
      // 16(i/8) + i%8; every rule of the lane's row folds into e <= lim.
      const int base = kt0 + 32 * hh + 8 * g;
      int lim = klen - 1 - base;
      if (kind == QK_CAUSAL) lim = min(lim, my_row_rel - base);
      if (kind == QK_LATE_ROWS && my_row_rel < qhalf) lim = -1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = 16 * (i >> 3) + (i & 7);
        s[hh][i] = e <= lim ? s[hh][i] : -INFINITY;
      }
    };
    auto softmax_half = [&](int hh) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[hh][i], c2, -l2));
        dp[hh][i] = p * (dp[hh][i] - dl);
      }
      dsp[2 * hh] = pack8(dp[hh], 0);
      dsp[2 * hh + 1] = pack8(dp[hh], 8);
    };
    // dQ^T += K^T dS^T over key blocks [bb0, bb1), A = K^T by transposing
    // reads of the K tile
    auto dq_products = [&](int bb0, int bb1) __attribute__((always_inline)) {
#pragma unroll
      for (int bb = bb0; bb < bb1; ++bb) {
        const int r = 16 * bb + trr;
#pragma unroll
        for (int nt = 0; nt < G::NQT; ++nt) {
          const int col = 64 * nt + trc;
          const bf16x8 ka = cat_tr(lds_tr(ks + dual_off<G::KROWB>(r, col)),
                                   lds_tr(ks + dual_off<G::KROWB>(r + 4, col)));
          dq[nt] = mma(ka, dsp[bb], dq[nt]);
        }
      }
    };
    constexpr int NSD = G::KK + G::VK;  // S^T and dP^T products of a half
    if constexpr (OREG) {
      // One wave per SIMD: the softmax of a half issues between products it
      // does not feed (half 0 beside the S^T/dP^T products of half 1, half
      // 1 beside the dQ products of half 0), so the vector work runs while
      // the matrix core does.
      sdp_products(0);
      pipeline_lds_mfma<NSD, 1, kBwdAhead>();
      __builtin_amdgcn_sched_barrier(0);
      mask_half(0);
      sdp_products(1);
      softmax_half(0);
      pipeline_lds_mfma_valu<NSD, 1, kBwdAhead, kSoftmaxValu / NSD + 1>();
      keep_here(dsp[0]);
      keep_here(dsp[1]);
      __builtin_amdgcn_sched_barrier(0);
      mask_half(1);
      dq_products(0, 2);
      softmax_half(1);
      pipeline_lds_mfma_valu<2 * G::NQT, 2, kBwdAhead, kSoftmaxValu / (2 * G::NQT) + 1>();
      keep_here(dsp[2]);
      keep_here(dsp[3]);
      __builtin_amdgcn_sched_barrier(0);
      dq_products(2, 4);
      pipeline_lds_mfma<2 * G::NQT, 2, kBwdAhead>();
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        sdp_products(hh);
        pipeline_lds_mfma_n<G::KK, 1, G::VK, 2, kBwdAhead>();
        __builtin_amdgcn_sched_barrier(0);
        mask_half(hh);
        softmax_half(hh);
        __builtin_amdgcn_sched_barrier(0);
      }
      dq_products(0, 4);
      pipeline_lds_mfma<4 * G::NQT, 2, kBwdAhead>();
    }
  };

  // this workgroup's tiles of the walk: the j-th is walk tile kshare + j * nks
  const int n_mine = total > kshare ? (total - kshare + nks - 1) / nks : 0;
  if (n_mine > 0) issue(lc, ks0, vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](int j, const char* ks, const char* vs, char* kn, char* vn)
      __attribute__((always_inline)) {
    if (j + 1 < n_mine) {
      advance(lc, nks);
      issue(lc, kn, vn);
    }
    tile(cc, ks, vs);
    advance(cc, nks);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int j = 0; j < n_mine; j += 2) {
    step(j, ks0, vs0, ks1, vs1);
    if (j + 1 < n_mine) step(j + 1, ks1, vs1, ks0, vs0);
  }
  if (!wave_live || !row_ok) return;

  // C: column = query row (this lane), rows = dims 32*nt + 8*(i/4) + 4g + i%4
  const float scale = a.scale;
  if (kshare == 0) {
    float* dqp = a.dq + ((int64_t)my_row * a.hq + h) * DQK;
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
  } else {
    float* dqp = a.dq_part + (((int64_t)(kshare - 1) * a.total_q + my_row) * a.hq + h) * DQK;
#pragma unroll
    for (int nt = 0; nt < G::NQT; ++nt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 x;
        x.x = scale * dq[nt][4 * q4 + 0];
        x.y = scale * dq[nt][4 * q4 + 1];
        x.z = scale * dq[nt][4 * q4 + 2];
        x.w = scale * dq[nt][4 * q4 + 3];
        *reinterpret_cast<float4*>(dqp + 32 * nt + 8 * q4 + 4 * g) = x;
      }
  }
}

// dq += the stored partials of key shares 1 .. ksplit-1, in share order,
// for every row the dQ launch covered (rows inside the q part of a segment
// whose k part is not empty).  One thread per 4 floats of a row's
// [hq, dqk] gradient; HBM-bound.
__global__ __launch_bounds__(256) void bwd_ksplit_reduce_kernel(AttnArgs a, int dqk,
                                                                 TileShares ts) {
  const int row4 = a.hq * dqk / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.total_q * row4) return;
  const int row = (int)(idx / row4), c = (int)(idx % row4);
  int lo = 0, hi = a.n_seq;  // segment of the row: cu_q[seg] <= row < cu_q[seg + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_q[mid] <= row) lo = mid; else hi = mid;
  }
  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[lo], a.cu_q[lo + 1], a.q_part, &q_lo, &q_hi);
  part_range(a.cu_k[lo], a.cu_k[lo + 1], a.k_part, &k_lo, &k_hi);
  if (k_hi <= k_lo || row < q_lo || row >= q_hi) return;
  const int64_t off = (int64_t)row * a.hq * dqk + 4 * c;
  const int64_t stride = (int64_t)a.total_q * a.hq * dqk;
  float4 acc = *reinterpret_cast<const float4*>(a.dq + off);
  // per-tile shares: this row's 128-row tile has ts.n[tile] of them
  const int ns = ts.var ? ts.n[(row - q_lo) >> 7] : a.ksplit;
  for (int s = 1; s < ns; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(a.dq_part + (s - 1) * stride + off);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  *reinterpret_cast<float4*>(a.dq + off) = acc;
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnArgs& a0, int dqk, int dv, bool causal, bool kv_split,
                                int total_k, hipStream_t st) {
  // a0.n_qtiles counts 128-row query tiles, a0.n_ktiles 128-key tiles; with
  // kv_split (d_qk = 128 only) the dK/dV kernel runs 32-key workgroups
  AttnArgs a = a0;
  if (a.ksplit < 1 || !a.dq_part) a.ksplit = 1;
  const long long nq = (long long)a.n_seq * a.hkv * a.n_qtiles * a.group * a.ksplit;
  AttnArgs ak = a;
  if (kv_split) ak.n_ktiles = 4 * a.n_ktiles;
  if (kv_split || ak.qsplit < 1) ak.qsplit = 1;
  const long long nk = (long long)a.n_seq * a.hkv * ak.n_ktiles * ak.qsplit;
  if (nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (kv_split && dqk != 128) return hipErrorInvalidValue;
  RankKV no_kv;
  RankGrad no_grad;
  memset(&no_kv, 0, sizeof(no_kv));
  memset(&no_grad, 0, sizeof(no_grad));
#define RA_BWD_LAUNCH(DQ, DVV, C, QSPLIT)                                                      \
  do {                                                                                         \
    if (nq > 0)                                                                                \
      hipLaunchKernelGGL((attn_bwd_dq_kernel<DQ, DVV, C>), dim3((unsigned)nq), dim3(NT), 0, st, \
                         a, no_kv);                                                            \
    if (nk > 0)                                                                                \
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQ, DVV, C, QSPLIT>), dim3((unsigned)nk),       \
                         dim3(NT), 0, st, ak, no_kv, no_grad);                                 \
  } while (0)
  if (dqk == 128 && dv == 128) {
    if (kv_split) {
      if (causal) RA_BWD_LAUNCH(128, 128, true, true);
      else RA_BWD_LAUNCH(128, 128, false, true);
    } else {
      if (causal) RA_BWD_LAUNCH(128, 128, true, false);
      else RA_BWD_LAUNCH(128, 128, false, false);
    }
  } else if (dqk == 192 && dv == 128) {
    if (causal) RA_BWD_LAUNCH(192, 128, true, false);
    else RA_BWD_LAUNCH(192, 128, false, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef RA_BWD_LAUNCH
  if (a.ksplit > 1 && nq > 0) {
    const long long n4 = (long long)a.total_q * a.hq * dqk / 4;
    const long long nb = (n4 + 255) / 256;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (nb > 0)
      {
      TileShares ts;
      ts.var = 0;
      hipLaunchKernelGGL(bwd_ksplit_reduce_kernel, dim3((unsigned)nb), dim3(256), 0, st, a, dqk, ts);
    }
  }
  if (ak.qsplit > 1 && nk > 0) {
    const long long n4 = (long long)total_k * a.hkv * (dqk + dv) / 4;
    const long long nb = (n4 + 255) / 256;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (nb > 0)
      hipLaunchKernelGGL(bwd_qsplit_reduce_kernel, dim3((unsigned)nb), dim3(256), 0, st, ak, dqk,
                         dv, total_k);
  }
  return hipGetLastError();
}

hipError_t launch_rank_bwd_bf16(const AttnArgs& a0, const RankKV& rk, const RankKV& rkq,
                                const RankGrad& rg, const TileShares& ts, int dqk, int dv,
                                hipStream_t st) {
  // the dQ grid is kv heads x rk.q_tiles live 128-row query tiles x group x
  // key shares, the dK/dV grid kv heads x rk.kv_tile_off[rk.cp] live
  // 128-key tiles
  AttnArgs a = a0;
  a.q_part = RA_PART_ALL;
  a.k_part = RA_PART_ALL;
  a.qsplit = 1;
  if (a.ksplit < 1 || !a.dq_part) a.ksplit = 1;
  // per-tile shares: rkq.q_tiles counts (tile, share) units
  const long long nq = (long long)a.hkv * rkq.q_tiles * a.group * (rkq.var_split ? 1 : a.ksplit);
  const long long nk = (long long)a.hkv * rk.kv_tile_off[rk.cp];
  if (nq > 0x7fffffffLL || nk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (dqk == 128 && dv == 128) {
    if (nk > 0)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<128, 128, false, false, true>), dim3((unsigned)nk),
                         dim3(NT), 0, st, a, rk, rg);
    if (nq > 0)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<128, 128, false, true>), dim3((unsigned)nq),
                         dim3(NT), 0, st, a, rkq);
  } else if (dqk == 192 && dv == 128) {
    if (nk > 0)
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<192, 128, false, false, true>), dim3((unsigned)nk),
                         dim3(NT), 0, st, a, rk, rg);
    if (nq > 0)
      hipLaunchKernelGGL((attn_bwd_dq_kernel<192, 128, false, true>), dim3((unsigned)nq),
                         dim3(NT), 0, st, a, rkq);
  } else {
    return hipErrorInvalidValue;
  }
  if (a.ksplit > 1 && nq > 0) {
    const long long n4 = (long long)a.total_q * a.hq * dqk / 4;
    const long long nb = (n4 + 255) / 256;
    if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (nb > 0)
      hipLaunchKernelGGL(bwd_ksplit_reduce_kernel, dim3((unsigned)nb), dim3(256), 0, st, a, dqk, ts);
  }
  return hipGetLastError();
}

}  // namespace ra
