// Block attention forward, bfloat16 inputs, float32 accumulation: the
// ping-pong variant for large launches (a rank's whole share).
//
// It computes exactly what attn_fwd_bf16.hip computes (the per-block
// (out, lse) of the block loop in "超长序列并行训练技术：Ulysses与Ring-Attention
// 详解", section 4.1, merged with the lse rule of section 4.2), with the
// same per-wave products on v_mfma_f32_32x32x16_bf16:
//   S^T[64 keys x 32 rows] = K_tile * Q^T
//   O^T[dv x 32 rows]     += V_tile^T * P^T
// and the same LDS layouts (fwd_tiles.h).  What differs is the schedule.
//
// A workgroup has 8 waves (256 query rows), i.e. two waves on every SIMD.
// The two waves of a SIMD take opposite roles and the workgroup alternates
// between two phases separated by barriers:
//   phase A: role-A waves run their matrix-core block (S of the current
//            tile, then P*V of the previous tile) while role-B waves run the
//            softmax of their current S on the vector ALU;
//   phase B: the other way round.
// So the matrix core of a SIMD is fed by one wave while the other wave's
// exponentials run beside it, instead of both waves hitting the same stage
// of the tile at the same time.  Roles are assigned from the hardware SIMD
// id of each wave, so the pairing holds whatever the wave placement.
//
// Both roles run the same code, one phase apart: a role-B wave passes one
// extra barrier before its first tile and a role-A wave one after its last.
// Per tile step st a wave runs
//   [matrix cores: S(st) = K(st) Q^T, O += V(st-1)^T P(st-1)^T]  barrier
//   [vector ALU:   mask and online softmax of S(st) -> P(st)]     barrier
// S goes first so that its products have landed when the softmax after the
// barrier reads them; the P*V results are not read until the next block.
// so role A computes step st in phases 2st, 2st+1 and role B in phases
// 2st+1, 2st+2.  Tile t's K is read in phases 2t and 2t+1 and its V in
// phases 2t+2 and 2t+3, so K and V have separate double buffers.  The
// matrix-core phase is the longer one, so the tile loads are issued by the
// role-B waves at the start of their vector-ALU phase: in step st (phase
// 2st+2) they load K(st+2) and V(st+1), into the buffers last read in
// phase 2st+1, and wait for them at the end of their next matrix-core phase
// (phase 2st+3), one phase before the first use.  The four buffers are
// separate LDS objects, so the compiler can tell the direct loads into one
// buffer from the reads of another and does not make the reads wait for the
// prefetch.

#include "fwd_tiles.h"

namespace ra {
namespace {

using namespace mfma;
using namespace fwd;

constexpr int PW = 8;                        // waves per workgroup
constexpr int PT = PW * 64;                  // threads per workgroup
constexpr int PBM = PW * kFwdRowsPerWave;    // 256 query rows per workgroup

// How many matrix-core products the LDS operand reads run ahead of, in the
// S = K Q^T and the P*V blocks (latency cover without the register cost of
// reading a whole tile at once).
#ifndef RA_PP_S_AHEAD
#define RA_PP_S_AHEAD 4
#endif
#ifndef RA_PP_PV_AHEAD
#define RA_PP_PV_AHEAD 4
#endif
constexpr int kSAhead = RA_PP_S_AHEAD;
constexpr int kPVAhead = RA_PP_PV_AHEAD;

// SIMD (0..3) the calling wave runs on: HW_ID register, bits 5:4.
__device__ __forceinline__ int simd_id() {
  return (int)__builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));
}

__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// MODE: 0 = one non-causal block, 1 = one causal block (as described by the
// AttnArgs parts), 2 = a rank's whole share: the C blocks of RankKV in ring
// order, merged in registers.
template <int DQK, int DV, int MODE, bool MERGE, bool OUT_BF16>
__global__ __launch_bounds__(PT, 1) void attn_fwd_pp_kernel(AttnArgs a, RankKV rk, int n_qtiles) {
  using G = Geo<DQK, DV>;
  __shared__ __attribute__((aligned(1024))) char ks0[G::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char ks1[G::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs0[G::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs1[G::V_BYTES];
  __shared__ int simd_of[PW];

  const int nb = gridDim.x;
  const int group = a.group;
  // causal work only (one causal block, or a rank share of one block), or a
  // rank share of packed documents: deal query tiles over the XCDs;
  // otherwise contiguous ranges per XCD
  const bool causal_only = MODE == 1 || (MODE == 2 && (rk.cp == 1 || a.n_seq > 1));
  int b = causal_only ? xcd_deal(blockIdx.x, nb, group) : xcd_remap(blockIdx.x, nb);
  const int hg = b % group;
  b /= group;
  int kvh, seg, qt;
  if (MODE == 2 && a.n_seq > 1) {
    // packed documents: only live tiles, the kv heads of one tile
    // together, segment by segment with each segment's heaviest tile first,
    // taken in the host's heaviest-first order of tiles (tile_ordered 1) or
    // of segments (2)
    kvh = b % a.hkv;
    const int u = b / a.hkv;
    const int j = rk.tile_ordered == 1 ? (int)rk.tile_order[u] : u;
    auto seg_at = [&](int s) { return rk.tile_ordered == 2 ? (int)rk.tile_order[s] : s; };
    auto count = [&](int s) {
      s = seg_at(s);
      const int len = a.cu_q[s + 1] - a.cu_q[s], half = len >> 1;
      return a.half_tiles ? (half + PBM - 1) / PBM + (len - half + PBM - 1) / PBM
                          : (len + PBM - 1) / PBM;
    };
    int idx, cnt;
    if (!locate_in_segments(a.n_seq, j, count, &seg, &idx, &cnt)) return;
    seg = seg_at(seg);
    qt = cnt - 1 - idx;
  } else {
    const int qt_rev = b % n_qtiles;
    b /= n_qtiles;
    kvh = b % a.hkv;
    seg = b / a.hkv;
    qt = MODE != 0 ? (n_qtiles - 1 - qt_rev) : qt_rev;  // heaviest first
  }
  const int h = kvh * group + hg;

  int q_lo, q_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], MODE == 2 ? RA_PART_ALL : a.q_part, &q_lo, &q_hi);
  const int qhalf = (q_hi - q_lo) >> 1;
  // the tile's rows [q0, t_hi): tiles over the whole segment, or (half
  // tiles) over each zig-zag chunk on its own, so that no tile straddles
  // the two and blocks seen by the second chunk only skip whole tiles
  int q0 = q_lo + qt * PBM, t_hi = q_hi;
  if (MODE == 2 && a.half_tiles) {
    const int nh = (qhalf + PBM - 1) / PBM;
    if (qt < nh) {
      t_hi = q_lo + qhalf;
    } else {
      q0 = q_lo + qhalf + (qt - nh) * PBM;
    }
  }
  if (q0 >= t_hi) return;  // whole workgroup

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int qrel_last_wg = min(q0 + PBM, t_hi) - 1 - q_lo;
  const int wq0 = q0 + wave * kFwdRowsPerWave;
  const bool wave_live = wq0 < t_hi;
  const int wq_first_rel = wq0 - q_lo;
  const int wq_last_rel = min(wq0 + kFwdRowsPerWave, t_hi) - 1 - q_lo;
  const int my_row = wq0 + l32;
  const int my_row_rel = my_row - q_lo;
  const int64_t ks_bytes = a.k_stride * 2, vs_bytes = a.v_stride * 2;
  const int nblocks = MODE == 2 ? rk.cp : 1;
  const int kseg0 = a.cu_k[seg], kseg1 = a.cu_k[seg + 1];

  auto get_block = [&](int bi) -> Block {
    Block blk;
    const void* kp;
    const void* vp;
    int kpart;
    if (MODE == 2) {
      const int owner = (rk.rank - bi + rk.cp) % rk.cp;
      kp = rk.k[owner];
      vp = rk.v[owner];
      blk.kind = bi == 0 ? KIND_CAUSAL : (owner < rk.rank ? KIND_ALL : KIND_LATE_ROWS);
      kpart = (bi != 0 && owner < rk.rank) ? RA_PART_FIRST_HALF : RA_PART_ALL;
    } else {
      kp = a.k;
      vp = a.v;
      blk.kind = MODE == 1 ? KIND_CAUSAL : KIND_ALL;
      kpart = a.k_part;
    }
    int k_lo, k_hi;
    part_range(kseg0, kseg1, kpart, &k_lo, &k_hi);
    blk.klen = k_hi - k_lo;
    blk.diag = 0;
    blk.kb = reinterpret_cast<const char*>(kp) + ((int64_t)k_lo * a.k_stride + (int64_t)kvh * DQK) * 2;
    blk.vb = reinterpret_cast<const char*>(vp) + ((int64_t)k_lo * a.v_stride + (int64_t)kvh * DV) * 2;
    int kend = blk.klen;
    if (blk.kind == KIND_CAUSAL) kend = min(blk.klen, qrel_last_wg + 1);
    if (blk.kind == KIND_LATE_ROWS && qrel_last_wg < qhalf) kend = 0;
    blk.ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
    return blk;
  };

  struct Cursor {
    int bi, t;
    Block blk;
  };
  auto first = [&](Cursor& c) {
    c.bi = 0;
    c.t = 0;
    c.blk = get_block(0);
    while (c.blk.ntiles == 0 && c.bi + 1 < nblocks) c.blk = get_block(++c.bi);
  };
  auto advance = [&](Cursor& c) {
    if (++c.t < c.blk.ntiles) return;
    c.t = 0;
    do {
      if (++c.bi >= nblocks) return;
      c.blk = get_block(c.bi);
    } while (c.blk.ntiles == 0);
  };
  int total = 0;
  for (int bi = 0; bi < nblocks; ++bi) total += get_block(bi).ntiles;
  if (total == 0 && MERGE) return;  // whole workgroup: merging nothing is the identity

  // role: on each SIMD the waves alternate A, B, A, ... in wave order;
  // b_rank numbers the role-B waves 0..3, which load the tiles
  if (lane == 0) simd_of[wave] = simd_id();
  __syncthreads();
  int role_b, b_rank;
  {
    int rb[PW];
    int n_b = 0;
#pragma unroll
    for (int w = 0; w < PW; ++w) {
      int same = 0;
#pragma unroll
      for (int w2 = 0; w2 < w; ++w2) same += simd_of[w2] == simd_of[w] ? 1 : 0;
      rb[w] = same & 1;
      n_b += rb[w];
    }
    // waves not spread two per SIMD: pair by wave index (correct, less overlap)
    if (n_b != PW / 2) {
#pragma unroll
      for (int w = 0; w < PW; ++w) rb[w] = w >= PW / 2 ? 1 : 0;
    }
    int mine = 0, before = 0;
#pragma unroll
    for (int w = 0; w < PW; ++w) {
      mine = w == wave ? rb[w] : mine;
      before += (w < wave && rb[w]) ? 1 : 0;
    }
    role_b = __builtin_amdgcn_readfirstlane(mine);
    b_rank = __builtin_amdgcn_readfirstlane(before);
  }

  TileLoader<DQK, DV, PW / 2> ld;
  ld.init(ks_bytes, vs_bytes, b_rank & (PW / 2 - 1), lane);
  // kc: next K tile to load, vc: next V tile to load, cc: next S tile
  Cursor kc, vc, cc;
  first(kc);
  vc = kc;
  cc = kc;
  auto load_k = [&](char* dst) {
    ld.issue_k(kc.blk.kb + (int64_t)kc.t * BN * ks_bytes, ks_bytes, kc.blk.klen - kc.t * BN, dst);
    advance(kc);
  };
  auto load_v = [&](char* dst) {
    ld.issue_v(vc.blk.vb + (int64_t)vc.t * BN * vs_bytes, vs_bytes, vc.blk.klen - vc.t * BN, dst);
    advance(vc);
  };
  // K(0), K(1) and V(0) before the loop
  if (role_b) {
    if (total > 0) load_k(ks0);
    if (total > 1) load_k(ks1);
    if (total > 0) load_v(vs0);
  }

  bf16x8 qf[G::KK];
  {
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + (int64_t)h * DQK;
    const int row = min(my_row, t_hi - 1);
    const __bf16* qp = qb + (int64_t)row * a.q_stride + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) qf[kk] = as_bf16x8(ldg16(qp + 16 * kk));
  }

  f32x16 o[G::OT];
#pragma unroll
  for (int t = 0; t < G::OT; ++t) o[t] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = a.scale_log2;

  int koff[4];
  {
    const int r = sigma(l32);
#pragma unroll
    for (int q = 0; q < 4; ++q) koff[q] = r * 128 + (k_slot(r, 2 * q + g) << 4);
  }
  int voff[2][G::OT];
  {
    const int trr = tr_row(lane), trc = tr_col_bytes(lane);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int tt = 0; tt < G::OT; ++tt) voff[h2][tt] = v_off<G::VROWB>(trr + 4 * h2, 64 * tt + trc);
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // S tile in flight between the matrix-core block and the softmax
  f32x16 s[2];
  bf16x8 p[4];
  int s_kt0 = 0, s_klen = 0, s_kind = 0;
  bool s_live = false, s_mask = false, p_live = false;

  // ---- S^T = K * Q^T of the next tile (matrix cores)
  auto gemm_s = [&](const char* kbuf) __attribute__((always_inline)) {
    s_kt0 = cc.t * BN;
    s_klen = cc.blk.klen;
    s_kind = cc.blk.kind;
    bool live = wave_live, need_mask;
    if (s_kind == KIND_CAUSAL) {
      live = live && s_kt0 <= wq_last_rel;
      need_mask = (s_kt0 + BN > s_klen) || (s_kt0 + BN - 1 > wq_first_rel);
    } else if (s_kind == KIND_LATE_ROWS) {
      live = live && wq_last_rel >= qhalf;
      need_mask = (s_kt0 + BN > s_klen) || (wq_first_rel < qhalf);
    } else {
      need_mask = s_kt0 + BN > s_klen;
    }
    s_live = live;
    s_mask = need_mask;
    advance(cc);
    if (!live) return;
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 kv = lds16(kbuf + koff[kk & 3] + (kk >> 2) * G::KPANEL_BYTES + hh * 32 * 128);
        s[hh] = mma(as_bf16x8(kv), qf[kk], s[hh]);
      }
    // keep LDS reads kSAhead products ahead of the matrix core
    constexpr int NM = 2 * G::KK;
    __builtin_amdgcn_sched_group_barrier(0x100, kSAhead, 0);
#pragma unroll
    for (int i = 0; i < NM - kSAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kSAhead, 0);
  };

  // ---- O^T += V^T * P^T of the previous tile (matrix cores)
  auto gemm_pv = [&](const char* vbuf) __attribute__((always_inline)) {
    if (!p_live) return;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int tt = 0; tt < G::OT; ++tt) {
        const char* vp = vbuf + bb * 16 * G::VROWB;
        const bf16x8 va = cat_tr(lds_tr(vp + voff[0][tt]), lds_tr(vp + voff[1][tt]));
        o[tt] = mma(va, p[bb], o[tt]);
      }
    // two transposing reads per product, kPVAhead products ahead
    constexpr int NM = 4 * G::OT;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPVAhead, 0);
#pragma unroll
    for (int i = 0; i < NM - kPVAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPVAhead, 0);
  };

  // ---- mask + online softmax of the current S tile (vector ALU)
  auto softmax = [&]() __attribute__((always_inline)) {
    p_live = s_live;
    if (!s_live) return;
    if (s_mask) {
      // last visible key of the row, relative to the lane's first key
      const int base = s_kt0 + (g << 3);
      int lim = s_klen - 1 - base;
      if (s_kind == KIND_CAUSAL) lim = min(lim, my_row_rel - base);
      if (s_kind == KIND_LATE_ROWS && my_row_rel < qhalf) lim = -1;
      mask_scores(s[0], s[1], lim);
    }
    online_softmax_tile(s[0], s[1], c2, m_run, l_run, o, p);
  };

  // One tile step st (two phases).  K(st) is in kcur, V(st-1) in vprev.
  // Role-B waves wait for their loads of K(st+1), V(st) at the end of the
  // matrix-core phase, then load K(st+2) into kcur and V(st+1) into vprev.
  auto step = [&](const int st, char* kcur, char* vprev) __attribute__((always_inline)) {
    if (st < total) gemm_s(kcur);
    __builtin_amdgcn_sched_barrier(0);
    if (st >= 1) gemm_pv(vprev);
    if (role_b) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    phase_barrier();
    if (role_b) {
      if (st + 2 < total) load_k(kcur);
      if (st + 1 < total) load_v(vprev);
    }
    if (st < total) softmax();
    phase_barrier();
  };
  if (role_b) phase_barrier();
  for (int st = 0; st <= total; st += 2) {
    step(st, ks0, vs1);
    if (st + 1 <= total) step(st + 1, ks1, vs0);
  }
  if (!role_b) phase_barrier();

  if (!wave_live || my_row >= t_hi) return;

  // ---- epilogue: lanes l and l^32 hold the two key halves of the same row
  const float l_tot = xhalf_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
  const float lse =
      empty ? -INFINITY : (m_fin * a.scale + __builtin_amdgcn_logf(l_tot) * 0.69314718055994531f);

  float* lrow = a.lse + (int64_t)h * a.total_q + my_row;
  if (OUT_BF16) {
    unsigned short* orow = reinterpret_cast<unsigned short*>(a.out) + ((int64_t)my_row * a.hq + h) * DV;
#pragma unroll
    for (int tt = 0; tt < G::OT; ++tt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 w;
        w.x = pack_bf16x2(o[tt][4 * q4 + 0] * inv, o[tt][4 * q4 + 1] * inv);
        w.y = pack_bf16x2(o[tt][4 * q4 + 2] * inv, o[tt][4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * tt + 8 * q4 + 4 * g) = w;
      }
    if (g == 0) *lrow = lse;
  } else if (!MERGE) {
    float* orow = a.out + ((int64_t)my_row * a.hq + h) * DV;
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
    float* orow = a.out + ((int64_t)my_row * a.hq + h) * DV;
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
        float4* pp = reinterpret_cast<float4*>(orow + 32 * tt + 8 * q4 + 4 * g);
        float4 acc = *pp;
        acc.x = ca * acc.x + cb * o[tt][4 * q4 + 0];
        acc.y = ca * acc.y + cb * o[tt][4 * q4 + 1];
        acc.z = ca * acc.z + cb * o[tt][4 * q4 + 2];
        acc.w = ca * acc.w + cb * o[tt][4 * q4 + 3];
        *pp = acc;
      }
    if (g == 0) *lrow = lnew;
  }
}

template <int DQK, int DV>
hipError_t launch_pp_t(const AttnArgs& a, const RankKV* rk, bool causal, bool merge,
                       bool out_bf16, hipStream_t st) {
  // query tiles of 256 rows from the 128-row count the host computed, or
  // the host's count of half tiles
  const int nq = (rk && a.half_tiles) ? a.n_qtiles_half : (a.n_qtiles + 1) / 2;
  // a packed rank share lists live tiles only (rk->fwd_tiles over all
  // segments), the kv heads of one tile together
  const long long nblk = (rk && a.n_seq > 1) ? (long long)rk->fwd_tiles * a.hkv * a.group
                                             : (long long)a.n_seq * a.hkv * nq * a.group;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nblk), block(PT);
  RankKV none;
  none.cp = 0;
  none.rank = 0;
  if (rk) {
    if (out_bf16)
      hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV, 2, false, true>), grid, block, 0, st, a, *rk, nq);
    else
      hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV, 2, false, false>), grid, block, 0, st, a, *rk, nq);
  } else if (causal) {
    if (merge) hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV, 1, true, false>), grid, block, 0, st, a, none, nq);
    else hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV, 1, false, false>), grid, block, 0, st, a, none, nq);
  } else {
    if (merge) hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV, 0, true, false>), grid, block, 0, st, a, none, nq);
    else hipLaunchKernelGGL((attn_fwd_pp_kernel<DQK, DV, 0, false, false>), grid, block, 0, st, a, none, nq);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_pp(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                              hipStream_t st) {
  if (dqk == 128 && dv == 128) return launch_pp_t<128, 128>(a, nullptr, causal, merge, false, st);
  if (dqk == 192 && dv == 128) return launch_pp_t<192, 128>(a, nullptr, causal, merge, false, st);
  if (dqk == 64 && dv == 64) return launch_pp_t<64, 64>(a, nullptr, causal, merge, false, st);
  return hipErrorInvalidValue;
}

hipError_t launch_rank_fwd_pp(const AttnArgs& a, const RankKV& rk, int dqk, int dv, bool out_bf16,
                              hipStream_t st) {
  if (dqk == 128 && dv == 128) return launch_pp_t<128, 128>(a, &rk, true, false, out_bf16, st);
  if (dqk == 192 && dv == 128) return launch_pp_t<192, 128>(a, &rk, true, false, out_bf16, st);
  if (dqk == 64 && dv == 64) return launch_pp_t<64, 64>(a, &rk, true, false, out_bf16, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
