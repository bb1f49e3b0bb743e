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
// with the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//
// K/V tiles go from global memory straight into LDS with the XOR-swizzled
// layouts of fwd_tiles.h, double-buffered: tile t+1 streams in while tile t
// is computed, with one barrier per tile.
//
// Blocks are remapped so that each of the 8 XCDs gets a contiguous range of
// tiles ordered (segment, kv head, query tile, head in group): the query
// heads sharing a kv head, and neighbouring query tiles, read the same K/V
// through the same L2.  Causal launches order query tiles heaviest first and
// deal (query tile x kv group) units round-robin over the XCDs instead, so
// that every XCD gets light and heavy tiles.

#include "fwd_tiles.h"

namespace ra {
namespace {

using namespace mfma;
using namespace fwd;

// Lazy-rescale threshold (log2 units) of the d_qk = 192 softmax below, the
// same as online_softmax_tile's: the running max is raised only when a
// row's max grows by more than this; numerator, row sum and lse use the
// same (possibly stale) max, so the result is exact.
constexpr float kRescaleLog2 = 8.0f;

constexpr int BM = kFwdBlockM;
constexpr int NW = kFwdWaves;
constexpr int NT = NW * 64;

// MODE: 0 = one non-causal block, 1 = one causal block (both as described by
// the AttnArgs parts), 2 = a rank's whole share: the C blocks of RankKV in
// ring order, merged in registers (no partials, no separate merge), 3 = a
// rectangle list (AttnArgs::segs): "segment" s is rectangle s, with its own
// query rows, key range and diagonal offset (other shard maps).
template <int DQK, int DV, int MODE, bool MERGE, bool OUT_BF16>
__global__ __launch_bounds__(NT, 2) void attn_fwd_bf16_kernel(AttnArgs a, RankKV rk) {
  using G = Geo<DQK, DV>;
  // two stages as separate objects: the compiler can then tell that the
  // direct loads into one stage never alias the reads of the other, and
  // does not wait for the prefetch before reading the current tile
  __shared__ __attribute__((aligned(1024))) char smem0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[G::STAGE];

  const int nb = gridDim.x;
  const int group = a.group;
  // causal work only (one causal block, or a rank share of one block), or a
  // rank share of packed documents (units of very unequal size, one
  // document's after another in logical order): deal query tiles over the
  // XCDs; otherwise contiguous ranges per XCD
  const bool causal_only =
      MODE == 1 || MODE == 3 || (MODE == 2 && (rk.cp == 1 || a.n_seq > 1 || rk.var_split));
  int b = causal_only ? xcd_deal(blockIdx.x, nb, group) : xcd_remap(blockIdx.x, nb);
  const int hg = b % group;
  b /= group;
  // kv_part of kv_split: part of a KV-split rank share; with a KV split this
  // workgroup takes every kv_split-th key tile of the share's tile
  // sequence, starting at tile kv_part
  int kvh, seg, kv_part = 0, qt, kv_split = MODE == 2 ? max(rk.split, 1) : 1;
  if (MODE == 2 && rk.var_split) {
    // per-tile parts, heaviest part first, the kv heads of one unit together
    kvh = b % a.hkv;
    const int e = rk.tile_order[b / a.hkv];
    seg = 0;
    qt = e >> 6;
    kv_part = (e >> 3) & 7;
    kv_split = (e & 7) + 1;
  } else if (MODE == 2 && a.n_seq > 1) {
    // packed documents: only live tiles, the kv heads of one tile together,
    // segment by segment with each segment's heaviest tile first, taken in
    // the host's heaviest-first order of tiles (tile_ordered 1) or of
    // segments (2); parts slowest
    kvh = b % a.hkv;
    b /= a.hkv;
    const int u = b % rk.fwd_tiles;
    kv_part = b / rk.fwd_tiles;
    const int j = rk.tile_ordered == 1 ? (int)rk.tile_order[u] : u;
    auto seg_at = [&](int s) { return rk.tile_ordered == 2 ? (int)rk.tile_order[s] : s; };
    auto count = [&](int s) {
      s = seg_at(s);
      return (a.cu_q[s + 1] - a.cu_q[s] + BM - 1) / BM;
    };
    int idx, cnt;
    if (!locate_in_segments(a.n_seq, j, count, &seg, &idx, &cnt)) return;
    seg = seg_at(seg);
    qt = cnt - 1 - idx;
  } else {
    const int qt_rev = b % a.n_qtiles;
    b /= a.n_qtiles;
    kvh = b % a.hkv;
    b /= a.hkv;
    seg = MODE == 2 ? b % a.n_seq : b;
    kv_part = MODE == 2 ? b / a.n_seq : 0;
    // heaviest query tiles first (causal: later rows see more keys; rank
    // share: second-half rows also see the blocks of later ranks)
    qt = MODE != 0 ? (a.n_qtiles - 1 - qt_rev) : qt_rev;
  }
  const int h = kvh * group + hg;

  int q_lo, q_hi, kseg0, kseg1, seg_diag = 0;
  if (MODE == 3) {
    const ra_segment sg = a.segs[seg];
    q_lo = sg.q_lo;
    q_hi = sg.q_hi;
    kseg0 = sg.k_lo;
    kseg1 = sg.k_hi;
    seg_diag = sg.diag;
  } else {
    part_range(a.cu_q[seg], a.cu_q[seg + 1], MODE == 2 ? RA_PART_ALL : a.q_part, &q_lo, &q_hi);
    // key segment bounds, read once: a vector load inside the tile loop
    // would make the wave wait for its outstanding prefetch
    kseg0 = a.cu_k[seg];
    kseg1 = a.cu_k[seg + 1];
  }
  const int q0 = q_lo + qt * BM;
  if (q0 >= q_hi) return;
  const int qhalf = (q_hi - q_lo) >> 1;  // second-half rows start here (part-relative)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int qrel_last_wg = min(q0 + BM, q_hi) - 1 - q_lo;
  const int wq0 = q0 + wave * kFwdRowsPerWave;
  const bool wave_live = wq0 < q_hi;
  const int wq_first_rel = wq0 - q_lo;
  const int wq_last_rel = min(wq0 + kFwdRowsPerWave, q_hi) - 1 - q_lo;
  const int my_row = wq0 + l32;
  const int my_row_rel = my_row - q_lo;
  const int64_t ks_bytes = a.k_stride * 2, vs_bytes = a.v_stride * 2;
  // a rank share's blocks (ring steps), or the one block
  const int nblocks = MODE == 2 ? rk.cp : 1;

  // block bi of this workgroup, with the number of key tiles it visits
  auto get_block = [&](int bi) -> Block {
    Block blk;
    const void* kp;
    const void* vp;
    int kpart;
    if (MODE == 2) {
      const int owner = (rk.rank - bi + rk.cp) % rk.cp;
      kp = rk.k[owner];
      vp = rk.v[owner];
      // diagonal: causal; earlier owners: all rows x their first half;
      // later owners: second-half rows x all their keys
      blk.kind = bi == 0 ? KIND_CAUSAL : (owner < rk.rank ? KIND_ALL : KIND_LATE_ROWS);
      kpart = (bi != 0 && owner < rk.rank) ? RA_PART_FIRST_HALF : RA_PART_ALL;
    } else {
      kp = a.k;
      vp = a.v;
      blk.kind = MODE == 1 ? KIND_CAUSAL : KIND_ALL;
      kpart = MODE == 3 ? RA_PART_ALL : a.k_part;
    }
    int k_lo, k_hi;
    part_range(kseg0, kseg1, kpart, &k_lo, &k_hi);
    blk.klen = k_hi - k_lo;
    blk.diag = 0;
    if (MODE == 3) {
      blk.kind = seg_diag >= blk.klen ? KIND_ALL : KIND_CAUSAL;
      blk.diag = seg_diag;
    }
    blk.kb = reinterpret_cast<const char*>(kp) + ((int64_t)k_lo * a.k_stride + (int64_t)kvh * DQK) * 2;
    blk.vb = reinterpret_cast<const char*>(vp) + ((int64_t)k_lo * a.v_stride + (int64_t)kvh * DV) * 2;
    int kend = blk.klen;
    if (blk.kind == KIND_CAUSAL) kend = min(blk.klen, qrel_last_wg + blk.diag + 1);
    if (blk.kind == KIND_LATE_ROWS && qrel_last_wg < qhalf) kend = 0;
    blk.ntiles = kend > 0 ? (kend + BN - 1) / BN : 0;
    return blk;
  };

  // cursors over the (block, tile) sequence: one for loads, one tile ahead
  // of the one for compute
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
  // the part's next tile: split tiles on
  auto advance_part = [&](Cursor& c) {
    for (int i = 0; i < kv_split; ++i) advance(c);
  };
  int total_all = 0;
  for (int bi = 0; bi < nblocks; ++bi) total_all += get_block(bi).ntiles;
  const int total = total_all > kv_part ? (total_all - kv_part + kv_split - 1) / kv_split : 0;
  if (total == 0 && MERGE) return;  // merging an empty block is the identity

  TileLoader<DQK, DV, NW> ld;
  ld.init(ks_bytes, vs_bytes, wave, lane);
  Cursor lc, cc;
  first(lc);
  for (int i = 0; i < kv_part; ++i) advance(lc);
  cc = lc;
  auto issue_next = [&](char* stage) {
    ld.issue_k(lc.blk.kb + (int64_t)lc.t * BN * ks_bytes, ks_bytes, lc.blk.klen - lc.t * BN, stage);
    ld.issue_v(lc.blk.vb + (int64_t)lc.t * BN * vs_bytes, vs_bytes, lc.blk.klen - lc.t * BN,
               stage + G::K_BYTES);
    advance_part(lc);
  };
  // the first K/V tile streams in while Q is fetched
  if (total > 0) issue_next(smem0);

  // Q^T operand: lane holds row my_row, dims 16*kk + 8*g .. +7
  bf16x8 qf[G::KK];
  {
    const __bf16* qb = reinterpret_cast<const __bf16*>(a.q) + (int64_t)h * DQK;
    const int row = min(my_row, q_hi - 1);
    const __bf16* qp = qb + (int64_t)row * a.q_stride + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) qf[kk] = as_bf16x8(ldg16(qp + 16 * kk));
  }

  f32x16 o[G::OT];
#pragma unroll
  for (int t = 0; t < G::OT; ++t) o[t] = zero16();
  float m_run = -INFINITY;  // running max of raw scores (possibly stale, see above)
  float l_run = 0.f;        // running sum of this lane's 16-key halves
  const float c2 = a.scale_log2;

  // per-lane LDS read offsets; K rows +32 and V rows +16 keep the swizzle
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

  auto tile = [&](const int gi, char* const stage, char* const next) __attribute__((always_inline)) {
    if (gi + 1 < total) issue_next(next);
    const int kt0 = cc.t * BN;  // relative to the block's first key
    const int klen = cc.blk.klen, kind = cc.blk.kind, diag = cc.blk.diag;
    // rows of this wave the tile can reach, and whether scores need a mask
    bool live = wave_live, need_mask;
    if (kind == KIND_CAUSAL) {
      live = live && kt0 <= wq_last_rel + diag;
      need_mask = (kt0 + BN > klen) || (kt0 + BN - 1 > wq_first_rel + diag);
    } else if (kind == KIND_LATE_ROWS) {
      live = live && wq_last_rel >= qhalf;
      need_mask = (kt0 + BN > klen) || (wq_first_rel < qhalf);
    } else {
      need_mask = kt0 + BN > klen;
    }
    if (live) {
      const char* ks = stage;
      const char* vsm = stage + G::K_BYTES;
      // ---- S^T = K * Q^T : two 32-key halves
      f32x16 s[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        s[hh] = zero16();
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
          const u32x4 kv = lds16(ks + koff[kk & 3] + (kk >> 2) * G::KPANEL_BYTES + hh * 32 * 128);
          s[hh] = mma(as_bf16x8(kv), qf[kk], s[hh]);
        }
      }
      // ---- mask (tiles crossing the causal diagonal, a part end, or the
      // segment's half for second-half-only blocks)
      // At d_qk = 128 one key limit per lane and a select per score; at
      // d_qk = 192 the per-score conditions (measured 1% faster there, the
      // select form 19% faster on the many masked tiles of short packed
      // documents at d_qk = 128).
      if (need_mask && DQK <= 128) {
        // last visible key of the row, relative to the lane's first key
        const int base = kt0 + (g << 3);
        int lim = klen - 1 - base;
        if (kind == KIND_CAUSAL) lim = min(lim, my_row_rel + diag - base);
        if (kind == KIND_LATE_ROWS && my_row_rel < qhalf) lim = -1;
        mask_scores(s[0], s[1], lim);
      } else if (need_mask) {
        const bool row_ok = kind != KIND_LATE_ROWS || my_row_rel >= qhalf;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kr = kt0 + 32 * hh + ((i >> 3) << 4) + (g << 3) + (i & 7);
            const bool ok = row_ok && (kr < klen) && (kind != KIND_CAUSAL || kr <= my_row_rel + diag);
            if (!ok) s[hh][i] = -INFINITY;
          }
      }
      // ---- online softmax (log2 domain, lazily rescaled).  At d_qk = 128
      // P is taken against the running max first (the row max only when
      // needed); at d_qk = 192, where the S products take longer and the
      // softmax is a smaller share of a tile, the row max goes first and
      // the bf16 packing of P runs between the P*V products instead of
      // ahead of them (measured faster there).
      bf16x8 pk[4];
      if constexpr (DQK <= 128) {
        online_softmax_tile(s[0], s[1], c2, m_run, l_run, o, pk);
      } else {
        // row max as pairwise maxima folded three at a time: more
        // instructions than one v_max3 chain, but a shorter dependency path
        // (nothing else runs beside it in this kernel)
        auto mx3 = [](float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); };
        float mx = mx3(s[0][0], s[0][1], s[0][2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = mx3(mx, s[0][i], s[0][i + 1]);
        mx = mx3(mx, s[0][15], s[1][0]);
#pragma unroll
        for (int i = 1; i < 15; i += 2) mx = mx3(mx, s[1][i], s[1][i + 1]);
        mx = xhalf_max(fmaxf(mx, s[1][15]));
        const bool raise = (mx - m_run) * c2 > kRescaleLog2;  // true on the first live tile
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
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[hh][i], c2, -mc));
            if (i & 1) rs1 += pv; else rs0 += pv;
            s[hh][i] = pv;
          }
        l_run += rs0 + rs1;
      }
      // ---- O^T += V^T * P^T : 4 k-steps of 16 keys
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const bf16x8 pb = DQK <= 128 ? pk[bb] : pack8(s[bb >> 1], 8 * (bb & 1));
#pragma unroll
        for (int tt = 0; tt < G::OT; ++tt) {
          const char* vp = vsm + bb * 16 * G::VROWB;
          const bf16x8 va = cat_tr(lds_tr(vp + voff[0][tt]), lds_tr(vp + voff[1][tt]));
          o[tt] = mma(va, pb, o[tt]);
        }
      }
    }
    advance_part(cc);
    // next tile landed (own loads) and every wave is done with this one
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int gi = 0; gi < total; gi += 2) {
    tile(gi, smem0, smem1);
    if (gi + 1 < total) tile(gi + 1, smem1, smem0);
  }

  if (!wave_live || my_row >= q_hi) return;

  // ---- epilogue: lanes l and l^32 hold the two key halves of the same row
  const float l_tot = xhalf_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const float m_fin = (m_run == -INFINITY) ? 0.f : m_run;
  const float lse =
      empty ? -INFINITY : (m_fin * a.scale + __builtin_amdgcn_logf(l_tot) * 0.69314718055994531f);

  float* const out_base = a.out + (MODE == 2 ? kv_part * rk.part_out_stride : 0);
  float* lrow = a.lse + (MODE == 2 ? kv_part * rk.part_lse_stride : 0) + (int64_t)h * a.total_q +
                my_row;
  if (MODE == 2 && rk.var_split && kv_part == 0 && g == 0) {
    // partial slots past this tile's parts hold nothing: the combine skips them
    for (int p = kv_split; p < rk.split; ++p) lrow[p * rk.part_lse_stride] = -INFINITY;
  }
  if (OUT_BF16) {
    // final output straight to bf16 (round to nearest even)
    unsigned short* orow = reinterpret_cast<unsigned short*>(out_base) + ((int64_t)my_row * a.hq + h) * DV;
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
    float* orow = out_base + ((int64_t)my_row * a.hq + h) * DV;
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
    float* orow = out_base + ((int64_t)my_row * a.hq + h) * DV;
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
hipError_t launch_t(const AttnArgs& a, const RankKV* rk, bool causal, bool merge, bool out_bf16,
                    hipStream_t st) {
  const int split = rk ? max(rk->split, 1) : 1;
  if (rk && split > 1 && out_bf16) return hipErrorInvalidValue;  // parts are float32
  // a packed rank share lists live tiles only (rk->fwd_tiles over all
  // segments)
  const long long nblk = (rk && rk->var_split)
                             ? (long long)rk->fwd_tiles * a.hkv * a.group
                         : (rk && a.n_seq > 1)
                             ? (long long)rk->fwd_tiles * a.hkv * a.group * split
                             : (long long)a.n_seq * a.hkv * a.n_qtiles * a.group * split;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nblk), block(NT);
  RankKV none;
  none.cp = 0;
  none.rank = 0;
  if (rk) {
    if (out_bf16)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 2, false, true>), grid, block, 0, st, a, *rk);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 2, false, false>), grid, block, 0, st, a, *rk);
  } else if (causal) {
    if (merge) hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 1, true, false>), grid, block, 0, st, a, none);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 1, false, false>), grid, block, 0, st, a, none);
  } else {
    if (merge) hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 0, true, false>), grid, block, 0, st, a, none);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 0, false, false>), grid, block, 0, st, a, none);
  }
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_seg_t(const AttnArgs& a, bool merge, hipStream_t st) {
  const long long nblk = (long long)a.n_seq * a.hkv * a.n_qtiles * a.group;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nblk), block(NT);
  RankKV none;
  none.cp = 0;
  none.rank = 0;
  if (merge) hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 3, true, false>), grid, block, 0, st, a, none);
  else hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, DV, 3, false, false>), grid, block, 0, st, a, none);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_segments(const AttnArgs& a, int dqk, int dv, bool merge,
                                    hipStream_t st) {
  if (dqk == 128 && dv == 128) return launch_seg_t<128, 128>(a, merge, st);
  if (dqk == 192 && dv == 128) return launch_seg_t<192, 128>(a, merge, st);
  if (dqk == 64 && dv == 64) return launch_seg_t<64, 64>(a, merge, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                                hipStream_t st) {
  if (dqk == 128 && dv == 128) return launch_t<128, 128>(a, nullptr, causal, merge, false, st);
  if (dqk == 192 && dv == 128) return launch_t<192, 128>(a, nullptr, causal, merge, false, st);
  if (dqk == 64 && dv == 64) return launch_t<64, 64>(a, nullptr, causal, merge, false, st);
  return hipErrorInvalidValue;
}

hipError_t launch_rank_fwd_bf16(const AttnArgs& a, const RankKV& rk, int dqk, int dv, bool out_bf16,
                                hipStream_t st) {
  if (dqk == 128 && dv == 128) return launch_t<128, 128>(a, &rk, true, false, out_bf16, st);
  if (dqk == 192 && dv == 128) return launch_t<192, 128>(a, &rk, true, false, out_bf16, st);
  if (dqk == 64 && dv == 64) return launch_t<64, 64>(a, &rk, true, false, out_bf16, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
