// Block attention forward in float32 throughout (float32 inputs, float32
// arithmetic, no matrix cores, no reduced-precision rounding of P).
//
// Same contract as the bf16 kernel (the per-block (out, lse) of the block
// loop in "超长序列并行训练技术：Ulysses与Ring-Attention详解", section 4.1):
// one wave per (segment, 64-row query tile, query head), one query row per
// lane held in registers; 32-key tiles of K and V are staged in LDS and read
// by every lane at the same address (LDS broadcast).  Per tile the lane
// forms its 32 scores, takes their max, rescales its running output once
// and accumulates exp(s - m) v.  exp/log are the accurate float32 library
// functions.

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int BM = kF32BlockM;
constexpr int BN = kF32BlockN;

template <int DQK, int DV, bool CAUSAL, bool MERGE>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnArgs a) {
  __shared__ float ks[BN][DQK];
  __shared__ float vs[BN][DV];

  int b = blockIdx.x;
  const int h = b % a.hq;
  b /= a.hq;
  const int qt = b % a.n_qtiles;
  const int seg = b / a.n_qtiles;
  const int kvh = h / a.group;

  int q_lo, q_hi, k_lo, k_hi;
  part_range(a.cu_q[seg], a.cu_q[seg + 1], a.q_part, &q_lo, &q_hi);
  part_range(a.cu_k[seg], a.cu_k[seg + 1], a.k_part, &k_lo, &k_hi);
  const int q0 = q_lo + qt * BM;
  if (q0 >= q_hi) return;
  const int klen = k_hi - k_lo;
  if (klen <= 0 && MERGE) return;

  const int lane = threadIdx.x;
  const int row = q0 + lane;
  const int row_rel = row - q_lo;
  const bool live = row < q_hi;
  const int qrel_last = min(q0 + BM, q_hi) - 1 - q_lo;
  const int kend = CAUSAL ? min(klen, qrel_last + 1) : klen;

  const float* qb = reinterpret_cast<const float*>(a.q);
  const float* kb = reinterpret_cast<const float*>(a.k) + (int64_t)kvh * DQK;
  const float* vb = reinterpret_cast<const float*>(a.v) + (int64_t)kvh * DV;

  float qr[DQK];
  {
    const float* qp = qb + (int64_t)min(row, q_hi - 1) * a.q_stride + (int64_t)h * DQK;
#pragma unroll
    for (int d = 0; d < DQK; ++d) qr[d] = qp[d];
  }
  float o[DV];
#pragma unroll
  for (int d = 0; d < DV; ++d) o[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt0 = 0; kt0 < kend; kt0 += BN) {
    __syncthreads();
    for (int idx = lane; idx < BN * DQK; idx += 64) {
      const int r = idx / DQK, d = idx % DQK;
      const int tok = k_lo + min(kt0 + r, klen - 1);
      ks[r][d] = kb[(int64_t)tok * a.k_stride + d];
    }
    for (int idx = lane; idx < BN * DV; idx += 64) {
      const int r = idx / DV, d = idx % DV;
      const int tok = k_lo + min(kt0 + r, klen - 1);
      vs[r][d] = vb[(int64_t)tok * a.v_stride + d];
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < DQK; ++d) acc = fmaf(qr[d], ks[j][d], acc);
      const int kr = kt0 + j;
      const bool ok = kr < kend && (!CAUSAL || kr <= row_rel);
      s[j] = ok ? acc * a.scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < DV; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BN; ++j) {
      const float p = expf(s[j] - m_use);
      l_run += p;
#pragma unroll
      for (int d = 0; d < DV; ++d) o[d] = fmaf(p, vs[j][d], o[d]);
    }
  }
  if (!live) return;

  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse = empty ? -INFINITY : m_run + logf(l_run);
  float* orow = a.out + ((int64_t)row * a.hq + h) * DV;
  float* lrow = a.lse + (int64_t)h * a.total_q + row;
  if (!MERGE) {
#pragma unroll
    for (int d = 0; d < DV; ++d) orow[d] = o[d] * inv;
    *lrow = lse;
  } else {
    const float la = *lrow;
    const float mm = fmaxf(la, lse);
    const bool both_empty = (mm == -INFINITY);
    const float ms = both_empty ? 0.f : mm;
    const float wa = expf(la - ms), wb = expf(lse - ms);
    const float tot = wa + wb;
    const float ca = both_empty ? 0.f : wa / tot;
    const float cb = both_empty ? 0.f : wb / tot * inv;
#pragma unroll
    for (int d = 0; d < DV; ++d) orow[d] = ca * orow[d] + cb * o[d];
    *lrow = both_empty ? -INFINITY : ms + logf(tot);
  }
}

template <int DQK, int DV>
hipError_t launch_t(const AttnArgs& a, bool causal, bool merge, hipStream_t st) {
  const long long nblk = (long long)a.n_seq * a.n_qtiles * a.hq;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)nblk), block(64);
  if (causal) {
    if (merge) hipLaunchKernelGGL((attn_fwd_f32_kernel<DQK, DV, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_fwd_f32_kernel<DQK, DV, true, false>), grid, block, 0, st, a);
  } else {
    if (merge) hipLaunchKernelGGL((attn_fwd_f32_kernel<DQK, DV, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_fwd_f32_kernel<DQK, DV, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnArgs& a, int dqk, int dv, bool causal, bool merge,
                               hipStream_t st) {
  if (dqk == 64 && dv == 64) return launch_t<64, 64>(a, causal, merge, st);
  if (dqk == 32 && dv == 32) return launch_t<32, 32>(a, causal, merge, st);
  if (dqk == 128 && dv == 128) return launch_t<128, 128>(a, causal, merge, st);
  if (dqk == 16 && dv == 16) return launch_t<16, 16>(a, causal, merge, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
