// Bandwidth-bound kernels of the rank share: the lse merge, the float32 ->
// bfloat16 finalisation, the zig-zag gather/scatter and the backward's
// row dot product delta = rowsum(dout * out).
//
// All of them stream [tokens, heads, dim] rows with 16-byte accesses; a
// group of consecutive lanes covers one (token, head) row, so every wave
// instruction touches whole, contiguous rows.

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ int pow2ceil_le64(int x) {
  int p = 1;
  while (p < x && p < 64) p <<= 1;
  return p;
}

// ---------------------------------------------------------------------------
// lse merge ("超长序列并行训练技术：Ulysses与Ring-Attention详解", section 4.2:
// lse_new = log(exp(lse_prev) + exp(lse_cur)); the output is re-weighted by
// exp(lse_side - lse_new), the exact correction of the oh-bug page's
// online softmax).  Each (token, head) row is handled by one lane group that
// reads both lse values before any lane writes the new one; a group never
// spans two waves, so the read-before-write order holds without barriers.
// ---------------------------------------------------------------------------
// Merge weights of one row: (ca, cb) and the new lse.
__device__ __forceinline__ void merge_weights(float la, float lb, float* ca, float* cb,
                                              float* lnew) {
  const float m = fmaxf(la, lb);
  const bool empty = (m == -INFINITY);
  const float ms = empty ? 0.f : m;
  const float wa = __expf(la - ms), wb = __expf(lb - ms);
  const float tot = wa + wb;
  *ca = empty ? 0.f : wa / tot;
  *cb = empty ? 0.f : wb / tot;
  *lnew = empty ? -INFINITY : ms + __logf(tot);
}

// Rows of dv = 4 LG floats (LG = 4 .. 32 lanes per row, one 16-byte chunk
// per lane): every wave takes kMergeRows row groups per pass and issues all
// their loads (both lse values, both partial rows) before any arithmetic,
// from clamped rows so that no load sits behind a branch; only the stores
// are guarded.
// (2 measured best, cache-cold on one box: 5.59 TB/s against 5.43 for one
// row group per pass, 5.12 for 4 and 4.69 for 8)
#ifndef RA_MERGE_ROWS_PER_PASS
#define RA_MERGE_ROWS_PER_PASS 2
#endif
constexpr int kMergeRows = RA_MERGE_ROWS_PER_PASS;

template <int LG>
__global__ __launch_bounds__(NT) void lse_merge_rows_kernel(float* __restrict__ out_acc,
                                                            float* __restrict__ lse_acc,
                                                            const float* __restrict__ out_part,
                                                            const float* __restrict__ lse_part,
                                                            int total_t, int h,
                                                            const int* __restrict__ cu,
                                                            int part) {
  constexpr int DV = 4 * LG, PER_WAVE = 64 / LG;
  const int seg = blockIdx.y;
  int lo, hi;
  part_range(cu[seg], cu[seg + 1], part, &lo, &hi);
  const int nrows = (hi - lo) * h;
  const int lane = threadIdx.x & 63;
  const int sub = lane / LG, li = lane % LG;
  const int wave_global = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int wstride = gridDim.x * (NT / 64);
  for (int base = wave_global * PER_WAVE * kMergeRows; base < nrows;
       base += wstride * PER_WAVE * kMergeRows) {
    bool ok[kMergeRows];
    int64_t row[kMergeRows], lrow[kMergeRows];
    float la[kMergeRows], lb[kMergeRows];
    float4 x[kMergeRows], y[kMergeRows];
#pragma unroll
    for (int u = 0; u < kMergeRows; ++u) {
      const int rh0 = base + u * PER_WAVE + sub;
      ok[u] = rh0 < nrows;
      const int rh = ok[u] ? rh0 : nrows - 1;
      const int t = lo + rh / h, hh = rh % h;
      row[u] = ((int64_t)t * h + hh) * DV;
      lrow[u] = (int64_t)hh * total_t + t;
      la[u] = lse_acc[lrow[u]];
      lb[u] = lse_part[lrow[u]];
      x[u] = reinterpret_cast<const float4*>(out_acc + row[u])[li];
      y[u] = reinterpret_cast<const float4*>(out_part + row[u])[li];
    }
#pragma unroll
    for (int u = 0; u < kMergeRows; ++u) {
      float ca, cb, lnew;
      merge_weights(la[u], lb[u], &ca, &cb, &lnew);
      float4 r;
      r.x = ca * x[u].x + cb * y[u].x;
      r.y = ca * x[u].y + cb * y[u].y;
      r.z = ca * x[u].z + cb * y[u].z;
      r.w = ca * x[u].w + cb * y[u].w;
      if (ok[u]) reinterpret_cast<float4*>(out_acc + row[u])[li] = r;
      // every lane of the wave read both lse values above
      if (ok[u] && li == 0) lse_acc[lrow[u]] = lnew;
    }
  }
}

// Any dv (a multiple of 4): a lane group of up to 64 lanes per row, looping
// over the row's 16-byte chunks.
__global__ __launch_bounds__(NT) void lse_merge_kernel(float* __restrict__ out_acc,
                                                       float* __restrict__ lse_acc,
                                                       const float* __restrict__ out_part,
                                                       const float* __restrict__ lse_part,
                                                       int total_t, int h, int dv,
                                                       const int* __restrict__ cu, int part) {
  const int seg = blockIdx.y;
  int lo, hi;
  part_range(cu[seg], cu[seg + 1], part, &lo, &hi);
  const int nrows = (hi - lo) * h;
  const int c4n = dv >> 2;
  const int lg = pow2ceil_le64(c4n);
  const int per_wave = 64 / lg;
  const int lane = threadIdx.x & 63;
  const int sub = lane / lg, li = lane % lg;
  const int wave_global = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int wstride = gridDim.x * (NT / 64);
  for (int base = wave_global * per_wave; base < nrows; base += wstride * per_wave) {
    const int rh = base + sub;
    const bool ok = rh < nrows;
    const int t = lo + (ok ? rh / h : 0);
    const int hh = ok ? rh % h : 0;
    float la = -INFINITY, lb = -INFINITY;
    if (ok) {
      la = lse_acc[(int64_t)hh * total_t + t];
      lb = lse_part[(int64_t)hh * total_t + t];
    }
    float ca, cb, lnew;
    merge_weights(la, lb, &ca, &cb, &lnew);
    if (ok) {
      float4* pa = reinterpret_cast<float4*>(out_acc + ((int64_t)t * h + hh) * dv);
      const float4* pb = reinterpret_cast<const float4*>(out_part + ((int64_t)t * h + hh) * dv);
      for (int c = li; c < c4n; c += lg) {
        const float4 xv = pa[c], yv = pb[c];
        float4 r;
        r.x = ca * xv.x + cb * yv.x;
        r.y = ca * xv.y + cb * yv.y;
        r.z = ca * xv.z + cb * yv.z;
        r.w = ca * xv.w + cb * yv.w;
        pa[c] = r;
      }
    }
    // every lane of the wave has read both lse values by now
    if (ok && li == 0) lse_acc[(int64_t)hh * total_t + t] = lnew;
  }
}

// ---------------------------------------------------------------------------
// float32 -> bfloat16, round to nearest even (NaN kept quiet)
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__global__ __launch_bounds__(NT) void cast_kernel(const float4* __restrict__ src,
                                                  ushort4* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NT) {
    const float4 x = src[i];
    ushort4 y;
    y.x = f32_to_bf16_rne(x.x);
    y.y = f32_to_bf16_rne(x.y);
    y.z = f32_to_bf16_rne(x.z);
    y.w = f32_to_bf16_rne(x.w);
    dst[i] = y;
  }
}

// ---------------------------------------------------------------------------
// zig-zag gather / scatter: local half 2d+j of segment d starts at global
// token src_start[2d+j] ("超长序列并行训练技术", section 4.2 placement).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void zigzag_copy_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst,
                                                         int64_t row16, const int* __restrict__ cu,
                                                         const int* __restrict__ start,
                                                         int gather) {
  const int seg = blockIdx.y;
  const int l0 = cu[seg], l1 = cu[seg + 1];
  const int c = (l1 - l0) >> 1;
  const int64_t n = (int64_t)(l1 - l0) * row16;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const int r = (int)(i / row16);
    const int64_t w = i % row16;
    const int half = r >= c ? 1 : 0;
    const int64_t g = (int64_t)start[2 * seg + half] + (r - half * c);
    const int64_t loc = (int64_t)(l0 + r);
    if (gather)
      dst[loc * row16 + w] = src[g * row16 + w];
    else
      dst[g * row16 + w] = src[loc * row16 + w];
  }
}

// Row copy by token index (other shard maps): gather dst[i] = src[tok[i]],
// scatter dst[tok[i]] = src[i]; 16-byte words, grid-stride.
__global__ __launch_bounds__(NT) void token_copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t row16,
                                                        const int* __restrict__ tok, int n,
                                                        int gather) {
  const int64_t total = (int64_t)n * row16;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += (int64_t)gridDim.x * NT) {
    const int r = (int)(i / row16);
    const int64_t w = i % row16;
    const int64_t g = tok[r];
    if (gather)
      dst[(int64_t)r * row16 + w] = src[g * row16 + w];
    else
      dst[g * row16 + w] = src[(int64_t)r * row16 + w];
  }
}

// ---------------------------------------------------------------------------
// delta[h, t] = sum_d dout[t, h, d] * out[t, h, d]
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ld_elem(const void* p, int dtype, int64_t i) {
  if (dtype == RA_FP32) return reinterpret_cast<const float*>(p)[i];
  const unsigned short b = reinterpret_cast<const unsigned short*>(p)[i];
  return __uint_as_float((unsigned)b << 16);
}

__global__ __launch_bounds__(NT) void bwd_delta_kernel(const void* __restrict__ out, int odt,
                                                       const void* __restrict__ dout, int ddt,
                                                       int total_t, int h, int dv,
                                                       float* __restrict__ delta) {
  // one (token, head) row per 16-lane group, 4 groups per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4, li = lane & 15;
  const int64_t nrows = (int64_t)total_t * h;
  const int64_t wave_global = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int64_t wstride = (int64_t)gridDim.x * (NT / 64);
  for (int64_t base = wave_global * 4; base < nrows; base += wstride * 4) {
    const int64_t rh = base + sub;
    float acc = 0.f;
    if (rh < nrows) {
      const int64_t off = rh * dv;
      for (int d = li; d < dv; d += 16) acc += ld_elem(out, odt, off + d) * ld_elem(dout, ddt, off + d);
    }
#pragma unroll
    for (int s = 8; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 16);
    if (rh < nrows && li == 0) {
      const int64_t t = rh / h, hh = rh % h;
      delta[hh * total_t + t] = acc;
    }
  }
}

// The same for bf16 out and dout with d_v a multiple of 8 and 16-byte aligned
// rows: each lane of a row's 16-lane group takes 8 consecutive elements per
// pass with one 16-byte load from each buffer (the form above issues one
// 2-byte load per element).
__device__ __forceinline__ float dot_bf16x8(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(x[i] << 16), __uint_as_float(y[i] << 16), acc);
    acc = fmaf(__uint_as_float(x[i] & 0xffff0000u), __uint_as_float(y[i] & 0xffff0000u), acc);
  }
  return acc;
}

__global__ __launch_bounds__(NT) void bwd_delta_bf16x8_kernel(const uint4* __restrict__ out,
                                                              const uint4* __restrict__ dout,
                                                              int total_t, int h, int dv8,
                                                              float* __restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4, li = lane & 15;
  const int64_t nrows = (int64_t)total_t * h;
  const int64_t wave_global = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int64_t wstride = (int64_t)gridDim.x * (NT / 64);
  for (int64_t base = wave_global * 4; base < nrows; base += wstride * 4) {
    const int64_t rh = base + sub;
    float acc = 0.f;
    if (rh < nrows) {
      const int64_t off = rh * dv8;
      for (int d = li; d < dv8; d += 16) acc += dot_bf16x8(out[off + d], dout[off + d]);
    }
#pragma unroll
    for (int s = 8; s >= 1; s >>= 1) acc += __shfl_xor(acc, s, 16);
    if (rh < nrows && li == 0) {
      const int64_t t = rh / h, hh = rh % h;
      delta[hh * total_t + t] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine of a KV-split rank share: the same lse weighting as the merge
// above, over `split` partials at once (weights exp(lse_p - max), summed in
// part order, so the result is deterministic).  One thread per 4 output
// dims of a (token, head) row; the thread of dims 0..3 writes the lse.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void split_combine_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse, int split,
    int64_t po, int64_t pl, void* __restrict__ out, int out_bf16, float* __restrict__ lse,
    int32_t total_t, int32_t h, int32_t dv4, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * NT) {
    const int64_t row = i / dv4;          // token * h + head
    const int c4 = (int)(i - row * dv4);
    const int64_t t = row / h;
    const int hh = (int)(row - t * h);
    const int64_t li = (int64_t)hh * total_t + t;
    float m = -INFINITY;
    for (int p = 0; p < split; ++p) m = fmaxf(m, part_lse[p * pl + li]);
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (m != -INFINITY) {
      for (int p = 0; p < split; ++p) {
        const float lp = part_lse[p * pl + li];
        if (lp == -INFINITY) continue;  // a part with no key of the row (its out may be unset)
        const float w = __expf(lp - m);
        const float4 o = reinterpret_cast<const float4*>(part_out + p * po)[i];
        acc.x += w * o.x;
        acc.y += w * o.y;
        acc.z += w * o.z;
        acc.w += w * o.w;
        den += w;
      }
      const float inv = 1.f / den;
      acc.x *= inv;
      acc.y *= inv;
      acc.z *= inv;
      acc.w *= inv;
    }
    if (out_bf16) {
      ushort4 b;
      b.x = f32_to_bf16_rne(acc.x);
      b.y = f32_to_bf16_rne(acc.y);
      b.z = f32_to_bf16_rne(acc.z);
      b.w = f32_to_bf16_rne(acc.w);
      reinterpret_cast<ushort4*>(out)[i] = b;
    } else {
      reinterpret_cast<float4*>(out)[i] = acc;
    }
    if (c4 == 0) lse[li] = m == -INFINITY ? -INFINITY : m + __logf(den);
  }
}

// The same for S parts (2, 4, 6 or 8) and rows of DV4 float4 (a power of
// two): each
// thread reads its row's S lse values once, and the row index comes from a
// shift and one 32-bit division (the generic kernel above divides in 64
// bits twice per float4).
template <int S, int DV4>
__global__ __launch_bounds__(NT) void split_combine_fixed_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse, int64_t po, int64_t pl,
    void* __restrict__ out, int out_bf16, float* __restrict__ lse, uint32_t total_t, uint32_t h,
    uint32_t n_rows) {
  const uint32_t i = blockIdx.x * NT + threadIdx.x;
  const uint32_t rh = i / DV4;  // token * h + head
  if (rh >= n_rows) return;
  const uint32_t c4 = i % DV4;
  const uint32_t t = rh / h;
  const uint32_t hh = rh - t * h;
  const int64_t li = (int64_t)hh * total_t + t;
  float lp[S];
  float m = -INFINITY;
#pragma unroll
  for (int p = 0; p < S; ++p) {
    lp[p] = part_lse[p * pl + li];
    m = fmaxf(m, lp[p]);
  }
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int p = 0; p < S; ++p) {
      if (lp[p] == -INFINITY) continue;  // a part with no key of the row (its out may be unset)
      const float w = __expf(lp[p] - m);
      const float4 o = reinterpret_cast<const float4*>(part_out + p * po)[i];
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
      den += w;
    }
    const float inv = 1.f / den;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
  }
  if (out_bf16) {
    ushort4 b;
    b.x = f32_to_bf16_rne(acc.x);
    b.y = f32_to_bf16_rne(acc.y);
    b.z = f32_to_bf16_rne(acc.z);
    b.w = f32_to_bf16_rne(acc.w);
    reinterpret_cast<ushort4*>(out)[i] = b;
  } else {
    reinterpret_cast<float4*>(out)[i] = acc;
  }
  if (c4 == 0) lse[li] = m == -INFINITY ? -INFINITY : m + __logf(den);
}

unsigned grid_for(int64_t work, int64_t per_block, unsigned cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_lse_merge(float* out_acc, float* lse_acc, const float* out_part,
                            const float* lse_part, int32_t total_t, int32_t h, int32_t dv,
                            int32_t n_seq, const int32_t* cu, int32_t part, int32_t max_rows,
                            hipStream_t st) {
  if (n_seq <= 0 || max_rows <= 0) return hipSuccess;
  const int64_t rows = (int64_t)max_rows * h;
  const int c4n = dv / 4;
  if (c4n == 4 || c4n == 8 || c4n == 16 || c4n == 32) {
    const int rows_per_block = (NT / c4n) * kMergeRows;
    dim3 grid(grid_for(rows, rows_per_block, 65535u), (unsigned)n_seq);
#define RA_MERGE_ROWS(LG)                                                                      \
  hipLaunchKernelGGL(lse_merge_rows_kernel<LG>, grid, dim3(NT), 0, st, out_acc, lse_acc, out_part, \
                     lse_part, total_t, h, cu, part)
    if (c4n == 4) RA_MERGE_ROWS(4);
    else if (c4n == 8) RA_MERGE_ROWS(8);
    else if (c4n == 16) RA_MERGE_ROWS(16);
    else RA_MERGE_ROWS(32);
#undef RA_MERGE_ROWS
    return hipGetLastError();
  }
  int lg = 1;
  while (lg < c4n && lg < 64) lg <<= 1;
  dim3 grid(grid_for(rows, NT / lg, 65535u), (unsigned)n_seq);
  hipLaunchKernelGGL(lse_merge_kernel, grid, dim3(NT), 0, st, out_acc, lse_acc, out_part,
                     lse_part, total_t, h, dv, cu, part);
  return hipGetLastError();
}

hipError_t launch_cast_f32_bf16(const float* src, void* dst, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_kernel, dim3(grid_for(n4, NT, 8192u)), dim3(NT), 0, st,
                     reinterpret_cast<const float4*>(src), reinterpret_cast<ushort4*>(dst), n4);
  return hipGetLastError();
}

hipError_t launch_split_combine(const float* part_out, const float* part_lse, int split,
                                int64_t part_out_stride, int64_t part_lse_stride, void* out,
                                ra_dtype out_dtype, float* lse, int32_t total_t, int32_t h,
                                int32_t dv, hipStream_t st) {
  const int64_t n = (int64_t)total_t * h * (dv / 4);
  if (n <= 0) return hipSuccess;
  if (split < 1 || (dv % 4) || part_out_stride < n * 4 || part_lse_stride < (int64_t)total_t * h)
    return hipErrorInvalidValue;
  const int bf = out_dtype == RA_BF16 ? 1 : 0;
  const int64_t rows = (int64_t)total_t * h;
  const unsigned blocks = (unsigned)((n + NT - 1) / NT);
#define RA_COMBINE_FIXED(S, DV4)                                                                \
  if (split == S && dv / 4 == DV4) {                                                           \
    hipLaunchKernelGGL((split_combine_fixed_kernel<S, DV4>), dim3(blocks), dim3(NT), 0, st,    \
                       part_out, part_lse, part_out_stride, part_lse_stride, out, bf, lse,     \
                       (uint32_t)total_t, (uint32_t)h, (uint32_t)rows);                        \
    return hipGetLastError();                                                                  \
  }
  if (n < ((int64_t)1 << 31)) {
    RA_COMBINE_FIXED(2, 32)
    RA_COMBINE_FIXED(4, 32)
    RA_COMBINE_FIXED(6, 32)
    RA_COMBINE_FIXED(8, 32)
    RA_COMBINE_FIXED(2, 16)
    RA_COMBINE_FIXED(4, 16)
    RA_COMBINE_FIXED(6, 16)
    RA_COMBINE_FIXED(8, 16)
  }
#undef RA_COMBINE_FIXED
  hipLaunchKernelGGL(split_combine_kernel, dim3(grid_for(n, NT, 8192u)), dim3(NT), 0, st,
                     part_out, part_lse, split, part_out_stride, part_lse_stride, out, bf, lse,
                     total_t, h, dv / 4, n);
  return hipGetLastError();
}

hipError_t launch_zigzag_copy(const void* src, void* dst, int64_t row_bytes, int32_t n_seq,
                              const int32_t* cu_local, const int32_t* src_start,
                              int32_t max_half, bool gather, hipStream_t st) {
  if (n_seq <= 0 || max_half <= 0) return hipSuccess;
  const int64_t row16 = row_bytes / 16;
  dim3 grid(grid_for((int64_t)2 * max_half * row16, NT, 4096u), (unsigned)n_seq);
  hipLaunchKernelGGL(zigzag_copy_kernel, grid, dim3(NT), 0, st,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), row16,
                     cu_local, src_start, gather ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_gather_tokens(const void* src, void* dst, int64_t row_bytes,
                                const int32_t* tokens, int32_t n, bool gather, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t row16 = row_bytes / 16;
  hipLaunchKernelGGL(token_copy_kernel, dim3(grid_for((int64_t)n * row16, NT, 8192u)), dim3(NT), 0,
                     st, reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), row16,
                     tokens, n, gather ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const void* out, int out_dtype, const void* dout, int dout_dtype,
                            int32_t total_t, int32_t hq, int32_t dv, float* delta,
                            hipStream_t st) {
  const int64_t rows = (int64_t)total_t * hq;
  if (rows <= 0) return hipSuccess;
  if (out_dtype == RA_BF16 && dout_dtype == RA_BF16 && dv % 8 == 0 &&
      reinterpret_cast<uintptr_t>(out) % 16 == 0 && reinterpret_cast<uintptr_t>(dout) % 16 == 0) {
    hipLaunchKernelGGL(bwd_delta_bf16x8_kernel, dim3(grid_for(rows, 16, 16384u)), dim3(NT), 0, st,
                       static_cast<const uint4*>(out), static_cast<const uint4*>(dout), total_t,
                       hq, dv / 8, delta);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(bwd_delta_kernel, dim3(grid_for(rows, 16, 16384u)), dim3(NT), 0, st, out,
                     out_dtype, dout, dout_dtype, total_t, hq, dv, delta);
  return hipGetLastError();
}

}  // namespace ra
