// Sustained rate of the matrix cores on the forward's product
// (v_mfma_f32_32x32x16_bf16) with operands drawn like the attention inputs:
// a measurement kernel, not part of the attention path.  It bounds what the
// attention kernels can reach on this data, since operand bit activity
// changes the clock the chip sustains.
//
// Each wave keeps 8 independent accumulator chains and cycles through 8 A
// and 8 B operand fragments read once from `operands` (bf16, per wave a
// distinct 8 KiB slice), so consecutive products see different random bits
// as in the attention products.  Two waves per SIMD, as in the ping-pong
// attention kernel.  The accumulators are summed and written to `out` (one
// float per wave) so that no product can be dropped.

#include "mfma_common.h"

namespace ra {
namespace {

using namespace mfma;

constexpr int kCeilWaves = 4;  // waves per workgroup; two workgroups per CU

__global__ __launch_bounds__(kCeilWaves * 64, 2) void mfma_ceiling_kernel(const u32x4* operands,
                                                                        int64_t n_frag,
                                                                        float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kCeilWaves + (threadIdx.x >> 6);
  // 16 fragments of 16 bytes per lane, from the wave's slice (wrapped)
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = as_bf16x8(operands[((wave * 16 + j) * 64 + lane) % n_frag]);
    b[j] = as_bf16x8(operands[((wave * 16 + 8 + j) * 64 + lane) % n_frag]);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = mma(a[j], b[(j + r) & 7], acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[wave * 64 + lane] = s;
}

}  // namespace
}  // namespace ra

extern "C" ra_status ra_mfma_ceiling(const void* operands, int64_t operand_bytes, float* out,
                                     int64_t out_floats, int32_t n_workgroups, int32_t iters,
                                     void* stream) {
  if (!operands || !out) return ra::set_error(RA_ERR_INVALID_ARG, "NULL buffer");
  if (n_workgroups <= 0 || iters <= 0 || operand_bytes < 16 * 64 * 16 || (operand_bytes % 16) ||
      (reinterpret_cast<uintptr_t>(operands) & 15))
    return ra::set_error(RA_ERR_INVALID_ARG, "bad sizes or alignment");
  if (out_floats < (int64_t)n_workgroups * ra::kCeilWaves * 64)
    return ra::set_error(RA_ERR_INVALID_ARG, "out holds %lld floats, %lld needed",
                         (long long)out_floats, (long long)n_workgroups * ra::kCeilWaves * 64);
  hipLaunchKernelGGL(ra::mfma_ceiling_kernel, dim3(n_workgroups), dim3(ra::kCeilWaves * 64), 0,
                     (hipStream_t)stream, static_cast<const ra::mfma::u32x4*>(operands),
                     (int64_t)(operand_bytes / 16), out, iters);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return ra::set_error(RA_ERR_HIP, "mfma ceiling launch: %s", hipGetErrorString(e));
  return RA_OK;
}
