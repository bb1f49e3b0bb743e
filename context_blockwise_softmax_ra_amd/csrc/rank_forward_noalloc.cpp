// ra_rank_forward_noalloc: ra_rank_forward with its workspace taken from a
// fixed device array of this library instead of a caller buffer, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so the device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.  Nothing here
// allocates, frees or synchronises.

#include <hip/hip_runtime.h>

#include <mutex>

#include "ra_internal.h"

namespace {

constexpr size_t kScratchBytes = RA_NOALLOC_SCRATCH_BYTES;  // per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

// Device address of this device's copy of `scratch` (looked up on the first
// call on each device).
ra_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ra::set_error(RA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return ra::set_error(RA_ERR_UNSUPPORTED, "device %d beyond the %d this entry point serves", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return ra::set_error(RA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                           hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

ra_status ra_rank_forward_noalloc(const ra_rank_desc* d, void* stream) {
  if (!d) return ra::set_error(RA_ERR_INVALID_ARG, "descriptor is NULL");
  size_t need = 0;
  ra_status st = ra_rank_forward_workspace(d, &need);
  if (st != RA_OK) return st;
  if (need > kScratchBytes)
    return ra::set_error(RA_ERR_INVALID_ARG,
                         "share needs %zu bytes of workspace, more than the %zu bytes of the "
                         "library's fixed scratch; use ra_rank_forward with a caller workspace",
                         need, kScratchBytes);
  ra_rank_desc t = *d;
  t.workspace = nullptr;
  t.workspace_bytes = 0;
  if (need) {
    void* p = nullptr;
    if ((st = scratch_address(&p)) != RA_OK) return st;
    t.workspace = p;
    t.workspace_bytes = kScratchBytes;
  }
  return ra_rank_forward(&t, stream);
}

}  // extern "C"
