// bgg_ternary_gemv_noalloc: the decode-time product of bgg_ternary_gemv for
// callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  Its workspace is
// one file-scope device array per GPU instead of a caller's buffer; the
// kernels, their arithmetic and their results are those of
// bgg_ternary_gemv.
//
// The array holds what a caller's workspace holds: the 64-bit row words of
// split-K launches (which must be zero when a call starts; every GEMV call
// leaves them zero) and scratch (encoded activations).  The code-object
// loader zero-fills the array; the first call on a device clears it once
// more with a fill kernel, stream-ordered before that call's own kernels.
// After that no call clears anything: each one finds the row words zero
// because the one before it left them so.  Calls on one GPU share the array,
// so calls that overlap in time on one GPU race.
#include "bgg_device.h"
#include "bgg_internal.h"

#include <mutex>

using namespace bgg;

namespace {

// Largest workspace the array serves: 32 MiB covers every format at every
// token count for K up to 262144 (the row words alone take 16 MiB).
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;        // device address of `scratch` on this GPU
  hipError_t err = hipSuccess;
  bool cleared = false;       // the first call's clear has been enqueued
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_clear_mu;

__global__ void __launch_bounds__(256) k_zero16(uint4* p, int64_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// This device's copy of `scratch` (its address taken once, with the device
// current); on the first call the array is cleared on `stream`.
bgg_status device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BGG_ERR_HIP, "bgg_ternary_gemv_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BGG_ERR_HIP, "bgg_ternary_gemv_noalloc: device %d beyond the %d served", dev, kMaxDevices);
  DeviceScratch& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess || !s.ptr)
    return fail(BGG_ERR_HIP, "bgg_ternary_gemv_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(s.err));
  {
    std::lock_guard<std::mutex> lock(g_clear_mu);
    if (!s.cleared) {
      hipLaunchKernelGGL(k_zero16, dim3(1024), dim3(256), 0, stream, (uint4*)s.ptr,
                         (int64_t)(kScratchBytes / sizeof(uint4)));
      bgg_status st = hip_check("bgg_ternary_gemv_noalloc");
      if (st) return st;
      s.cleared = true;
    }
  }
  *out = s.ptr;
  return BGG_OK;
}

}  // namespace

extern "C" bgg_status bgg_ternary_gemv_noalloc(const bgg_weights_desc* d, const void* packed_dev,
                                               const void* x_dev, void* y_dev, int64_t M, uint32_t flags,
                                               void* stream) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (M < 1 || M > BGG_MAX_GEMV_M)
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv_noalloc: M must be in 1..%d (got %lld)", BGG_MAX_GEMV_M,
                (long long)M);
  const size_t need = bgg_gemv_workspace_size(d, M);
  if (need == 0) return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv_noalloc: K = %lld is too long", (long long)d->K);
  if (need > kScratchBytes)
    return fail(BGG_ERR_SHAPE,
                "bgg_ternary_gemv_noalloc: N = %lld, K = %lld, M = %lld need %zu workspace bytes, "
                "more than the %zu of the static workspace",
                (long long)d->N, (long long)d->K, (long long)M, need, kScratchBytes);
  if (!packed_dev || !x_dev || !y_dev) return fail(BGG_ERR_NULL, "bgg_ternary_gemv_noalloc: NULL buffer");
  void* ws = nullptr;
  if ((st = device_scratch((hipStream_t)stream, &ws))) return st;
  return bgg_ternary_gemv(d, packed_dev, x_dev, y_dev, M, flags, ws, kScratchBytes, stream);
}
