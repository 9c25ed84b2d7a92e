// Measurement helpers for the benchmark, built as libbgg_probe.so beside
// the library (not part of the product interface): plain streaming kernels
// of known byte counts, for the achievable HBM read rate and for calibrating
// the profiler's FETCH_SIZE / WRITE_SIZE counters against bytes this
// project's own code moves.
//
//   bgg_probe_read   reads `bytes` (a multiple of 16) once with 16-byte
//                    non-temporal loads; writes one 32-bit word per
//                    workgroup to `sink` (at least bgg_probe_sink_words()
//                    words) so the loads are not optimised away.
//   bgg_probe_write  writes `bytes` (a multiple of 16) of zeros with
//                    16-byte stores.
//   bgg_probe_empty  launches a kernel of `grid` workgroups of `block`
//                    threads that does no work: the fixed cost of one launch
//                    (dispatch, the wait for the previous launch on the
//                    stream, completion) that every kernel pays.
// Both return 0, or the HIP error code of the launch; asynchronous on
// `stream`.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr unsigned kBlocks = 4096;  // 16 workgroups per CU on 256 CUs

__global__ void __launch_bounds__(kThreads) k_probe_read(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < kThreads; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

__global__ void __launch_bounds__(kThreads) k_probe_write(u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(z, dst + i);
}

// never stores (no thread index reaches kThreads * 1024); the pointer keeps
// the kernel from being an empty function body the runtime could skip
__global__ void k_probe_empty(uint32_t* sink) {
  if (threadIdx.x == kThreads * 1024u) sink[0] = 0u;
}

}  // namespace

extern "C" {

size_t bgg_probe_sink_words(void) { return kBlocks; }

int bgg_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_read, dim3(kBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (int64_t)(bytes / 16), (uint32_t*)sink);
  return (int)hipGetLastError();
}

int bgg_probe_write(void* dst, size_t bytes, void* stream) {
  if (!dst || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_write, dim3(kBlocks), dim3(kThreads), 0, (hipStream_t)stream, (u32x4*)dst,
                     (int64_t)(bytes / 16));
  return (int)hipGetLastError();
}

int bgg_probe_empty(unsigned grid, unsigned block, void* sink, void* stream) {
  if (!sink || grid == 0 || block == 0 || block > 1024) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_empty, dim3(grid), dim3(block), 0, (hipStream_t)stream, (uint32_t*)sink);
  return (int)hipGetLastError();
}

}  // extern "C"
