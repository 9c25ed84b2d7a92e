// The activation transform x' = blockdiag(H_128 / sqrt(128)) x on fp16 rows.
//
// allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), runtime paragraph: the
// runtime must apply the Hadamard transform to the activations;
// 10100.com/article/156675786, section "它怎么做到的": the input gets the
// transform that matches the rotated weights, or the output is silently
// wrong.
//
// One 128-block per 16 lanes, 8 values per lane from one 16-byte load:
// strides 1..4 inside the lane, 8..64 across lanes; fp32 butterflies, one
// RNE rounding to fp16 at the end.  Read and write are each one coalesced
// 16-byte access per lane, so the kernel is bound by HBM.
#include "bgg_device.h"

using namespace bgg;

namespace {

__global__ void __launch_bounds__(256) k_hadamard_rotate(const uint16_t* x, uint16_t* y,
                                                          int64_t slices /* M*K/8 */) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = i < slices;  // whole 16-lane groups are valid or not
  float v[8];
  if (valid) {
    load8h(x + i * 8, v);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  fwht128_unscaled(v, threadIdx.x & 15);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (uint32_t)f2h(v[2 * j] * kHadamardNorm) |
           ((uint32_t)f2h(v[2 * j + 1] * kHadamardNorm) << 16);
  if (valid) *reinterpret_cast<uint4*>(y + i * 8) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

extern "C" bgg_status bgg_hadamard_rotate(const void* x_dev, void* xr_dev, int64_t M, int64_t K,
                                          void* stream) {
  if (!x_dev || !xr_dev) return fail(BGG_ERR_NULL, "bgg_hadamard_rotate: NULL buffer");
  if (M < 0 || K < kGroup || K % kGroup)
    return fail(BGG_ERR_SHAPE, "bgg_hadamard_rotate: need M >= 0 and K a positive multiple of 128");
  if (!aligned16(x_dev) || !aligned16(xr_dev))
    return fail(BGG_ERR_BUFFER, "bgg_hadamard_rotate: buffers must be 16-byte aligned");
  if (M == 0) return BGG_OK;
  const int64_t slices = M * K / 8;
  hipLaunchKernelGGL(k_hadamard_rotate, dim3((unsigned)ceil_div(slices, 256)), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)x_dev, (uint16_t*)xr_dev, slices);
  return hip_check("bgg_hadamard_rotate");
}
