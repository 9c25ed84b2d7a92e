// Offline front end: float weight rows -> trits and fp16 scales in the
// coordinates the layer stores.
//
// 10100.com/article/156675786 ("Bonsai 2，把27B压进6个G"), section
// "它怎么做到的": the weight matrix is rotated by a Hadamard transform and
// then rounded to -1, 0, +1; allhereai.com/news/1346, method paragraph: one
// FP16 scale per 128 weights and a block Hadamard rotation.  The pages give
// no scale rule; this library takes the mean magnitude of a group's rotated
// weights (rounded to fp16 once) and sends each rotated weight to the
// nearest of -s, 0, +s, a tie at s/2 going to 0.
//
// The stored rows are W blockdiag(H_128/sqrt(128)): the product W x equals
// (W Hn)(Hn x) because Hn is symmetric and orthogonal, so each 128-block of
// a weight row gets the same transform as a block of activations.
//
// One 128-block per 16 lanes, 8 weights per lane from two 16-byte loads;
// the fp32 butterflies of the activation transform; the block's magnitude
// sum across the 16 lanes; one RNE rounding to the fp16 scale; each trit
// from comparing 2|w'| with that scale (exact in fp32).  A lane writes its
// eight trits as one 8-byte store.  4 bytes are read and 1 written per
// weight (plus 2 per block): bound by HBM.
#include "bgg_device.h"

using namespace bgg;

namespace {

__global__ void __launch_bounds__(256) k_rotate_ternarize(const float* __restrict__ w,
                                                          int8_t* __restrict__ t,
                                                          uint16_t* __restrict__ s,
                                                          int64_t slices /* N*K/8 */) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int l16 = threadIdx.x & 15;
  const bool valid = i < slices;  // whole 16-lane groups are valid or not
  float v[8];
  if (valid) {
    const float4 a = reinterpret_cast<const float4*>(w + i * 8)[0];
    const float4 b = reinterpret_cast<const float4*>(w + i * 8)[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
    v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  fwht128_unscaled(v, l16);
  float mag = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] *= kHadamardNorm;
    mag += fabsf(v[j]);
  }
  mag += xor16_f<1>(mag);
  mag += xor16_f<2>(mag);
  mag += xor16_f<4>(mag);
  mag += xor16_f<8>(mag);
  const uint16_t sh = f2h(mag * (1.0f / 128.0f));  // (the division by 128 is exact)
  const float sf = h2f(sh);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tj = 2.0f * fabsf(v[j]) > sf ? (v[j] > 0.0f ? 1 : -1) : 0;
    const uint32_t byte = (uint32_t)(uint8_t)(int8_t)tj;
    if (j < 4)
      lo |= byte << (8 * j);
    else
      hi |= byte << (8 * (j - 4));
  }
  if (!valid) return;
  *reinterpret_cast<uint2*>(t + i * 8) = make_uint2(lo, hi);
  if (l16 == 0) s[i / 16] = sh;
}

}  // namespace

extern "C" bgg_status bgg_rotate_ternarize(const void* w_dev, int64_t N, int64_t K,
                                           int8_t* trits_dev, uint16_t* scales_dev, void* stream) {
  if (!w_dev || !trits_dev || !scales_dev)
    return fail(BGG_ERR_NULL, "bgg_rotate_ternarize: NULL buffer");
  if (N < 0 || K < kGroup || K % kGroup || N > (int64_t(1) << 31) || K > (int64_t(1) << 28))
    return fail(BGG_ERR_SHAPE, "bgg_rotate_ternarize: need N >= 0 and K a positive multiple of 128");
  if (!aligned16(w_dev) || ((uintptr_t)trits_dev & 7) || ((uintptr_t)scales_dev & 1))
    return fail(BGG_ERR_BUFFER, "bgg_rotate_ternarize: w must be 16-byte, trits 8-byte and "
                                "scales 2-byte aligned");
  if (N == 0) return BGG_OK;
  if (N * K > (int64_t(1) << 40))
    return fail(BGG_ERR_SHAPE, "bgg_rotate_ternarize: more than 2^40 weights in one call");
  const int64_t slices = N * K / 8;
  hipLaunchKernelGGL(k_rotate_ternarize, dim3((unsigned)ceil_div(slices, 256)), dim3(256), 0,
                     (hipStream_t)stream, (const float*)w_dev, trits_dev, scales_dev, slices);
  return hip_check("bgg_rotate_ternarize");
}
