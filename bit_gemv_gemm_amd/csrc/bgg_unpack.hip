// Device unpack: packed device layout -> int8 weights [N][K] and fp16 scales
// [N][K/scale_group], through the same decoders the products use (PQ2_0 and
// Q2_0_g64 nibble spreading; PTQ1_0 through the one-token GEMV's LDS table,
// built by the same builder and read with the same addressing; Q1_0 bits).
// For checking; not on the hot path.
//
// Packings: allhereai.com/news/1346, packing paragraph (PQ2_0 one trit per
// 2-bit slot, PTQ1_0 compact); wmrh.cn/news/471187, section 关键机制 (five
// trits per byte).
#include "bgg_device.h"

using namespace bgg;

namespace {

template <int FMT>
__global__ void __launch_bounds__(256)
    k_unpack(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t NT, int64_t C,
             int64_t G, int64_t N, int64_t K, int8_t* __restrict__ trits,
             uint16_t* __restrict__ scales) {
  __shared__ uint32_t lut[FMT == BGG_FMT_PTQ1_0 ? 256 * kLutRowBytes / 4 : 1];
  __shared__ uint32_t lut_seed[FMT == BGG_FMT_PTQ1_0 ? 256 : 1];
  if (FMT == BGG_FMT_PTQ1_0) {
    build_lut32(lut, lut_seed);
    __syncthreads();
  }
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t l = idx % kTile, tc = idx / kTile;  // tc = tile * C + chunk
  const int64_t tile = tc / C, c = tc % C;
  const int64_t row = tile * kTile + l;
  if (tile < NT && row < N) {
    const uint4 ch = reinterpret_cast<const uint4*>(packed)[tc * kTile + l];
    const uint32_t cw[4] = {ch.x, ch.y, ch.z, ch.w};
    int8_t* out = trits + row * K;
    if (FMT == BGG_FMT_Q1_0) {
#pragma unroll
      for (int b = 0; b < 128; ++b) {
        const int64_t k = c * 128 + b;
        if (k < K) out[k] = (int8_t)(((cw[b >> 5] >> (b & 31)) & 1u) ? 1 : -1);
      }
    } else if (FMT == BGG_FMT_PQ2_0 || FMT == BGG_FMT_Q2_0_G64) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t E = pq2_even(cw[d]), O = pq2_odd(cw[d]);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int64_t k = c * 64 + 16 * d + 2 * n;
          const int te = (int)((E >> (4 * n)) & 15u), to = (int)((O >> (4 * n)) & 15u);
          if (k < K) out[k] = (int8_t)(te == 3 ? 0 : te - 1);
          if (k + 1 < K) out[k + 1] = (int8_t)(to == 3 ? 0 : to - 1);
        }
      }
    } else {
      const uint32_t lane_off = lut_lane_off((int)(threadIdx.x & 63));
      const char* lbase = reinterpret_cast<const char*>(lut);
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint32_t w = cw[b >> 2];
        const uint32_t addr = (b & 3) == 0 ? lut_addr<0>(w, lane_off)
                              : (b & 3) == 1 ? lut_addr<1>(w, lane_off)
                              : (b & 3) == 2 ? lut_addr<2>(w, lane_off)
                                             : lut_addr<3>(w, lane_off);
        const uint32_t e = *reinterpret_cast<const uint32_t*>(lbase + addr);  // five signed trit nibbles
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const int64_t k = (c * 16 + b) * 5 + i;
          if (k < K) out[k] = (int8_t)((int)(e << (28 - 4 * i)) >> 28);
        }
      }
    }
  }
  // scales: one thread per (row, group)
  const int64_t total_s = NT * G * kTile;
  const uint16_t* sdata = reinterpret_cast<const uint16_t*>(packed + scale_offset);
  for (int64_t i = idx; i < total_s; i += (int64_t)gridDim.x * 256) {
    const int64_t ll = i % kTile, tg = i / kTile;
    const int64_t t = tg / G, g = tg % G;
    const int64_t r = t * kTile + ll;
    if (r < N) scales[r * G + g] = sdata[i];
  }
}

}  // namespace

extern "C" bgg_status bgg_unpack_weights(const bgg_weights_desc* d, const void* packed_dev,
                                         int8_t* trits_dev, uint16_t* scales_dev, void* stream) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!packed_dev || !trits_dev || !scales_dev)
    return fail(BGG_ERR_NULL, "bgg_unpack_weights: NULL buffer");
  if (!aligned16(packed_dev)) return fail(BGG_ERR_BUFFER, "bgg_unpack_weights: packed misaligned");
  const int64_t threads = d->row_tiles * d->chunks * kTile;
  const dim3 grid((unsigned)ceil_div(threads, 256));
#define BGG_UNPACK(F)                                                                       \
  hipLaunchKernelGGL(k_unpack<F>, grid, dim3(256), 0, (hipStream_t)stream,                \
                     (const uint8_t*)packed_dev, d->scale_offset, d->row_tiles, d->chunks, \
                     d->scales, d->N, d->K, trits_dev, scales_dev)
  switch (d->format) {
    case BGG_FMT_PQ2_0: BGG_UNPACK(BGG_FMT_PQ2_0); break;
    case BGG_FMT_PTQ1_0: BGG_UNPACK(BGG_FMT_PTQ1_0); break;
    case BGG_FMT_Q1_0: BGG_UNPACK(BGG_FMT_Q1_0); break;
    default: BGG_UNPACK(BGG_FMT_Q2_0_G64); break;
  }
#undef BGG_UNPACK
  return hip_check("bgg_unpack_weights");
}
