// Device half of libbgg for gfx950 (CDNA4): the Hadamard transform of the
// activations, the decode-time GEMV for both packings, and the device unpack.
//
// What is computed follows allhereai.com/news/1346 ("27B 模型压到 5.95GB…":
// method paragraph -- trits with one FP16 scale per 128 weights in
// block-Hadamard-rotated coordinates; runtime paragraph -- the activations
// get the Hadamard transform at run time; packing paragraph -- PQ2_0 and
// PTQ1_0) and 10100.com/article/156675786 (section "它怎么做到的": the input
// gets the transform that matches the rotated weights).
//
// GEMV design (one MI355X has 256 CUs in 8 XCDs, 64-lane waves, HBM3E):
//   * one lane per weight row: a 64-row tile is read as 1 KiB coalesced
//     16-byte loads, chunk by chunk along K, so every lane works on the same
//     K positions and the activation operands are wave-uniform (scalar
//     registers, no LDS traffic for x);
//   * K is split into slices so that ~1500 single-wave work items cover the
//     chip; the last wave to finish a tile adds the slices' partial sums in
//     a fixed order (deterministic) and writes fp16 y;
//   * trits are never turned into floats: the rotated activations are cut
//     into four signed 4-bit digits of a 15-bit block-fixed-point integer,
//     the 2-bit codes c = t + 1 are spread into 4-bit lanes with one mask,
//     and v_dot8_i32_i4 multiplies 8 codes by 8 digits per instruction.  The
//     exact integer sum of c*q over a group, minus the group's sum of q,
//     is the group's sum of t*q; it is scaled by s * 2^(e-14) and added in fp32.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "bgg_internal.h"

using bgg::fail;

namespace {

constexpr int kGroup = BGG_GROUP;   // 128
constexpr int kTile = BGG_ROW_TILE;  // 64
constexpr int kWaves = 8;            // XCDs: consecutive workgroups go round-robin over them

// PTQ1_0 period: 5 groups = 640 trits = 128 row bytes = 8 chunks.
constexpr int kPeriodGroups = 5;
constexpr int kPeriodBytes = 128;
constexpr int kPeriodChunks = 8;
// Activation operands of one PTQ1_0 period: 4 digit words per byte, plus 4
// words for the upper part of each of the 4 bytes that straddle a group end.
constexpr int kPtqFragWords = kPeriodBytes * 4 + 4 * 4;  // 528
// Activation operands of one PQ2_0 chunk (64 trits): 4 code words x {even,
// odd} positions x 4 digits.
constexpr int kPqFragWords = 32;

constexpr int kPrepGroups = 20;  // groups per x-prep workgroup (4 PTQ1_0 periods)
constexpr int kPrepThreads = kPrepGroups * 16;

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of data that is read once (packed weights): non-temporal.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// Normalised fast Walsh-Hadamard transform of one 128-block held by 16 lanes,
// 8 consecutive values each (lane i of the 16 holds positions 8i..8i+7).
// Butterflies (a, b) -> (a + b, a - b) over strides 1..64 in fp32; Sylvester
// order.  The 1/sqrt(128) is applied by the caller.
__device__ __forceinline__ void fwht128_unscaled(float v[8], int lane16) {
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & s)) {
        float a = v[i], b = v[i + s];
        v[i] = a + b;
        v[i + s] = a - b;
      }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const float sgn = (lane16 & m) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float p = __shfl_xor(v[i], m, 16);
      v[i] = fmaf(sgn, v[i], p);  // low lane: v + p; high lane: p - v
    }
  }
}

__device__ __forceinline__ void load8h(const uint16_t* p, float v[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = h2f((uint16_t)(w[i] & 0xFFFF));
    v[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
}

// Signed 4-bit digit L of q (|q| <= 2^14): q = d0 + 16 d1 + 256 d2 + 4096 d3,
// every d in [-8, 7] (d3 in [-4, 4]).
__device__ __forceinline__ int digit4(int q, int L) {
  int d = 0;
#pragma unroll
  for (int i = 0; i <= 3; ++i) {
    d = (int)((unsigned)q << 28) >> 28;  // sign-extended low nibble
    if (i == L) break;
    q = (q - d) >> 4;
  }
  return L == 3 ? q : d;
}

// PQ2_0: 16 codes of one word -> codes of even positions in the low two
// bits of each nibble (E) and of odd positions likewise (O).
__device__ __forceinline__ uint32_t pq2_even(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t pq2_odd(uint32_t w) { return (w >> 2) & 0x33333333u; }

// PTQ1_0: the five base-3 digits of a byte (= t + 1 of five trits), one per
// nibble 0..4.  Bytes 243..255 are not produced by any trits; they decode as
// five zero trits (digits 1).
__device__ __forceinline__ uint32_t ptq1_entry(uint32_t b) {
  if (b >= 243) return 0x11111u;
  uint32_t e = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    e |= (b % 3u) << (4 * i);
    b /= 3u;
  }
  return e;
}

// The LUT: 256 entries, each stored 32 times so that lane l reads copy l%32
// and a wave's 64 random lookups hit 32 distinct banks (32 KiB of LDS).
constexpr int kLutCopies = 32;
__device__ __forceinline__ void build_lut(uint32_t* lut) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    const uint32_t e = ptq1_entry((uint32_t)b);
    uint4 v = make_uint4(e, e, e, e);
    uint4* dst = reinterpret_cast<uint4*>(lut + b * kLutCopies);
#pragma unroll
    for (int c = 0; c < kLutCopies / 4; ++c) dst[c] = v;
  }
}

// ---------------------------------------------------------------------------
// hadamard_rotate: fp16 [M][K] -> fp16 [M][K]
// ---------------------------------------------------------------------------
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
  const float norm = 0.08838834764831845f;  // 1/sqrt(128), rounded to fp32
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (uint32_t)f2h(v[2 * j] * norm) | ((uint32_t)f2h(v[2 * j + 1] * norm) << 16);
  if (valid) *reinterpret_cast<uint4*>(y + i * 8) = make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------------------
// GEMV activation prep: x (fp16) -> x' (fp32, rotated unless told not to)
// -> per group: e = exponent with max|x'| < 2^e, q = rint(x' * 2^(14-e)),
// F = 2^(e-14), Q = sum q -> digit words laid out for the GEMV.  Also zeroes
// the per-tile arrival counters of the GEMV that follows on the stream.
// grid: (ceil(Gpad / 20), Mb); block: 320 threads = 20 groups x 16 lanes.
// Tokens Mreal..Mb-1 (padding up to a built token count) get zeros.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(kPrepThreads)
    k_gemv_prep(const uint16_t* __restrict__ x, int64_t K, int Mreal, int rotate,
                uint32_t* __restrict__ frag,
                int64_t frag_words_per_token, int32_t* __restrict__ metaQ, float* __restrict__ metaF,
                int64_t gpad, uint32_t* __restrict__ counters, int64_t n_counters) {
  __shared__ int16_t sq[kPrepGroups * kGroup];
  const int tid = threadIdx.x;
  const int m = blockIdx.y;
  const int64_t G = K / kGroup;
  const int64_t g0 = (int64_t)blockIdx.x * kPrepGroups;
  const int gl = tid >> 4, lane16 = tid & 15;
  const int64_t g = g0 + gl;
  const bool valid = g < G && m < Mreal;  // tokens past Mreal are zero padding

  if (blockIdx.x == 0 && m == 0)
    for (int64_t i = tid; i < n_counters; i += kPrepThreads) counters[i] = 0u;

  float v[8];
  if (valid) {
    load8h(x + (int64_t)m * K + g * kGroup + lane16 * 8, v);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  if (rotate) {
    fwht128_unscaled(v, lane16);
    const float norm = 0.08838834764831845f;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= norm;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 16));
  int e = 0;
  frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1): |x'| < 2^e
  int qsum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = amax > 0.0f ? (int)rintf(ldexpf(v[j], 14 - e)) : 0;
    sq[gl * kGroup + lane16 * 8 + j] = (int16_t)q;
    qsum += q;
  }
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) qsum += __shfl_xor(qsum, s, 16);
  if (lane16 == 0 && g < gpad) {
    metaQ[(int64_t)m * gpad + g] = qsum;
    metaF[(int64_t)m * gpad + g] = amax > 0.0f ? ldexpf(1.0f, e - 14) : 0.0f;
  }
  __syncthreads();

  uint32_t* out = frag + (int64_t)m * frag_words_per_token;
  if (FMT == BGG_FMT_PQ2_0) {
    // 40 chunks x 32 words; word (d, par, L) of chunk c: nibble n = digit L
    // of q at chunk position 16 d + 2 n + par.
    const int64_t C = K / 64;
    for (int w = tid; w < 2 * kPrepGroups * kPqFragWords; w += kPrepThreads) {
      const int cl = w / kPqFragWords, r = w % kPqFragWords;
      const int d = r >> 3, par = (r >> 2) & 1, L = r & 3;
      const int64_t c = g0 * 2 + cl;
      if (c >= C) continue;
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n)
        word |= (uint32_t)(digit4(sq[cl * 64 + 16 * d + 2 * n + par], L) & 15) << (4 * n);
      out[c * kPqFragWords + r] = word;
    }
  } else {
    // 4 periods x 528 words.  Word (byte jb, L), jb < 128: nibble i = digit L
    // of q at period position 5 jb + i, kept only if that position is in the
    // same group as 5 jb.  Word 512 + 4 s + L: the upper part of the s-th
    // straddling byte (positions in the next group).
    const int64_t P = (G + kPeriodGroups - 1) / kPeriodGroups;
    const int64_t p0 = g0 / kPeriodGroups;
    for (int w = tid; w < (kPrepGroups / kPeriodGroups) * kPtqFragWords; w += kPrepThreads) {
      const int pl = w / kPtqFragWords, r = w % kPtqFragWords;
      const int64_t p = p0 + pl;
      if (p >= P) continue;
      int jb, L, upper;
      if (r < kPeriodBytes * 4) {
        jb = r >> 2, L = r & 3, upper = 0;
      } else {
        const int s = (r - kPeriodBytes * 4) >> 2;
        L = r & 3, upper = 1;
        // the bytes whose five trits cross a group end: 25, 51, 76, 102
        jb = (kGroup * (s + 1)) / 5;
      }
      const int first_group = (5 * jb) / kGroup;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int pos = 5 * jb + i;
        if (pos / kGroup == first_group + upper)
          word |= (uint32_t)(digit4(sq[pl * 640 + pos], L) & 15) << (4 * i);
      }
      out[p * kPtqFragWords + r] = word;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K finish: every (tile, slice) wave stores its 64 x M partial sums;
// the last wave of a tile to arrive adds all slices in slice order.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ void finish_tile(const float (&acc)[M], int64_t tile, int slice, int S,
                                            int64_t rows_pad, int64_t N, int Mreal,
                                            float* __restrict__ partial,
                                            uint32_t* __restrict__ counters,
                                            uint16_t* __restrict__ y, int lane) {
  const int64_t row = tile * kTile + lane;
  if (S == 1) {
    if (row < N)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (m < Mreal) y[m * N + row] = f2h(acc[m]);
    return;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) partial[((int64_t)m * S + slice) * rows_pad + row] = acc[m];
  uint32_t prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  if (prev != (uint32_t)(S - 1)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  float sum[M];
#pragma unroll
  for (int m = 0; m < M; ++m) sum[m] = 0.0f;
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int m = 0; m < M; ++m)
      sum[m] += s == slice ? acc[m]
                           : __builtin_nontemporal_load(&partial[((int64_t)m * S + s) * rows_pad + row]);
  if (row < N)
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (m < Mreal) y[m * N + row] = f2h(sum[m]);
  if (lane == 0) counters[tile] = 0u;
}

// Work item of a GEMV wave: (tile, slice), with all slices of a tile on the
// same XCD (workgroup b runs on XCD b % 8).
__device__ __forceinline__ bool work_item(int64_t item_in_xcd, int xcd, int S, int64_t NT,
                                          int64_t& tile, int& slice) {
  slice = (int)(item_in_xcd % S);
  tile = (item_in_xcd / S) * kWaves + xcd;
  return tile < NT;
}

// ---------------------------------------------------------------------------
// PQ2_0 GEMV: one wave = 64 rows x BPS groups, M tokens.
// grid: 8 * ceil(NT/8) * S single-wave workgroups.
// ---------------------------------------------------------------------------
template <int M, int BPS>
__global__ void __launch_bounds__(64)
    k_gemv_pq2(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t NT, int64_t C,
               int64_t G, int64_t N, int S, int Mreal, const uint32_t* __restrict__ frag,
               const int32_t* __restrict__ metaQ, const float* __restrict__ metaF,
               float* __restrict__ partial, uint32_t* __restrict__ counters,
               uint16_t* __restrict__ y) {
  const int lane = threadIdx.x;
  int64_t tile;
  int slice;
  if (!work_item(blockIdx.x / kWaves, blockIdx.x % kWaves, S, NT, tile, slice)) return;
  const int64_t gbeg = (int64_t)slice * BPS;
  const uint4* tdata = reinterpret_cast<const uint4*>(packed) + (tile * C) * kTile + lane;
  const uint16_t* sdata =
      reinterpret_cast<const uint16_t*>(packed + scale_offset) + (tile * G) * kTile + lane;

  uint4 w[2 * BPS];
  uint16_t sc[BPS];
#pragma unroll
  for (int i = 0; i < BPS; ++i) {
    const int64_t g = gbeg + i;
    if (g < G) {
      w[2 * i] = ld_stream(tdata + (2 * g) * kTile);
      w[2 * i + 1] = ld_stream(tdata + (2 * g + 1) * kTile);
      sc[i] = sdata[g * kTile];
    }
  }

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

#pragma unroll
  for (int i = 0; i < BPS; ++i) {
    const int64_t g = gbeg + i;
    if (g >= G) break;
    const float s = h2f(sc[i]);
    uint32_t E[8], O[8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t cw[4] = {w[2 * i + c].x, w[2 * i + c].y, w[2 * i + c].z, w[2 * i + c].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        E[c * 4 + d] = pq2_even(cw[d]);
        O[c * 4 + d] = pq2_odd(cw[d]);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t* xf = frag + ((int64_t)m * C + 2 * g) * kPqFragWords;
      int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t* f = xf + c * kPqFragWords + d * 8;
          const int e = (int)E[c * 4 + d], o = (int)O[c * 4 + d];
          a0 = __builtin_amdgcn_sdot8(e, (int)f[0], a0, false);
          a1 = __builtin_amdgcn_sdot8(e, (int)f[1], a1, false);
          a2 = __builtin_amdgcn_sdot8(e, (int)f[2], a2, false);
          a3 = __builtin_amdgcn_sdot8(e, (int)f[3], a3, false);
          a0 = __builtin_amdgcn_sdot8(o, (int)f[4], a0, false);
          a1 = __builtin_amdgcn_sdot8(o, (int)f[5], a1, false);
          a2 = __builtin_amdgcn_sdot8(o, (int)f[6], a2, false);
          a3 = __builtin_amdgcn_sdot8(o, (int)f[7], a3, false);
        }
      const int p = a0 + (a1 << 4) + (a2 << 8) + (a3 << 12) - metaQ[(int64_t)m * G + g];
      acc[m] = fmaf(s * metaF[(int64_t)m * G + g], (float)p, acc[m]);
    }
  }
  finish_tile<M>(acc, tile, slice, S, NT * kTile, N, Mreal, partial, counters, y, lane);
}

// ---------------------------------------------------------------------------
// PTQ1_0 GEMV: one wave = 64 rows x PPS periods (5 groups each), M tokens.
// 4 independent waves per workgroup share the LUT.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ void ptq1_close(int (&a)[M][4], float (&acc)[M], int64_t gb, int64_t G,
                                           int64_t gpad, float s, const int32_t* __restrict__ metaQ,
                                           const float* __restrict__ metaF) {
  if (gb < G) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int p = a[m][0] + (a[m][1] << 4) + (a[m][2] << 8) + (a[m][3] << 12) -
                    metaQ[(int64_t)m * gpad + gb];
      acc[m] = fmaf(s * metaF[(int64_t)m * gpad + gb], (float)p, acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int L = 0; L < 4; ++L) a[m][L] = 0;
}

template <int M, int PPS>
__global__ void __launch_bounds__(256)
    k_gemv_ptq1(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t NT, int64_t C,
                int64_t G, int64_t N, int S, int Mreal, int64_t items_per_xcd,
                const uint32_t* __restrict__ frag, int64_t frag_words_per_token,
                const int32_t* __restrict__ metaQ, const float* __restrict__ metaF, int64_t gpad,
                float* __restrict__ partial, uint32_t* __restrict__ counters,
                uint16_t* __restrict__ y) {
  __shared__ uint32_t lut[256 * kLutCopies];
  build_lut(lut);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  // wave index within the workgroup, made provably wave-uniform so that all
  // addressing below lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = (int64_t)(blockIdx.x / kWaves) * 4 + wave;
  int64_t tile;
  int slice;
  if (item >= items_per_xcd) return;
  if (!work_item(item, blockIdx.x % kWaves, S, NT, tile, slice)) return;
  const uint32_t* lrow = lut + (lane & (kLutCopies - 1));
  const uint4* tdata = reinterpret_cast<const uint4*>(packed) + (tile * C) * kTile + lane;
  const uint16_t* sdata =
      reinterpret_cast<const uint16_t*>(packed + scale_offset) + (tile * G) * kTile + lane;

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  int a[M][4];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int L = 0; L < 4; ++L) a[m][L] = 0;

  for (int pp = 0; pp < PPS; ++pp) {
    const int64_t p = (int64_t)slice * PPS + pp;
    const int64_t gp = p * kPeriodGroups;
    if (gp >= G) break;
    uint4 w[kPeriodChunks];
#pragma unroll
    for (int c = 0; c < kPeriodChunks; ++c) {
      const int64_t j = p * kPeriodChunks + c;
      w[c] = j < C ? ld_stream(tdata + j * kTile) : make_uint4(0, 0, 0, 0);
    }
    float sc[kPeriodGroups];
#pragma unroll
    for (int k = 0; k < kPeriodGroups; ++k) sc[k] = gp + k < G ? h2f(sdata[(gp + k) * kTile]) : 0.0f;

    const uint32_t* fp = frag + p * kPtqFragWords;
    // fully unrolled: byte positions, group ends and straddles are constants
#pragma clang loop unroll(full)
    for (int jb = 0; jb < kPeriodBytes; ++jb) {
      const uint4 ch = w[jb >> 4];
      const uint32_t word = ((jb >> 2) & 3) == 0 ? ch.x : ((jb >> 2) & 3) == 1 ? ch.y
                            : ((jb >> 2) & 3) == 2 ? ch.z : ch.w;
      const uint32_t byte = (word >> (8 * (jb & 3))) & 0xFFu;
      const int codes = (int)lrow[byte * kLutCopies];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t* f = fp + m * frag_words_per_token + jb * 4;
#pragma unroll
        for (int L = 0; L < 4; ++L) a[m][L] = __builtin_amdgcn_sdot8(codes, (int)f[L], a[m][L], false);
      }
      const int k_first = (5 * jb) / kGroup, k_last = (5 * jb + 4) / kGroup;
      if (k_last != k_first) {
        // this byte's trits cross a group end: close the lower group and
        // start the next one with the byte's upper trits
        ptq1_close<M>(a, acc, gp + k_first, G, gpad, sc[k_first], metaQ, metaF);
        const int s = k_first;  // straddle index 0..3
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint32_t* f = fp + m * frag_words_per_token + kPeriodBytes * 4 + s * 4;
#pragma unroll
          for (int L = 0; L < 4; ++L) a[m][L] = __builtin_amdgcn_sdot8(codes, (int)f[L], a[m][L], false);
        }
      } else if ((5 * jb + 5) % kGroup == 0) {
        ptq1_close<M>(a, acc, gp + k_first, G, gpad, sc[k_first], metaQ, metaF);
      }
    }
  }
  finish_tile<M>(acc, tile, slice, S, NT * kTile, N, Mreal, partial, counters, y, lane);
}

// ---------------------------------------------------------------------------
// unpack: device layout -> int8 trits [N][K] and fp16 scales [N][G]
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(256)
    k_unpack(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t NT, int64_t C,
             int64_t G, int64_t N, int64_t K, int8_t* __restrict__ trits,
             uint16_t* __restrict__ scales) {
  __shared__ uint32_t lut[FMT == BGG_FMT_PTQ1_0 ? 256 * kLutCopies : 1];
  if (FMT == BGG_FMT_PTQ1_0) {
    build_lut(lut);
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
    if (FMT == BGG_FMT_PQ2_0) {
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
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint32_t e = lut[((cw[b >> 2] >> (8 * (b & 3))) & 0xFFu) * kLutCopies];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const int64_t k = (c * 16 + b) * 5 + i;
          if (k < K) out[k] = (int8_t)((int)((e >> (4 * i)) & 15u) - 1);
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

// ---------------------------------------------------------------------------
// host-side launch helpers
// ---------------------------------------------------------------------------
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bgg_status hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BGG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return BGG_OK;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Token counts one GEMV kernel handles at once; a larger M runs in groups of
// kGemvTokens tokens (each group reads the weights again).
constexpr int kGemvTokens = 4;
inline int gemv_m_bucket(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

int64_t target_waves() {
  static int64_t t = [] {
    const char* e = getenv("BGG_GEMV_TARGET_WAVES");
    int64_t v = e ? atoll(e) : 0;
    return v > 0 ? v : int64_t(1536);
  }();
  return t;
}

// Split of K for a GEMV: units of work along K (PQ2_0: groups, PTQ1_0:
// periods of 5 groups), units per slice, slice count, and workspace layout.
struct GemvPlan {
  int64_t G, gpad, units, per_slice, S, NT, Mb, frag_words_per_token;
  uint64_t off_meta_q, off_meta_f, off_partial, off_counters, total;
};

GemvPlan plan_gemv(const bgg_weights_desc* d, int64_t M) {
  GemvPlan p{};
  p.G = d->groups;
  p.NT = d->row_tiles;
  p.Mb = gemv_m_bucket(M);
  if (d->format == BGG_FMT_PQ2_0) {
    p.gpad = p.G;
    p.units = p.G;
    p.frag_words_per_token = (d->K / 64) * kPqFragWords;
    // groups per slice: 8, 4 or 2 -- the largest that still gives the
    // target number of waves
    p.per_slice = 8;
    while (p.per_slice > 2 && p.NT * ceil_div(p.units, p.per_slice) < target_waves()) p.per_slice /= 2;
  } else {
    const int64_t P = ceil_div(p.G, kPeriodGroups);
    p.gpad = P * kPeriodGroups;
    p.units = P;
    p.frag_words_per_token = P * kPtqFragWords;
    p.per_slice = (p.NT * ceil_div(P, 2) >= target_waves()) ? 2 : 1;
  }
  p.S = ceil_div(p.units, p.per_slice);
  uint64_t off = align256((uint64_t)p.Mb * p.frag_words_per_token * 4);
  p.off_meta_q = off;
  off = align256(off + (uint64_t)p.Mb * p.gpad * 4);
  p.off_meta_f = off;
  off = align256(off + (uint64_t)p.Mb * p.gpad * 4);
  p.off_partial = off;
  off = align256(off + (p.S > 1 ? (uint64_t)p.Mb * p.S * p.NT * kTile * 4 : 0));
  p.off_counters = off;
  off = align256(off + (uint64_t)p.NT * 4);
  p.total = off;
  return p;
}

struct GemvArgs {
  const bgg_weights_desc* d;
  const uint8_t* packed;
  const uint16_t* x;
  uint16_t* y;
  int Mreal;
  int rotate;
  uint8_t* ws;
  hipStream_t st;
};

template <int M>
void launch_gemv(const GemvArgs& a, const GemvPlan& p) {
  const bgg_weights_desc* d = a.d;
  uint32_t* frag = reinterpret_cast<uint32_t*>(a.ws);
  int32_t* mq = reinterpret_cast<int32_t*>(a.ws + p.off_meta_q);
  float* mf = reinterpret_cast<float*>(a.ws + p.off_meta_f);
  float* part = reinterpret_cast<float*>(a.ws + p.off_partial);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(a.ws + p.off_counters);
  const int S = (int)p.S;
  const int64_t tiles_per_xcd = ceil_div(p.NT, kWaves);
  const dim3 pgrid((unsigned)ceil_div(p.gpad, kPrepGroups), (unsigned)M);
  if (d->format == BGG_FMT_PQ2_0) {
    hipLaunchKernelGGL(k_gemv_prep<BGG_FMT_PQ2_0>, pgrid, dim3(kPrepThreads), 0, a.st, a.x, d->K,
                       a.Mreal, a.rotate, frag, p.frag_words_per_token, mq, mf, p.gpad, cnt, p.NT);
    const dim3 grid((unsigned)(kWaves * tiles_per_xcd * S));
#define BGG_PQ2(BPS)                                                                              \
  hipLaunchKernelGGL((k_gemv_pq2<M, BPS>), grid, dim3(64), 0, a.st, a.packed, d->scale_offset,  \
                     p.NT, d->chunks, p.G, d->N, S, a.Mreal, frag, mq, mf, part, cnt, a.y)
    if (p.per_slice == 8)
      BGG_PQ2(8);
    else if (p.per_slice == 4)
      BGG_PQ2(4);
    else
      BGG_PQ2(2);
#undef BGG_PQ2
  } else {
    hipLaunchKernelGGL(k_gemv_prep<BGG_FMT_PTQ1_0>, pgrid, dim3(kPrepThreads), 0, a.st, a.x, d->K,
                       a.Mreal, a.rotate, frag, p.frag_words_per_token, mq, mf, p.gpad, cnt, p.NT);
    const int64_t items = tiles_per_xcd * S;
    const dim3 grid((unsigned)(kWaves * ceil_div(items, 4)));
#define BGG_PTQ1(PPS)                                                                              \
  hipLaunchKernelGGL((k_gemv_ptq1<M, PPS>), grid, dim3(256), 0, a.st, a.packed, d->scale_offset, \
                     p.NT, d->chunks, p.G, d->N, S, a.Mreal, items, frag, p.frag_words_per_token, \
                     mq, mf, p.gpad, part, cnt, a.y)
    if (p.per_slice == 2)
      BGG_PTQ1(2);
    else
      BGG_PTQ1(1);
#undef BGG_PTQ1
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

bgg_status bgg_hadamard_rotate(const void* x_dev, void* xr_dev, int64_t M, int64_t K,
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

bgg_status bgg_unpack_weights(const bgg_weights_desc* d, const void* packed_dev, int8_t* trits_dev,
                              uint16_t* scales_dev, void* stream) {
  bgg_status st = bgg::check_desc(d);
  if (st) return st;
  if (!packed_dev || !trits_dev || !scales_dev)
    return fail(BGG_ERR_NULL, "bgg_unpack_weights: NULL buffer");
  if (!aligned16(packed_dev)) return fail(BGG_ERR_BUFFER, "bgg_unpack_weights: packed misaligned");
  const int64_t threads = d->row_tiles * d->chunks * kTile;
  const dim3 grid((unsigned)ceil_div(threads, 256));
  if (d->format == BGG_FMT_PQ2_0)
    hipLaunchKernelGGL(k_unpack<BGG_FMT_PQ2_0>, grid, dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)packed_dev, d->scale_offset, d->row_tiles, d->chunks,
                       d->groups, d->N, d->K, trits_dev, scales_dev);
  else
    hipLaunchKernelGGL(k_unpack<BGG_FMT_PTQ1_0>, grid, dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)packed_dev, d->scale_offset, d->row_tiles, d->chunks,
                       d->groups, d->N, d->K, trits_dev, scales_dev);
  return hip_check("bgg_unpack_weights");
}

size_t bgg_gemv_workspace_size(const bgg_weights_desc* d, int64_t M) {
  if (bgg::check_desc(d) != BGG_OK || M < 1 || M > BGG_MAX_GEMV_M) return 0;
  return (size_t)plan_gemv(d, M).total;
}

bgg_status bgg_ternary_gemv(const bgg_weights_desc* d, const void* packed_dev, const void* x_dev,
                            void* y_dev, int64_t M, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bgg_status st = bgg::check_desc(d);
  if (st) return st;
  if (!packed_dev || !x_dev || !y_dev || !workspace)
    return fail(BGG_ERR_NULL, "bgg_ternary_gemv: NULL buffer");
  if (M < 1 || M > BGG_MAX_GEMV_M)
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: M must be in 1..16 (got %lld)", (long long)M);
  if (flags & ~(uint32_t)BGG_ROTATE_INPUT)
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: unknown flags 0x%x", flags);
  if (!aligned16(packed_dev) || !aligned16(x_dev) || !aligned16(workspace) || ((uintptr_t)y_dev & 1))
    return fail(BGG_ERR_BUFFER, "bgg_ternary_gemv: misaligned buffer");
  const GemvPlan p = plan_gemv(d, M);
  if (workspace_bytes < p.total)
    return fail(BGG_ERR_BUFFER, "bgg_ternary_gemv: workspace has %zu bytes, needs %llu",
                workspace_bytes, (unsigned long long)p.total);
  GemvArgs a{d, (const uint8_t*)packed_dev, nullptr, nullptr, 0,
             (flags & BGG_ROTATE_INPUT) ? 1 : 0, (uint8_t*)workspace, (hipStream_t)stream};
  for (int64_t m0 = 0; m0 < M; m0 += kGemvTokens) {
    const int64_t mg = M - m0 < kGemvTokens ? M - m0 : kGemvTokens;
    a.x = (const uint16_t*)x_dev + m0 * d->K;
    a.y = (uint16_t*)y_dev + m0 * d->N;
    a.Mreal = (int)mg;
    switch (gemv_m_bucket(mg)) {
      case 1: launch_gemv<1>(a, p); break;
      case 2: launch_gemv<2>(a, p); break;
      default: launch_gemv<4>(a, p); break;
    }
    if ((st = hip_check("bgg_ternary_gemv"))) return st;
  }
  return BGG_OK;
}

}  // extern "C"
