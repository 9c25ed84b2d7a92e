// Prompt-time products for gfx950: Y[M][N] = X'[M][K] . (S*T)[N][K]^T, for
// PQ2_0 (k_gemm_pq2) and PTQ1_0 (k_gemm_ptq1).
//
// allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), packing paragraph: PQ2_0
// is the packing that wins prompt processing; method paragraph: trits with
// one FP16 scale per 128 weights.  This is the one dense contraction of the
// path, so it runs on the matrix cores: trit tiles are decoded to fp16 s*t
// (exact: the value is +-s or 0) straight into LDS and multiplied with fp16
// x' tiles by v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//
// Tiling: a 256-thread workgroup computes a 128 (tokens) x 256 (weight rows)
// block of Y; each of its four waves owns 64 weight rows (one row tile of
// the packed layout) and all 128 tokens: 4 x 2 MFMA tiles of 32 x 32, K
// stepping by 64 (one 16-byte packed chunk per weight row).
//   * activations: the 128 x 64 fp16 tile of a step is staged in LDS
//     (double-buffered, shared by the four waves); the loads of step k+1 are
//     in flight while the matrix cores work on step k;
//   * weights: every lane loads the packed chunk of its own weight row
//     straight into registers (2 bits per weight: 1 KiB per wave per step)
//     and decodes the codes it feeds to the MFMA to fp16 s*t in registers --
//     exact, since the value is +-s or 0 -- so the weights never touch LDS.
//     The decode (a few VALU operations per pair of weights) overlaps the
//     MFMAs of the other waves; the tall wave tile (128 tokens) spreads it
//     over four MFMA rows.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>

#include "bgg_device.h"

using bgg::fail;
using bgg::f16x8;
using bgg::f32x16;
using bgg::decode8_pq2;
using bgg::ceil_div;

namespace {

constexpr int kBM = 128, kBN = 256, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // halves per LDS row (+16 bytes against bank conflicts)
constexpr int kTileRows = BGG_ROW_TILE;

// K split (gridDim.z == 2): workgroup z runs K steps [0, kmid) or [kmid,
// steps) and writes fp32 partial sums to P[z][M][N]; k_gemm_sum2 adds the two
// and rounds to fp16.  gridDim.z == 1: all of K, fp16 y.
__global__ void __launch_bounds__(256, 2)
    k_gemm_pq2(const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed,
               uint64_t scale_offset, int64_t M, int64_t N, int64_t K, int64_t C, int64_t G,
               int64_t NT, int64_t kmid, float* __restrict__ P, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsStride];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

  // activation loader: row tid/2 of the tile, k half tid%2 (32 values);
  // rows past M re-read row M-1 (never stored)
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t am = m0 + lr < M ? m0 + lr : M - 1;
  const uint16_t* a_src = X + am * K + lh * 32;

  // this wave's weight rows: row tile n0/64 + wave (past the last tile it
  // re-reads the last one and stores nothing); N-subtile j holds rows
  // j*32 + li of the tile
  const int64_t tw = n0 / kTileRows + wave;
  const bool w_ok = tw < NT;
  const int64_t tcl = w_ok ? tw : NT - 1;
  const uint4* b_src = reinterpret_cast<const uint4*>(packed) + tcl * C * kTileRows + li;
  const uint16_t* s_src =
      reinterpret_cast<const uint16_t*>(packed + scale_offset) + tcl * G * kTileRows + li;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Software pipeline over K steps of 64: the activation pieces of step
  // ks+2 and the packed chunks and scales of step ks+1 are loaded while step
  // ks is multiplied; step ks+1's activations (loaded one iteration earlier)
  // go to the other LDS buffer at the end of the iteration.  Loads past the
  // last step re-read the last step (no branch splits the registers), and
  // the two activation register sets alternate, so the loop is unrolled by
  // two (K / 64 is even since K is a multiple of 128).
  // this workgroup's K steps [kb, steps): both ranges have even lengths
  const int64_t kb = blockIdx.z == 0 ? 0 : kmid;
  const int64_t steps = gridDim.z == 1 || blockIdx.z == 1 ? K / kBK : kmid;
  uint4 xa0, xa1, xa2, xa3, ya0, ya1, ya2, ya3, b0, b1;
  uint16_t s0, s1;
#define BGG_LOAD_A(KS, R0, R1, R2, R3)                                       \
  do {                                                                       \
    const int64_t kc_ = (KS) < steps ? (KS) : steps - 1;                     \
    const uint4* ap_ = reinterpret_cast<const uint4*>(a_src + kc_ * kBK);    \
    R0 = ap_[0], R1 = ap_[1], R2 = ap_[2], R3 = ap_[3];                      \
  } while (0)
#define BGG_LOAD_B(KS)                                                       \
  do {                                                                       \
    const int64_t kc_ = (KS) < steps ? (KS) : steps - 1;                     \
    b0 = b_src[kc_ * kTileRows], b1 = b_src[kc_ * kTileRows + 32];           \
    s0 = s_src[(kc_ / 2) * kTileRows], s1 = s_src[(kc_ / 2) * kTileRows + 32]; \
  } while (0)
#define BGG_STORE_A(BUF, R0, R1, R2, R3)                                     \
  do {                                                                       \
    uint4* d_ = reinterpret_cast<uint4*>(&As[BUF][lr * kLdsStride + lh * 32]); \
    d_[0] = R0, d_[1] = R1, d_[2] = R2, d_[3] = R3;                          \
  } while (0)
#define BGG_STEP(KS, CUR, L0, L1, L2, L3, S0, S1, S2, S3)                    \
  do {                                                                       \
    const uint4 bw[2] = {b0, b1};                                            \
    __half2 s2[2];                                                           \
    s2[0] = __halves2half2(__ushort_as_half(s0), __ushort_as_half(s0));      \
    s2[1] = __halves2half2(__ushort_as_half(s1), __ushort_as_half(s1));      \
    BGG_LOAD_A((KS) + 2, L0, L1, L2, L3);                                    \
    BGG_LOAD_B((KS) + 1);                                                    \
    __builtin_amdgcn_sched_barrier(0);                                       \
    _Pragma("unroll") for (int kk = 0; kk < kBK / 16; ++kk) {                \
      f16x8 a[4], b[2];                                                      \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) a[i] =                   \
          *reinterpret_cast<const f16x8*>(                                   \
              &As[CUR][(i * 32 + li) * kLdsStride + kk * 16 + h * 8]);       \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                        \
        const uint32_t w_ = kk == 0 ? bw[j].x : kk == 1 ? bw[j].y            \
                            : kk == 2 ? bw[j].z : bw[j].w;                   \
        b[j] = decode8_pq2(w_ >> (16 * h), s2[j]);                               \
      }                                                                      \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                          \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] =           \
          __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0); \
    }                                                                        \
    BGG_STORE_A((CUR) ^ 1, S0, S1, S2, S3);                                  \
    __syncthreads();                                                         \
  } while (0)

  BGG_LOAD_A(kb, xa0, xa1, xa2, xa3);
  BGG_LOAD_B(kb);
  BGG_STORE_A(0, xa0, xa1, xa2, xa3);
  BGG_LOAD_A(kb + 1, ya0, ya1, ya2, ya3);
  __syncthreads();
  for (int64_t ks = kb; ks < steps; ks += 2) {
    BGG_STEP(ks, 0, xa0, xa1, xa2, xa3, ya0, ya1, ya2, ya3);
    BGG_STEP(ks + 1, 1, ya0, ya1, ya2, ya3, xa0, xa1, xa2, xa3);
  }
#undef BGG_LOAD_A
#undef BGG_LOAD_B
#undef BGG_STORE_A
#undef BGG_STEP

  // D layout of a 32x32 tile: lane l holds column l%32 (a weight row), rows
  // (tokens) 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
  if (!w_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = tw * kTileRows + j * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M && n < N) {
          if (gridDim.z > 1)
            P[(blockIdx.z * M + m) * N + n] = acc[i][j][r];
          else
            Y[m * N + n] = __half_as_ushort(__float2half_rn(acc[i][j][r]));
        }
      }
    }
}

// y = fp16(P[0] + P[1]) over M*N values, four per thread (16-byte loads
// when M*N is a multiple of 4, so that the second partial is aligned too;
// else, and for the tail, one by one).
__global__ void __launch_bounds__(256) k_gemm_sum2(const float* __restrict__ P, int64_t MN,
                                                   uint16_t* __restrict__ Y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  if (i + 4 <= MN && (MN & 3) == 0) {
    const float4 a = *reinterpret_cast<const float4*>(P + i);
    const float4 b = *reinterpret_cast<const float4*>(P + MN + i);
    const uint32_t lo = (uint32_t)__half_as_ushort(__float2half_rn(a.x + b.x)) |
                        ((uint32_t)__half_as_ushort(__float2half_rn(a.y + b.y)) << 16);
    const uint32_t hi = (uint32_t)__half_as_ushort(__float2half_rn(a.z + b.z)) |
                        ((uint32_t)__half_as_ushort(__float2half_rn(a.w + b.w)) << 16);
    if (((uintptr_t)(Y + i) & 7) == 0) {
      *reinterpret_cast<uint2*>(Y + i) = make_uint2(lo, hi);
    } else {
      Y[i] = (uint16_t)lo, Y[i + 1] = (uint16_t)(lo >> 16);
      Y[i + 2] = (uint16_t)hi, Y[i + 3] = (uint16_t)(hi >> 16);
    }
  } else {
    const int64_t e = i + 4 < MN ? i + 4 : MN;
    for (int64_t k = i; k < e; ++k) Y[k] = __half_as_ushort(__float2half_rn(P[k] + P[MN + k]));
  }
}

// ---------------------------------------------------------------------------
// PTQ1_0 (allhereai.com/news/1346, packing paragraph: the compact packing;
// wmrh.cn/news/471187, section 关键机制: five trits per byte).  The same
// tiling as k_gemm_pq2 with a K step of 80: one 16-byte chunk of a row's
// base-3 stream.  Each lane turns the 16 bytes of its two rows into the
// 2-bit code string of their 80 trits (code t + 1 in natural order, ten bits
// per byte from a 256-entry LDS table), which is exactly the PQ2_0 code
// word layout, so the same fp16 s*t decode feeds the MFMA; every 16-K slice
// lies inside one 128-group, whose scale it takes.  Activation loads past K
// (the last chunk's tail, and the padding step when the chunk count is odd)
// are zero, so the zero trits there meet zeros.
// ---------------------------------------------------------------------------
constexpr int kBK3 = 80;
constexpr int kLdsStride3 = kBK3 + 8;  // halves per LDS row (176 bytes)

__global__ void __launch_bounds__(256, 2)
    k_gemm_ptq1(const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed,
                uint64_t scale_offset, int64_t M, int64_t N, int64_t K, int64_t C, int64_t G,
                int64_t NT, int64_t kmid, float* __restrict__ P, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsStride3];
  __shared__ uint32_t lut[256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

  // byte -> its five codes t_i + 1 in bits 2i..2i+1 (bytes past 242: zero trits)
  {
    uint32_t b = (uint32_t)tid, c = 0;
    if (b < 243) {
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        c |= (b % 3u) << (2 * i);
        b /= 3u;
      }
    } else {
      c = 0x155u;
    }
    lut[tid] = c;
  }

  // activation loader: row tid/2 of the tile, 40 halves (five 16-byte
  // pieces) at 40 (tid % 2); rows past M re-read row M-1 (never stored)
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t am = m0 + lr < M ? m0 + lr : M - 1;
  const uint16_t* a_src = X + am * K + lh * 40;

  const int64_t tw = n0 / kTileRows + wave;
  const bool w_ok = tw < NT;
  const int64_t tcl = w_ok ? tw : NT - 1;
  const uint4* b_src = reinterpret_cast<const uint4*>(packed) + tcl * C * kTileRows + li;
  const uint16_t* s_src =
      reinterpret_cast<const uint16_t*>(packed + scale_offset) + tcl * G * kTileRows + li;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // The pipeline of k_gemm_pq2 over steps of 80; an odd chunk count gets a
  // padding step of zero activations so the two register sets alternate.
  // this workgroup's chunks [kb, steps) (the K split as in k_gemm_pq2),
  // padded to an even count with zero activations
  const int64_t kb = blockIdx.z == 0 ? 0 : kmid;
  const int64_t steps = gridDim.z == 1 || blockIdx.z == 1 ? C : kmid;
  const int64_t steps2 = kb + ((steps - kb + 1) & ~int64_t(1));
  uint4 xa[5], ya[5], bown;
  uint16_t s0[2], s1[2];
#define BGG_LOAD_A3(KS, R)                                                      \
  do {                                                                         \
    const int64_t k_ = (KS) * kBK3 + lh * 40;                                  \
    const uint4* ap_ = reinterpret_cast<const uint4*>(a_src + (KS) * kBK3);     \
    _Pragma("unroll") for (int q = 0; q < 5; ++q)                              \
      R[q] = (KS) < steps && k_ + 8 * q < K ? ap_[q] : make_uint4(0, 0, 0, 0);  \
  } while (0)
#define BGG_LOAD_B3(KS)                                                         \
  do {                                                                         \
    const int64_t kc_ = (KS) < steps ? (KS) : steps - 1;                       \
    bown = b_src[kc_ * kTileRows + 32 * h];                                    \
    const int64_t g0_ = (kc_ * kBK3) >> 7;                                      \
    const int64_t g1_ = g0_ + 1 < G ? g0_ + 1 : G - 1;                          \
    s0[0] = s_src[g0_ * kTileRows], s1[0] = s_src[g0_ * kTileRows + 32];       \
    s0[1] = s_src[g1_ * kTileRows], s1[1] = s_src[g1_ * kTileRows + 32];       \
  } while (0)
#define BGG_STORE_A3(BUF, R)                                                    \
  do {                                                                         \
    uint4* d_ = reinterpret_cast<uint4*>(&As[BUF][lr * kLdsStride3 + lh * 40]); \
    _Pragma("unroll") for (int q = 0; q < 5; ++q) d_[q] = R[q];                \
  } while (0)
#define BGG_STEP3(KS, CUR, L, S)                                                \
  do {                                                                         \
    const uint4 bw = bown;                                                     \
    __half2 s2[2][2];                                                          \
    _Pragma("unroll") for (int e = 0; e < 2; ++e) {                            \
      s2[0][e] = __halves2half2(__ushort_as_half(s0[e]), __ushort_as_half(s0[e])); \
      s2[1][e] = __halves2half2(__ushort_as_half(s1[e]), __ushort_as_half(s1[e])); \
    }                                                                          \
    /* lane (li, h) turns the chunk of its own row 32 h + li into the 80     \
       codes (five words of sixteen 2-bit codes), keeps the halves its K   \
       slices read (codes 16 kk + 8 h .. + 7) and hands the other halves    \
       to lane (li, 1 - h), which reads the same slices of the other half   \
       of K for this row; two halves per register */                        \
    uint32_t mine[3], theirs[3];                                               \
    {                                                                          \
      uint64_t bits_ = 0;                                                      \
      int nb_ = 0, w_ = 0;                                                     \
      _Pragma("unroll") for (int q = 0; q < 16; ++q) {                         \
        const uint32_t word_ = q < 4 ? bw.x : q < 8 ? bw.y : q < 12 ? bw.z : bw.w; \
        bits_ |= (uint64_t)lut[(word_ >> (8 * (q & 3))) & 0xFFu] << nb_;       \
        nb_ += 10;                                                             \
        if (nb_ >= 32) {                                                       \
          const uint32_t cw_ = (uint32_t)bits_;                                \
          const uint32_t my_ = __builtin_amdgcn_ubfe(cw_, 16 * h, 16);         \
          const uint32_t ot_ = __builtin_amdgcn_ubfe(cw_, 16 - 16 * h, 16);    \
          if (w_ % 2 == 0) {                                                   \
            mine[w_ / 2] = my_;                                                \
            theirs[w_ / 2] = ot_;                                              \
          } else {                                                             \
            mine[w_ / 2] |= my_ << 16;                                         \
            theirs[w_ / 2] |= ot_ << 16;                                       \
          }                                                                    \
          ++w_;                                                                \
          bits_ >>= 32;                                                        \
          nb_ -= 32;                                                           \
        }                                                                      \
      }                                                                        \
    }                                                                          \
    uint32_t ch[2][3];                                                         \
    _Pragma("unroll") for (int r_ = 0; r_ < 3; ++r_) {                         \
      const uint32_t got_ = (uint32_t)__builtin_amdgcn_ds_bpermute(            \
          (lane ^ 32) * 4, (int)theirs[r_]);                                   \
      ch[0][r_] = h ? got_ : mine[r_];                                         \
      ch[1][r_] = h ? mine[r_] : got_;                                         \
    }                                                                          \
    const int64_t g0s_ = ((KS) < steps ? (KS) : steps - 1) * kBK3 >> 7;        \
    const int64_t kbase_ = ((KS) < steps ? (KS) : steps - 1) * kBK3;            \
    BGG_LOAD_A3((KS) + 2, L);                                                  \
    BGG_LOAD_B3((KS) + 1);                                                     \
    __builtin_amdgcn_sched_barrier(0);                                         \
    _Pragma("unroll") for (int kk = 0; kk < kBK3 / 16; ++kk) {                 \
      const int sel_ = ((kbase_ + 16 * kk) >> 7) != g0s_;                      \
      f16x8 a[4], b[2];                                                        \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) a[i] =                     \
          *reinterpret_cast<const f16x8*>(                                     \
              &As[CUR][(i * 32 + li) * kLdsStride3 + kk * 16 + h * 8]);        \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                            \
          b[j] = decode8_pq2(ch[j][kk / 2] >> (16 * (kk % 2)), sel_ ? s2[j][1] : s2[j][0]); \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                            \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] =             \
          __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0); \
    }                                                                          \
    BGG_STORE_A3((CUR) ^ 1, S);                                                \
    __syncthreads();                                                           \
  } while (0)

  BGG_LOAD_A3(kb, xa);
  BGG_LOAD_B3(kb);
  BGG_STORE_A3(0, xa);
  BGG_LOAD_A3(kb + 1, ya);
  __syncthreads();  // (also publishes the code table)
  for (int64_t ks = kb; ks < steps2; ks += 2) {
    BGG_STEP3(ks, 0, xa, ya);
    BGG_STEP3(ks + 1, 1, ya, xa);
  }
#undef BGG_LOAD_A3
#undef BGG_LOAD_B3
#undef BGG_STORE_A3
#undef BGG_STEP3

  if (!w_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = tw * kTileRows + j * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M && n < N) {
          if (gridDim.z > 1)
            P[(blockIdx.z * M + m) * N + n] = acc[i][j][r];
          else
            Y[m * N + n] = __half_as_ushort(__float2half_rn(acc[i][j][r]));
        }
      }
    }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (cached per device).
int64_t gemm_device_cus() {
  static int64_t cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// K split in two when the output blocks fill the resident workgroup slots
// (two per CU) much less evenly than twice as many would: the last, partly
// empty round of workgroups (e.g. 640 blocks on 512 slots for 4096 tokens x
// 5120 rows) costs as much as a full one.  The fp32 partials cost an extra
// pass over 2 M N floats, so the split must gain at least 15 %.
bool gemm_split(const bgg_weights_desc* d, int64_t M) {
  static const int64_t on = [] {
    const char* e = getenv("BGG_GEMM_SPLIT");
    return e && *e ? (int64_t)atoll(e) : int64_t(1);
  }();
  if (!on) return false;
  const int64_t steps = d->format == BGG_FMT_PQ2_0 ? d->K / kBK : d->chunks;
  if (steps < 8) return false;
  const int64_t mc = M < int64_t(65535) * kBM ? M : int64_t(65535) * kBM;
  const double wgs = (double)((d->N + kBN - 1) / kBN) * (double)((mc + kBM - 1) / kBM);
  const double waves = wgs / (double)(2 * gemm_device_cus());
  const double eff1 = waves / std::ceil(waves), eff2 = 2 * waves / std::ceil(2 * waves);
  return eff2 > 1.15 * eff1;
}

uint64_t gemm_rot_bytes(const bgg_weights_desc* d, int64_t M) {
  return ((uint64_t)M * d->K * 2 + 255) & ~uint64_t(255);
}

// fp32 partials of one launch (at most 65535 token blocks)
uint64_t gemm_part_bytes(const bgg_weights_desc* d, int64_t M) {
  const int64_t mc = M < int64_t(65535) * kBM ? M : int64_t(65535) * kBM;
  return (uint64_t)2 * mc * d->N * 4;
}

}  // namespace

extern "C" {

size_t bgg_gemm_workspace_size(const bgg_weights_desc* d, int64_t M) {
  if (bgg::check_desc(d) != BGG_OK || M < 1) return 0;
  return (size_t)(gemm_rot_bytes(d, M) + (gemm_split(d, M) ? gemm_part_bytes(d, M) : 0));
}

bgg_status bgg_ternary_gemm(const bgg_weights_desc* d, const void* packed_dev, const void* x_dev,
                            void* y_dev, int64_t M, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bgg_status st = bgg::check_desc(d);
  if (st) return st;
  if (d->format != BGG_FMT_PQ2_0 && d->format != BGG_FMT_PTQ1_0)
    return fail(BGG_ERR_FORMAT, "bgg_ternary_gemm: only PQ2_0 and PTQ1_0 weights have a "
                                "prompt-time kernel");
  if (!packed_dev || !x_dev || !y_dev) return fail(BGG_ERR_NULL, "bgg_ternary_gemm: NULL buffer");
  if (M < 1 || M > (int64_t(1) << 31))
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemm: M must be >= 1 (got %lld)", (long long)M);
  if (flags & ~(uint32_t)BGG_ROTATE_INPUT)
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemm: unknown flags 0x%x", flags);
  if (!aligned16(packed_dev) || !aligned16(x_dev) || ((uintptr_t)y_dev & 1))
    return fail(BGG_ERR_BUFFER, "bgg_ternary_gemm: misaligned buffer");
  if (workspace && !aligned16(workspace))
    return fail(BGG_ERR_BUFFER, "bgg_ternary_gemm: misaligned workspace");
  hipStream_t s = (hipStream_t)stream;
  const void* xr = x_dev;
  uint64_t used = 0;
  if (flags & BGG_ROTATE_INPUT) {
    const uint64_t need = gemm_rot_bytes(d, M);
    if (!workspace || workspace_bytes < need)
      return fail(BGG_ERR_BUFFER, "bgg_ternary_gemm: rotation needs a 16-byte aligned workspace "
                                  "of %llu bytes", (unsigned long long)need);
    if ((st = bgg_hadamard_rotate(x_dev, workspace, M, d->K, stream))) return st;
    xr = workspace;
    used = need;
  }
  // the K split runs only when the workspace also holds its partials
  float* P = nullptr;
  if (workspace && gemm_split(d, M) && workspace_bytes >= used + gemm_part_bytes(d, M))
    P = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + used);
  const int64_t steps = d->format == BGG_FMT_PQ2_0 ? d->K / kBK : d->chunks;
  const int64_t kmid = (steps / 2) & ~int64_t(1);  // even: both halves stay even
  // token blocks go on grid.y, which holds at most 65535 blocks: longer
  // prompts run as several launches over consecutive token ranges
  const int64_t max_m = int64_t(65535) * kBM;
  for (int64_t m0 = 0; m0 < M; m0 += max_m) {
    const int64_t mc = M - m0 < max_m ? M - m0 : max_m;
    const dim3 grid((unsigned)((d->N + kBN - 1) / kBN), (unsigned)((mc + kBM - 1) / kBM),
                    P ? 2u : 1u);
    uint16_t* y = (uint16_t*)y_dev + m0 * d->N;
    hipLaunchKernelGGL(d->format == BGG_FMT_PQ2_0 ? k_gemm_pq2 : k_gemm_ptq1, grid, dim3(256), 0, s,
                       (const uint16_t*)xr + m0 * d->K, (const uint8_t*)packed_dev,
                       d->scale_offset, mc, d->N, d->K, d->chunks, d->groups, d->row_tiles, kmid,
                       P, y);
    if (P) {
      const int64_t mn = mc * d->N;
      hipLaunchKernelGGL(k_gemm_sum2, dim3((unsigned)ceil_div(ceil_div(mn, 4), 256)), dim3(256), 0,
                         s, (const float*)P, mn, y);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BGG_ERR_HIP, "bgg_ternary_gemm: %s", hipGetErrorString(e));
  return BGG_OK;
}

}  // extern "C"
