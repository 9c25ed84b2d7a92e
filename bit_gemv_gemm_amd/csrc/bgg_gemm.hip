// Prompt-time products for gfx950: Y[M][N] = X'[M][K] . (S*T)[N][K]^T, for
// PQ2_0 (k_gemm_pq2) and PTQ1_0 (k_gemm_ptq1).
//
// allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), packing paragraph: PQ2_0
// is the packing that wins prompt processing; method paragraph: trits with
// one FP16 scale per 128 weights.  This is the one dense contraction of the
// path, so it runs on the matrix cores: trit tiles are decoded to fp16 s*t
// (exact: the value is +-s or 0) in registers and multiplied with fp16 x'
// tiles by v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//
// Tiling: a 256-thread workgroup computes a 128 (tokens) x 256 (weight rows)
// block of Y; each of its four waves owns 64 weight rows (one row tile of
// the packed layout) and all 128 tokens: 4 x 2 MFMA tiles of 32 x 32, K
// stepping by 128 (two 16-byte packed chunks per weight row, one scale
// group).
//   * activations: the 128 x 128 fp16 tile of a step goes from global memory
//     straight into LDS (gfx950 global-to-LDS loads, no registers on the
//     way), double-buffered and shared by the four waves; the loads of step
//     k+1 are in flight while the matrix cores work on step k;
//   * weights: every lane loads the packed chunks of its own weight row
//     straight into registers (2 bits per weight: 2 KiB per wave per step)
//     and decodes the codes it feeds to the MFMA to fp16 s*t in registers --
//     exact, since the value is +-s or 0 -- so the weights never touch LDS.
//     The decode (two byte permutes per pair of weights, reading a table of
//     -s, 0, +s built once per scale) overlaps the MFMAs of the other waves;
//     the tall wave tile (128 tokens) spreads it over four MFMA rows.
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

constexpr int kBM = 128, kBN = 256, kBK = 64;  // kBK: one packed chunk
constexpr int kTileRows = BGG_ROW_TILE;

// K split in S = gridDim.z ranges (S <= K / 128): workgroup z runs the
// 128-wide K steps [z T / S, (z + 1) T / S) of the T = K / 128 and writes
// fp32 partial sums to P[z][M][N]; k_gemm_sum adds the S partials in order
// z = 0, 1, ... and rounds to fp16.  gridDim.z == 1: all of K, fp16 y.
//
// An LDS activation buffer holds the 128 x 128 tile of a step as 16-byte
// pieces, piece q (halves 8q..8q+7) of row r at slot r * 16 + (q ^ (r & 15)).
// A global-to-LDS load writes the 16 bytes of lane l at the wave's LDS base
// + 16 l, so one load instruction fills four whole rows (each lane fetching
// the piece its slot holds), and the MFMA reads (sixteen consecutive rows
// at one q per 16 lanes) hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ int a_slot(int r, int q) { return r * 16 + (q ^ (r & 15)); }

// Wait for this wave's outstanding loads (global-to-LDS included) and LDS
// reads, then the workgroup barrier.  Written out because the fence that
// __syncthreads carries would make the compiler wait for them all before
// every barrier anyway, while the "memory" clobber keeps it from moving LDS
// accesses across this point.
__device__ __forceinline__ void lds_dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ void __launch_bounds__(256, 2)
    k_gemm_pq2(const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed,
               const uint16_t* __restrict__ scales, int64_t M, int64_t N, int64_t K, int64_t C,
               int64_t G,
               int64_t NT, int64_t kmid, float* __restrict__ P, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint4 As0[kBM * 16];
  __shared__ __attribute__((aligned(16))) uint4 As1[kBM * 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

  // activation loader: load instruction i of this wave fills slots
  // (8 wave + i) * 64 + lane, i.e. row (8 wave + i) * 4 + lane / 16, piece
  // (lane % 16) ^ (row & 15); rows past M re-read row M-1 (never stored)
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (8 * wave + i) * 4 + (lane >> 4);
    const int q = (lane & 15) ^ (r & 15);
    const int64_t am = m0 + r < M ? m0 + r : M - 1;
    a_src[i] = X + am * K + 8 * q;
  }

  // this wave's weight rows: row tile n0/64 + wave (past the last tile it
  // re-reads the last one and stores nothing); N-subtile j holds rows
  // j*32 + li of the tile
  const int64_t tw = n0 / kTileRows + wave;
  const bool w_ok = tw < NT;
  const int64_t tcl = w_ok ? tw : NT - 1;
  const uint4* b_src = reinterpret_cast<const uint4*>(packed) + tcl * C * kTileRows + li;
  const uint16_t* s_src = scales + tcl * G * kTileRows + li;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // this workgroup's 128-wide K steps [kb, steps).  Step ks multiplies the
  // buffer filled during step ks-1 while step ks+1's activations stream into
  // the other buffer and its packed chunks (b2/b3: the second chunk) and
  // scales into registers (the last step reloads its own activations into
  // the idle buffer instead); each step ends with every wave's loads landed
  // and the barrier.  The loop is unrolled by two so that each buffer is its
  // own LDS object, which lets the compiler see that the loads in flight
  // never write the buffer being read.
  const int64_t T = K / (2 * kBK);
  const int64_t kb = (int64_t)blockIdx.z * T / gridDim.z;
  const int64_t steps = (int64_t)(blockIdx.z + 1) * T / gridDim.z;
  uint4 b0, b1, b2, b3;
  uint16_t s0, s1;
#define BGG_LOAD_A(KS, BUF)                                                   \
  do {                                                                        \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                             \
      __builtin_amdgcn_global_load_lds(                                       \
          a_src[i] + (KS) * 128,                                              \
          (__attribute__((address_space(3))) void*)&BUF[(8 * wave + i) * 64], \
          16, 0, 0);                                                          \
  } while (0)
#define BGG_LOAD_B(KS)                                                        \
  do {                                                                        \
    const int64_t kc_ = 2 * ((KS) < steps ? (KS) : steps - 1);                \
    b0 = b_src[kc_ * kTileRows], b1 = b_src[kc_ * kTileRows + 32];            \
    b2 = b_src[(kc_ + 1) * kTileRows], b3 = b_src[(kc_ + 1) * kTileRows + 32]; \
    s0 = s_src[(kc_ / 2) * kTileRows], s1 = s_src[(kc_ / 2) * kTileRows + 32]; \
  } while (0)
#define BGG_STEP(KS, CUR, NXT)                                                \
  do {                                                                        \
    const uint4 bw[2][2] = {{b0, b1}, {b2, b3}};                              \
    const bgg::Pq2Table tb[2] = {bgg::pq2_table(s0), bgg::pq2_table(s1)};     \
    __builtin_amdgcn_sched_barrier(0);                                        \
    BGG_LOAD_A((KS) + 1 < steps ? (KS) + 1 : (KS), NXT);                      \
    BGG_LOAD_B((KS) + 1);                                                     \
    __builtin_amdgcn_sched_barrier(0);                                        \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) {                        \
      f16x8 a[4], b[2];                                                       \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) a[i] =                    \
          *reinterpret_cast<const f16x8*>(&CUR[a_slot(i * 32 + li, 2 * kk + h)]); \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                         \
        const uint4 c_ = bw[kk >> 2][j];                                      \
        const int k4_ = kk & 3;                                               \
        const uint32_t w_ = k4_ == 0 ? c_.x : k4_ == 1 ? c_.y : k4_ == 2 ? c_.z : c_.w; \
        b[j] = decode8_pq2(w_, 16 * h, tb[j]);                                \
      }                                                                       \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                           \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] =            \
          __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0); \
    }                                                                         \
    lds_dma_barrier();                                                        \
  } while (0)

  BGG_LOAD_A(kb, As0);
  BGG_LOAD_B(kb);
  lds_dma_barrier();
  int64_t ks = kb;
  for (; ks + 1 < steps; ks += 2) {
    BGG_STEP(ks, As0, As1);
    BGG_STEP(ks + 1, As1, As0);
  }
  if (ks < steps) BGG_STEP(ks, As0, As1);
#undef BGG_LOAD_A
#undef BGG_LOAD_B
#undef BGG_STEP

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

// y = fp16(P[0] + P[1] + ... + P[S-1]) over M*N values (fp32 sums in that
// order), four per thread (16-byte loads when M*N is a multiple of 4, so
// that every partial is aligned too; else, and for the tail, one by one).
__global__ void __launch_bounds__(256) k_gemm_sum(const float* __restrict__ P, int S, int64_t MN,
                                                  uint16_t* __restrict__ Y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  if (i + 4 <= MN && (MN & 3) == 0) {
    float4 a = *reinterpret_cast<const float4*>(P + i);
    for (int z = 1; z < S; ++z) {
      const float4 b = *reinterpret_cast<const float4*>(P + z * MN + i);
      a.x += b.x, a.y += b.y, a.z += b.z, a.w += b.w;
    }
    const uint32_t lo = (uint32_t)__half_as_ushort(__float2half_rn(a.x)) |
                        ((uint32_t)__half_as_ushort(__float2half_rn(a.y)) << 16);
    const uint32_t hi = (uint32_t)__half_as_ushort(__float2half_rn(a.z)) |
                        ((uint32_t)__half_as_ushort(__float2half_rn(a.w)) << 16);
    if (((uintptr_t)(Y + i) & 7) == 0) {
      *reinterpret_cast<uint2*>(Y + i) = make_uint2(lo, hi);
    } else {
      Y[i] = (uint16_t)lo, Y[i + 1] = (uint16_t)(lo >> 16);
      Y[i + 2] = (uint16_t)hi, Y[i + 3] = (uint16_t)(hi >> 16);
    }
  } else {
    const int64_t e = i + 4 < MN ? i + 4 : MN;
    for (int64_t k = i; k < e; ++k) {
      float a = P[k];
      for (int z = 1; z < S; ++z) a += P[z * MN + k];
      Y[k] = __half_as_ushort(__float2half_rn(a));
    }
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
                const uint16_t* __restrict__ scales, int64_t M, int64_t N, int64_t K, int64_t C,
                int64_t G,
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
  const uint16_t* s_src = scales + tcl * G * kTileRows + li;

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
    bgg::Pq2Table tb[2][2];                                                    \
    _Pragma("unroll") for (int e = 0; e < 2; ++e) {                            \
      tb[0][e] = bgg::pq2_table(s0[e]);                                        \
      tb[1][e] = bgg::pq2_table(s1[e]);                                        \
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
          b[j] = decode8_pq2(ch[j][kk / 2], 16 * (kk % 2), sel_ ? tb[j][1] : tb[j][0]); \
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

// ---------------------------------------------------------------------------
// PTQ1_0 -> PQ2_0 row streams of one matrix (wmrh.cn/news/471187, section
// 关键机制: five trits per byte; allhereai.com/news/1346, packing paragraph:
// the 2-bit packing is the one that wins prompt processing).  When the
// workspace has room, the PTQ1_0 GEMM rewrites its weights once per call
// into the PQ2_0 device layout (same tiles, same scales) and runs k_gemm_pq2: the rewrite streams
// 1.6 + 2 bits per weight once, where the byte-to-code conversion inside
// k_gemm_ptq1 runs again for every 128 tokens.  Exact: both layouts hold the
// same trits.  k_gemm_ptq1 remains for calls without room for the rewrite.
//
// One thread per (row tile, 320-trit block, row of the tile): four PTQ1_0
// chunks (64 bytes, each byte five codes t + 1 low digit first, ten bits from
// a 256-entry table) in, the 640-bit code string = five PQ2_0 chunks out.
// Chunks past the end of the row are neither read nor written; bytes past
// 242 read as zero trits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    k_ptq1_to_pq2(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t C3, int64_t C2,
                  int64_t nblk, int64_t total) {
  __shared__ uint32_t lut[256];
  {
    uint32_t b = threadIdx.x, c = 0;
    if (b < 243) {
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        c |= (b % 3u) << (2 * i);
        b /= 3u;
      }
    } else {
      c = 0x155u;
    }
    lut[threadIdx.x] = c;
  }
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int64_t li = idx & 63, rest = idx >> 6;
  const int64_t blk = rest % nblk, t = rest / nblk;
  uint32_t w[20];
#pragma unroll
  for (int i = 0; i < 20; ++i) w[i] = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t c = 4 * blk + j;
    const uint4 v = c < C3 ? src[(t * C3 + c) * 64 + li] : make_uint4(0, 0, 0, 0);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t code = lut[(vw[q >> 2] >> (8 * (q & 3))) & 0xFFu];
      const int pos = 10 * (16 * j + q);  // bit of this byte's first code
      w[pos >> 5] |= code << (pos & 31);
      if ((pos & 31) > 22) w[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
    }
  }
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int64_t c = 5 * blk + j;
    if (c < C2) dst[(t * C2 + c) * 64 + li] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
  }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// What one call does beyond the product itself, in workspace order: the
// rotated x', the PTQ1_0 weights rewritten to PQ2_0, the fp32 K-split
// partials.
struct GemmPlan {
  bool rewrite;  // PTQ1_0 weights rewritten, k_gemm_pq2 runs
  int splits;    // K ranges (gridDim.z); from 2 on, k_gemm_sum adds the partials
  uint64_t rot_bytes, rewrite_bytes, part_bytes;
};

constexpr int kMaxSplits = 32;

// K ranges for a product of `wgs` output blocks over T 128-wide K steps.
//  * Output blocks that do not fill the resident workgroup slots (two per
//    CU; short prompts): S ranges with S * wgs within the slots, S chosen to
//    minimise T / S steps of about 3.2 us plus the fp32 partials (S M N
//    floats written and read once more, at about 5 TB/s, and the adding
//    launch).  A 64-token gate/up product runs 7 ranges, k/v 32.
//  * Otherwise two ranges when the blocks fill the slots much less evenly
//    than twice as many would (the last, partly empty round of workgroups,
//    e.g. 640 blocks on 512 slots for 4096 tokens x 5120 rows, costs nearly
//    as much as a full one) by at least 15 %, which the extra pass over the
//    partials must repay.
// `steps` counts the kernel's own K steps (128-wide; 80-wide chunks for
// k_gemm_ptq1, which takes at most two ranges).
int gemm_splits(const bgg_weights_desc* d, int64_t mc, int64_t steps, bool any_split) {
  const double wgs = (double)((d->N + kBN - 1) / kBN) * (double)((mc + kBM - 1) / kBM);
  const double slots = (double)(2 * bgg::device_cus());
  if (any_split && wgs < slots) {
    const double mn = (double)mc * (double)d->N;
    int best = 1;
    double best_t = (double)steps * 3.2e-6;
    for (int S = 2; S <= kMaxSplits && S <= steps && S * wgs <= slots; ++S) {
      const double t = (double)steps / S * 3.2e-6 + (double)S * mn * 8.0 / 5e12 + 3e-6;
      if (t < best_t) best = S, best_t = t;
    }
    return best;
  }
  if (steps < 4) return 1;
  const double waves = wgs / slots;
  const double eff1 = waves / std::ceil(waves), eff2 = 2 * waves / std::ceil(2 * waves);
  return eff2 > 1.15 * eff1 ? 2 : 1;
}

// The plan for M tokens given `avail` workspace bytes (UINT64_MAX: as much
// as the plan wants).  Each optional part runs only if the workspace also
// holds it; the rotation is not optional (the caller checks it).
GemmPlan gemm_plan(const bgg_weights_desc* d, int64_t M, bool rotate, uint64_t avail) {
  GemmPlan p{};
  p.splits = 1;
  p.rot_bytes = rotate ? bgg::align256((uint64_t)M * d->K * 2) : 0;
  uint64_t used = p.rot_bytes;
  // PTQ1_0: the rewrite to PQ2_0 costs one pass over 3.6 bits per weight
  // (5-11 us for the projection shapes), less than what the PQ2_0 kernel
  // saves at any token count
  if (d->format == BGG_FMT_PTQ1_0) {
    const uint64_t b = bgg::align256((uint64_t)d->row_tiles * kTileRows * (uint64_t)d->K / 4);
    if (avail >= used && avail - used >= b) {
      p.rewrite = true;
      p.rewrite_bytes = b;
      used += b;
    }
  }
  const bool pq2 = d->format == BGG_FMT_PQ2_0 || p.rewrite;
  // fp32 partials of one launch (at most 65535 token blocks)
  const int64_t mc = M < int64_t(65535) * kBM ? M : int64_t(65535) * kBM;
  const int S = gemm_splits(d, mc, pq2 ? d->K / (2 * kBK) : d->chunks, pq2);
  if (S > 1) {
    const uint64_t b = (uint64_t)S * mc * d->N * 4;
    if (avail >= used && avail - used >= b) {
      p.splits = S;
      p.part_bytes = b;
    }
  }
  return p;
}

}  // namespace

extern "C" {

size_t bgg_gemm_workspace_size(const bgg_weights_desc* d, int64_t M) {
  if (bgg::check_desc(d) != BGG_OK || M < 1) return 0;
  const GemmPlan p = gemm_plan(d, M, true, UINT64_MAX);
  return (size_t)(p.rot_bytes + p.rewrite_bytes + p.part_bytes);
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
  const bool rotate = (flags & BGG_ROTATE_INPUT) != 0;
  const GemmPlan p = gemm_plan(d, M, rotate, workspace ? (uint64_t)workspace_bytes : 0);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const void* xr = x_dev;
  if (rotate) {
    if (!workspace || workspace_bytes < p.rot_bytes)
      return fail(BGG_ERR_BUFFER, "bgg_ternary_gemm: rotation needs a 16-byte aligned workspace "
                                  "of %llu bytes", (unsigned long long)p.rot_bytes);
    if ((st = bgg_hadamard_rotate(x_dev, workspace, M, d->K, stream))) return st;
    xr = workspace;
  }
  const uint8_t* wts = (const uint8_t*)packed_dev;
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(wts + d->scale_offset);
  const bool pq2 = d->format == BGG_FMT_PQ2_0 || p.rewrite;
  const int64_t C = pq2 ? d->K / kBK : d->chunks;  // chunks per row of the kernel's layout
  if (p.rewrite) {
    uint8_t* dst = ws + p.rot_bytes;
    const int64_t nblk = ceil_div(C, 5);
    const int64_t total = d->row_tiles * nblk * kTileRows;
    hipLaunchKernelGGL(k_ptq1_to_pq2, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, s,
                       (const uint4*)packed_dev, (uint4*)dst, d->chunks, C, nblk, total);
    wts = dst;
  }
  float* P = p.splits > 1 ? reinterpret_cast<float*>(ws + p.rot_bytes + p.rewrite_bytes) : nullptr;
  const int64_t kmid = (C / 2) & ~int64_t(1);  // k_gemm_ptq1's two ranges (k_gemm_pq2: unused)
  // token blocks go on grid.y, which holds at most 65535 blocks: longer
  // prompts run as several launches over consecutive token ranges
  const int64_t max_m = int64_t(65535) * kBM;
  for (int64_t m0 = 0; m0 < M; m0 += max_m) {
    const int64_t mc = M - m0 < max_m ? M - m0 : max_m;
    const dim3 grid((unsigned)((d->N + kBN - 1) / kBN), (unsigned)((mc + kBM - 1) / kBM),
                    (unsigned)p.splits);
    uint16_t* y = (uint16_t*)y_dev + m0 * d->N;
    hipLaunchKernelGGL(pq2 ? k_gemm_pq2 : k_gemm_ptq1, grid, dim3(256), 0, s,
                       (const uint16_t*)xr + m0 * d->K, wts, scales, mc, d->N, d->K, C, d->groups,
                       d->row_tiles, kmid, P, y);
    if (P) {
      const int64_t mn = mc * d->N;
      hipLaunchKernelGGL(k_gemm_sum, dim3((unsigned)ceil_div(ceil_div(mn, 4), 256)), dim3(256), 0,
                         s, (const float*)P, p.splits, mn, y);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BGG_ERR_HIP, "bgg_ternary_gemm: %s", hipGetErrorString(e));
  return BGG_OK;
}

}  // extern "C"
