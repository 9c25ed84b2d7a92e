// Prompt-time product (PQ2_0) for gfx950: Y[M][N] = X'[M][K] . (S*T)[N][K]^T.
//
// allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), packing paragraph: PQ2_0
// is the packing that wins prompt processing; method paragraph: trits with
// one FP16 scale per 128 weights.  This is the one dense contraction of the
// path, so it runs on the matrix cores: trit tiles are decoded to fp16 s*t
// (exact: the value is +-s or 0) straight into LDS and multiplied with fp16
// x' tiles by v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//
// Tiling: a 256-thread workgroup computes a 128 (tokens) x 128 (weight rows)
// block of Y, four waves of 64 x 64 (2 x 2 MFMA tiles of 32 x 32), stepping
// K by 64 (one 16-byte packed chunk per weight row, half a scale group) with
// double-buffered LDS: global loads of step k+1 are in flight while the
// matrix cores work on step k.
//
// K order inside LDS: within every 16 consecutive k the elements are stored
// as k = 0,8,1,9,...,7,15.  Decoding a 2-bit code word yields exactly these
// pairs ((w >> 2j) & 0x00030003 holds codes j and j+8), and the activation
// tile is permuted the same way while it is copied to LDS, so the two MFMA
// operands always agree on k.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "bgg_internal.h"

using bgg::fail;

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // halves per LDS row (+16 bytes against bank conflicts)
constexpr int kTileRows = BGG_ROW_TILE;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// (x_{2j}, x_{2j+1}) words of 16 activations -> (x_j, x_{j+8}) words.
__device__ __forceinline__ void permute16(const uint32_t in[8], uint32_t out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    out[j] = perm(in[4 + j / 2], in[j / 2], (j & 1) ? 0x07060302u : 0x05040100u);
}

// 16 PQ2_0 codes (one word) and an fp16 scale -> 8 words of fp16 pairs
// (s*t_j, s*t_{j+8}).  0x6400 | c is the fp16 1024 + c; subtracting 1025
// gives t = c - 1 exactly, and t * s is exact.
__device__ __forceinline__ void decode16(uint32_t w, __half2 s2, uint32_t out[8]) {
  const __half2 bias = __halves2half2(__ushort_as_half(0xE401), __ushort_as_half(0xE401));  // -1025
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t p = ((w >> (2 * j)) & 0x00030003u) | 0x64006400u;
    __half2 h = *reinterpret_cast<__half2*>(&p);
    h = __hmul2(__hadd2(h, bias), s2);
    out[j] = *reinterpret_cast<uint32_t*>(&h);
  }
}

__global__ void __launch_bounds__(256)
    k_gemm_pq2(const uint16_t* __restrict__ X, const uint8_t* __restrict__ packed,
               uint64_t scale_offset, int64_t M, int64_t N, int64_t K, int64_t C, int64_t G,
               int64_t rows_pad, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kLdsStride];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

  // loader roles: A: row tid/2, 16-blocks 2*(tid%2) and 2*(tid%2)+1;
  //               B: weight row tid/2, code words 2*(tid%2) and 2*(tid%2)+1
  const int lr = tid >> 1, lh = tid & 1;
  const int64_t am = m0 + lr;
  const bool a_ok = am < M;
  const uint16_t* a_src = X + am * K + lh * 32;
  const int64_t bn = n0 + lr;
  const bool b_ok = bn < rows_pad;
  const uint2* b_src = reinterpret_cast<const uint2*>(packed) +
                       ((bn / kTileRows) * C * kTileRows + (bn % kTileRows)) * 2 + lh;
  const uint16_t* s_src = reinterpret_cast<const uint16_t*>(packed + scale_offset) +
                          (bn / kTileRows) * G * kTileRows + (bn % kTileRows);

  uint4 ra[4];
  uint2 rb;
  uint16_t rs;
  auto gload = [&](int64_t ks) {
    const int64_t k0 = ks * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = a_ok ? *reinterpret_cast<const uint4*>(a_src + k0 + i * 8) : make_uint4(0, 0, 0, 0);
    rb = b_ok ? b_src[ks * kTileRows * 2] : make_uint2(0x55555555u, 0x55555555u);
    rs = b_ok ? s_src[(k0 / 128) * kTileRows] : 0;
  };
  auto lstore = [&](int buf) {
    uint32_t in[8], out[8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint4 u0 = ra[2 * blk], u1 = ra[2 * blk + 1];
      in[0] = u0.x, in[1] = u0.y, in[2] = u0.z, in[3] = u0.w;
      in[4] = u1.x, in[5] = u1.y, in[6] = u1.z, in[7] = u1.w;
      permute16(in, out);
      uint4* dst = reinterpret_cast<uint4*>(&As[buf][lr * kLdsStride + lh * 32 + blk * 16]);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
    const __half sh = __ushort_as_half(rs);
    const __half2 s2 = __halves2half2(sh, sh);
    const uint32_t cw[2] = {rb.x, rb.y};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      decode16(cw[blk], s2, out);
      uint4* dst = reinterpret_cast<uint4*>(&Bs[buf][lr * kLdsStride + lh * 32 + blk * 16]);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t steps = K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int li = lane & 31, lk = (lane >> 5) * 8;
  for (int64_t ks = 0; ks < steps; ++ks) {
    const int cur = (int)(ks & 1);
    if (ks + 1 < steps) gload(ks + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      f16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const f16x8*>(&As[cur][(wm * 64 + t * 32 + li) * kLdsStride + kk * 16 + lk]);
        b[t] = *reinterpret_cast<const f16x8*>(&Bs[cur][(wn * 64 + t * 32 + li) * kLdsStride + kk * 16 + lk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < steps) lstore(cur ^ 1);
    __syncthreads();
  }

  // D layout of a 32x32 tile: lane l holds column l%32, rows
  // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + li;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (m < M && n < N) Y[m * N + n] = __half_as_ushort(__float2half_rn(acc[i][j][r]));
      }
    }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

size_t bgg_gemm_workspace_size(const bgg_weights_desc* d, int64_t M) {
  if (bgg::check_desc(d) != BGG_OK || M < 1) return 0;
  return (size_t)(((uint64_t)M * d->K * 2 + 255) & ~uint64_t(255));
}

bgg_status bgg_ternary_gemm(const bgg_weights_desc* d, const void* packed_dev, const void* x_dev,
                            void* y_dev, int64_t M, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bgg_status st = bgg::check_desc(d);
  if (st) return st;
  if (d->format != BGG_FMT_PQ2_0)
    return fail(BGG_ERR_FORMAT, "bgg_ternary_gemm: only PQ2_0 weights have a prompt-time kernel");
  if (!packed_dev || !x_dev || !y_dev) return fail(BGG_ERR_NULL, "bgg_ternary_gemm: NULL buffer");
  if (M < 1 || M > (int64_t(1) << 31))
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemm: M must be >= 1 (got %lld)", (long long)M);
  if (flags & ~(uint32_t)BGG_ROTATE_INPUT)
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemm: unknown flags 0x%x", flags);
  if (!aligned16(packed_dev) || !aligned16(x_dev) || ((uintptr_t)y_dev & 1))
    return fail(BGG_ERR_BUFFER, "bgg_ternary_gemm: misaligned buffer");
  hipStream_t s = (hipStream_t)stream;
  const void* xr = x_dev;
  if (flags & BGG_ROTATE_INPUT) {
    const size_t need = bgg_gemm_workspace_size(d, M);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
      return fail(BGG_ERR_BUFFER, "bgg_ternary_gemm: rotation needs a 16-byte aligned workspace "
                                  "of %zu bytes", need);
    if ((st = bgg_hadamard_rotate(x_dev, workspace, M, d->K, stream))) return st;
    xr = workspace;
  }
  const dim3 grid((unsigned)((d->N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL(k_gemm_pq2, grid, dim3(256), 0, s, (const uint16_t*)xr,
                     (const uint8_t*)packed_dev, d->scale_offset, M, d->N, d->K, d->chunks,
                     d->groups, d->row_tiles * (int64_t)kTileRows, (uint16_t*)y_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BGG_ERR_HIP, "bgg_ternary_gemm: %s", hipGetErrorString(e));
  return BGG_OK;
}

}  // extern "C"
