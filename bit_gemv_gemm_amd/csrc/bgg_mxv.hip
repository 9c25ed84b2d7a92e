// Decode-time GEMV y[M][N] = x'[M][K] . (S*T)[N][K]^T on the gfx950 matrix
// cores, for the PQ2_0 and PTQ1_0 packings and 1 <= M <= 4 tokens: one launch
// per call, which also applies the block-128 Walsh-Hadamard transform to x.
//
// What is computed: allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), method
// paragraph (trits, one FP16 scale per 128 weights, block-Hadamard-rotated
// storage), runtime paragraph (the activations get the matching transform at
// run time) and packing paragraph (PQ2_0: one trit per 2-bit slot; PTQ1_0:
// five trits per byte, whose decoding costs arithmetic);
// 10100.com/article/156675786 ("Bonsai 2，把27B压进6个G"), section 它怎么做到的.
//
// Work split (one MI355X: 256 CUs, 64-lane waves):
//   * a workgroup is 8 waves; wave w owns one 64-row tile of the packed
//     matrix (four 16-row blocks) and all 8 waves work on the same K slice
//     (GS groups for PQ2_0, PS five-group periods for PTQ1_0), so the slice's
//     activations are transformed and encoded once per 512 rows and shared
//     through LDS;
//   * every wave issues all of its weight loads before it waits for
//     anything (the x loads of its encode share go first, so that encoding
//     waits for x only);
//   * slices of one row range are added in fixed-point row words with one
//     device-scope atomic per row and token; the atomic also counts the
//     arrivals, and the workgroup that arrives last writes y and clears the
//     word (deterministic: integer addition does not depend on order).
//
// Arithmetic (exact up to one rounding per group and the final sum):
//   * x' = H128 x / sqrt(128) in fp32; per 128-block an exponent e with
//     max |x'| < 2^e and q = rint(x' 2^(14-e)), |q| <= 2^14, split into three
//     balanced base-32 digits q = 1024 d0 + 32 d1 + d2, d in [-16, 16], each
//     an exact e4m3 value;
//   * one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 weight rows and unit:
//     A (fp8, 16 rows) = four row quads, each quad (d0, d1, d2, 0) of one
//     token (PQ2_0: quad = token, unit = 128-group; PTQ1_0: quad = (token,
//     which of the two groups an 80-trit chunk touches), unit = chunk), with
//     A's E8M0 block scale 2^(e-14+10-5k) on digit k; B (fp4, 16 columns) =
//     the weights of 16 rows: PQ2_0 codes c = t + 1 as nibbles (value c/2,
//     B scale 2), PTQ1_0 trits t as e2m1 nibbles from an LDS table (value t,
//     B scale 1);
//   * output lane (quad G, row j) adds its quad's three digit rows: every
//     partial is a multiple of 2^(e-14) below 2^23 of them, so the sum is
//     exact; PQ2_0 subtracts 2^(e-14) sum q (c - 1 = t); the group's fp16
//     scale multiplies it into an fp32 accumulator (one rounding per group);
//   * a block with a non-finite x' carries NaN in that correction term, so
//     every row of its token becomes NaN, as 0 * inf and NaN do in the
//     fp64 product the method defines.
#include "bgg_device.h"
#include "bgg_rowsum.h"

#include <algorithm>
#include <cmath>

using namespace bgg;

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;       // waves per workgroup, one 64-row tile each
constexpr int kBlocks = 4;      // 16-row blocks per tile
constexpr int kPqGsMax = 8;     // PQ2_0: groups per slice (compile-time bound)
constexpr int kPtqPsMax = 1;    // PTQ1_0: periods per slice (38 loads per wave: within vmcnt)
constexpr int kChunkTrits = 80; // PTQ1_0: one 16-byte chunk of a row

struct MxvArgs {
  const uint8_t* packed;
  uint64_t scale_offset;
  int64_t C;      // 16-byte chunks per row
  int64_t G;      // 128-groups per row
  int64_t N;
  int64_t tile0;  // first 64-row tile of this launch
  int64_t NTl;    // tiles of this launch
  int64_t RR;     // row ranges (kWaves tiles each) of this launch
  int GS;         // PQ2_0: groups per slice; PTQ1_0: periods per slice
  int P;          // slices
  int M;          // tokens
  int rotate;
  const uint16_t* x;  // [M][K] fp16
  int64_t K;
  RowWords rw;
  uint16_t* y;  // [M][N] fp16
};

// The four row blocks' results of one lane (token m, rows 16 b + col of the
// tile): stored directly (one slice), else through the row words (all four
// arrivals issued before any is checked).
__device__ __forceinline__ void store_rows(const MxvArgs& a, int m, int64_t ltile, int64_t tile, int col,
                                           const float (&v)[kBlocks]) {
  if (a.P == 1) {
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      const int64_t row = tile * kTile + 16 * b + col;
      if (row < a.N) a.y[(int64_t)m * a.N + row] = f2h(v[b]);
    }
    return;
  }
  uint64_t term[kBlocks], old[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b)
    term[b] = partial_term(a.rw, m, ltile * kTile + 16 * b + col, v[b]);
#pragma unroll
  for (int b = 0; b < kBlocks; ++b)
    if (tile * kTile + 16 * b + col < a.N) old[b] = arrive(a.rw, m, ltile * kTile + 16 * b + col, term[b]);
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    const int64_t row = tile * kTile + 16 * b + col;
    if (row < a.N)
      finish_row(a.rw, m, ltile * kTile + 16 * b + col, a.P, old[b], term[b], a.y + (int64_t)m * a.N + row);
  }
}

// ---------------------------------------------------------------------------
// Activation encoding: one 128-block of one token by a whole wave, lane l
// holding positions 2 l and 2 l + 1 (so a token's block costs each lane two
// values, not eight: the transform is short and all 64 lanes work).
// ---------------------------------------------------------------------------
template <int m>
__device__ __forceinline__ float xor64_f(float v, int lane) {
  if constexpr (m < 16) {
    return xor16_f<m>(v);
  } else if constexpr (m == 16) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16
  } else {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));
  }
}
template <int m>
__device__ __forceinline__ void fwht64_stage(float& v0, float& v1, int lane) {
  const float sgn = (lane & m) ? -1.0f : 1.0f;
  const float p0 = xor64_f<m>(v0, lane), p1 = xor64_f<m>(v1, lane);
  v0 = fmaf(sgn, v0, p0);  // low lane: v + p; high lane: p - v
  v1 = fmaf(sgn, v1, p1);
}
template <int m>
__device__ __forceinline__ float max64_step(float v, int lane) { return fmaxf(v, xor64_f<m>(v, lane)); }
template <int m>
__device__ __forceinline__ float sum64_step(float v, int lane) { return v + xor64_f<m>(v, lane); }

struct BlockCode {
  float d[3][2];  // the digits of q for the lane's two positions
  float corr;     // 2^(e-14) sum q over the block; NaN if the block is non-finite
  int e;          // the block exponent (0 for an all-zero or non-finite block)
};

__device__ __forceinline__ BlockCode encode_block(uint32_t raw, int rotate, int lane) {
  float v0 = h2f((uint16_t)(raw & 0xFFFFu)), v1 = h2f((uint16_t)(raw >> 16));
  if (rotate) {
    const float a = v0 + v1, b = v0 - v1;  // stride 1, in the lane
    v0 = a;
    v1 = b;
    fwht64_stage<1>(v0, v1, lane);  // strides 2 .. 64: lane ^ 1 .. lane ^ 32
    fwht64_stage<2>(v0, v1, lane);
    fwht64_stage<4>(v0, v1, lane);
    fwht64_stage<8>(v0, v1, lane);
    fwht64_stage<16>(v0, v1, lane);
    fwht64_stage<32>(v0, v1, lane);
    v0 *= kHadamardNorm;
    v1 *= kHadamardNorm;
  }
  // non-finite flag (NaN or inf) and max |x'| over the block
  const float a0 = fabsf(v0), a1 = fabsf(v1);
  float nf = (a0 < INFINITY && a1 < INFINITY) ? 0.0f : 1.0f;
  float amax = fmaxf(a0, a1);
  nf = max64_step<1>(nf, lane);
  amax = max64_step<1>(amax, lane);
  nf = max64_step<2>(nf, lane);
  amax = max64_step<2>(amax, lane);
  nf = max64_step<4>(nf, lane);
  amax = max64_step<4>(amax, lane);
  nf = max64_step<8>(nf, lane);
  amax = max64_step<8>(amax, lane);
  nf = max64_step<16>(nf, lane);
  amax = max64_step<16>(amax, lane);
  nf = max64_step<32>(nf, lane);
  amax = max64_step<32>(amax, lane);
  BlockCode r;
  const bool ok = nf == 0.0f && amax > 0.0f;
  int e = 0;
  if (ok) frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1): |x'| < 2^e
  const float up = ok ? ldexpf(1.0f, 14 - e) : 0.0f;
  float qs = 0.0f;
  const float vv[2] = {v0, v1};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float q = rintf(vv[j] * up);          // |q| <= 2^14 (0 for a non-finite block)
    qs += q;
    const float d0 = rintf(q * 0x1p-10f);       // [-16, 16]
    const float r1 = fmaf(-1024.0f, d0, q);     // [-512, 512], exact
    const float d1 = rintf(r1 * 0x1p-5f);       // [-16, 16]
    r.d[0][j] = d0;
    r.d[1][j] = d1;
    r.d[2][j] = fmaf(-32.0f, d1, r1);           // [-16, 16], exact
  }
  qs = sum64_step<1>(qs, lane);  // integers below 2^21: exact
  qs = sum64_step<2>(qs, lane);
  qs = sum64_step<4>(qs, lane);
  qs = sum64_step<8>(qs, lane);
  qs = sum64_step<16>(qs, lane);
  qs = sum64_step<32>(qs, lane);
  r.e = ok ? e : 0;
  r.corr = nf != 0.0f ? __builtin_nanf("") : qs * ldexpf(1.0f, r.e - 14);
  return r;
}

// The same for 16 lanes of a block (lane l16 holding positions 8 l16 ..
// 8 l16 + 7): four blocks per wave at once, all lane moves in DPP.
struct BlockCode16 {
  float d[3][8];
  float corr;
  int e;
};
__device__ __forceinline__ BlockCode16 encode_block16(uint4 raw, int rotate, int l16) {
  float v[8];
  unpack8h(raw, v);
  if (rotate) fwht128_unscaled(v, l16);
  const float norm = rotate ? kHadamardNorm : 1.0f;
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = fabsf(v[j]);
    amax = fmaxf(amax, a < INFINITY ? a : INFINITY);  // NaN counts as inf: flags the block
  }
  amax = fmaxf(amax, xor16_f<1>(amax));
  amax = fmaxf(amax, xor16_f<2>(amax));
  amax = fmaxf(amax, xor16_f<4>(amax));
  amax = fmaxf(amax, xor16_f<8>(amax));
  amax *= norm;  // max |x'| (inf for a non-finite block)
  BlockCode16 r;
  const bool nf = !(amax < INFINITY);
  const bool ok = !nf && amax > 0.0f;
  int e = 0;
  if (ok) frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1): |x'| < 2^e
  const float up = ok ? ldexpf(norm, 14 - e) : 0.0f;
  float qs = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = rintf(v[j] * up);          // |q| <= 2^14 (0 for a non-finite block)
    qs += q;
    const float d0 = rintf(q * 0x1p-10f);       // [-16, 16]
    const float r1 = fmaf(-1024.0f, d0, q);     // [-512, 512], exact
    const float d1 = rintf(r1 * 0x1p-5f);       // [-16, 16]
    r.d[0][j] = d0;
    r.d[1][j] = d1;
    r.d[2][j] = fmaf(-32.0f, d1, r1);           // [-16, 16], exact
  }
  qs += xor16_f<1>(qs);  // integers below 2^21: exact
  qs += xor16_f<2>(qs);
  qs += xor16_f<4>(qs);
  qs += xor16_f<8>(qs);
  r.e = ok ? e : 0;
  r.corr = nf ? __builtin_nanf("") : qs * ldexpf(1.0f, r.e - 14);
  return r;
}

// e4m3 byte of an integer-valued |d| <= 16 (exact): from the fp32 bits,
// exponent rebiased 127 -> 7 and the top three mantissa bits.
__device__ __forceinline__ uint32_t e4m3_of(float d) {
  const uint32_t u = __float_as_uint(d);
  const uint32_t mag = ((u >> 20) & 0x7FFu) - (120u << 3);
  return d == 0.0f ? 0u : (((u >> 24) & 0x80u) | mag);
}
__device__ __forceinline__ uint32_t e4m3_word(float a, float b, float c, float d) {
  // v_cvt_pk_fp8_f32 (OCP e4m3 on gfx950; the digits are exact e4m3 values)
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// A-operand placement (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4): lane
// (row i, group kg) holds K 16 kg .. 16 kg + 15 in bytes 0-15 and 64 + 16 kg
// .. 64 + 16 kg + 15 in bytes 16-31; lane index i + 16 kg, 32 bytes each.
__device__ __forceinline__ int a_lane_of_k(int k) { return ((k & 63) >> 4) * 16; }  // + row
__device__ __forceinline__ int a_byte_of_k(int k) { return ((k >> 6) << 4) + (k & 15); }

// B-operand (fp4) of PQ2_0: lane (col, kg) holds K 32 kg .. 32 kg + 31 of
// column col; the kernel feeds it (w0 & m, (w0 >> 2) & m, w1 & m, (w1 >> 2) & m)
// of the lane's two code words, so logical K 32 kg + 8 r + n carries group
// position 32 kg + 16 (r >> 1) + 2 n + (r & 1).  Position 2 l + j of an
// encoding lane l is therefore logical K 32 (l >> 4) + 16 ((l >> 3) & 1) +
// 8 j + (l & 7).
// In the 16-lane layout, position 8 l16 + j goes to logical K
// pq2_run_k0(l16, j & 1) + (j >> 1): two runs of four consecutive K (even and
// odd j), each one 32-bit word of one A lane.
__device__ __forceinline__ int pq2_run_k0(int l16, int h) {
  return 32 * (l16 >> 2) + 16 * ((l16 >> 1) & 1) + 8 * h + 4 * (l16 & 1);
}
__device__ __forceinline__ int pq2_k_of_pos(int lane, int j) {
  return 32 * (lane >> 4) + 16 * ((lane >> 3) & 1) + 8 * j + (lane & 7);
}

// ---------------------------------------------------------------------------
// PQ2_0 kernel
// ---------------------------------------------------------------------------

// Workgroup: kWaves waves, one 64-row tile each, all on the same K slice.
// Wave w also encodes group w of the slice for every token (16 lanes per
// token, so up to four tokens in one pass): it issues the x load of that
// group, then the first half of its weight loads, encodes while those are
// in flight, and then issues the second half -- the encode overlaps the
// weight stream instead of waiting behind it (the vector memory path of a
// CU serves requests in order, and a wave cannot run past a load it is
// still trying to issue).
template <int GSMAX>
__global__ void __launch_bounds__(64 * kWaves) k_mxv_pq2(MxvArgs a) {
  static_assert(GSMAX <= kWaves, "one group per wave to encode");
  __shared__ __attribute__((aligned(16))) uint8_t sA[GSMAX][64 * 32];
  __shared__ uint8_t sSc[GSMAX][64];
  __shared__ float sCorr[GSMAX][4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int l16 = lane & 15, quarter = lane >> 4;
  const int64_t rr = blockIdx.x % a.RR, sl = blockIdx.x / a.RR;
  const int64_t g0 = sl * a.GS;
  const int ng = (int)(a.G - g0 < a.GS ? a.G - g0 : a.GS);
  const int64_t ltile = rr * kWaves + wave;  // tile within this launch
  const bool live = ltile < a.NTl;
  // (a wave past the last tile loads the last tile and drops the results:
  // every load below is unconditional, so that the compiler's wait counts
  // stay exact -- behind a branch it would wait for all of them at once)
  const int64_t tile = a.tile0 + (live ? ltile : a.NTl - 1);
  const bool enc = wave < ng;

  // 1. x of group `wave` for token `quarter`
  const bool xreal = enc && quarter < a.M;
  const uint4 xraw = *reinterpret_cast<const uint4*>(
      a.x + (int64_t)(xreal ? quarter : 0) * a.K + (g0 + (enc ? wave : 0)) * kGroup + 8 * l16);
  __builtin_amdgcn_sched_barrier(0);

  // 2. scales, then the first half of the code loads: codes of rows 16 b +
  //    col, K 32 kg .. +31 of group g -- chunk 2 g + kg / 2, half kg % 2
  //    (u32x2 units); a group past the slice re-reads its last
  constexpr int kHalf = (GSMAX + 1) / 2;
  u32x2 w[GSMAX][kBlocks];
  uint32_t sraw[GSMAX];
  const u32x2* wsrc = reinterpret_cast<const u32x2*>(a.packed) +
                      ((tile * a.C + 2 * g0 + (kg >> 1)) * kTile + col) * 2 + (kg & 1);
  {
    const uint16_t* ssrc =
        reinterpret_cast<const uint16_t*>(a.packed + a.scale_offset) + (tile * a.G + g0) * kTile + lane;
#pragma unroll
    for (int g = 0; g < GSMAX; ++g) sraw[g] = ssrc[(int64_t)(g < ng ? g : ng - 1) * kTile];
#pragma unroll
    for (int g = 0; g < kHalf; ++g) {
      const int gl = g < ng ? g : ng - 1;
#pragma unroll
      for (int b = 0; b < kBlocks; ++b)
        w[g][b] = __builtin_nontemporal_load(wsrc + (int64_t)gl * (4 * kTile) + b * 32);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. encode group `wave`: its A operand cleared, then each token's digits
  //    in rows 4 t .. 4 t + 2 (the wave's own LDS writes land in order)
  if (enc) {
    uint8_t* ab = sA[wave];
    reinterpret_cast<uint4*>(ab + lane * 32)[0] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint4*>(ab + lane * 32)[1] = make_uint4(0, 0, 0, 0);
    const BlockCode16 c = encode_block16(xraw, a.rotate, l16);
    if (xreal) {
      const int t = quarter;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k0 = pq2_run_k0(l16, h);
        uint8_t* dst = ab + (a_lane_of_k(k0) + 4 * t) * 32 + a_byte_of_k(k0);
#pragma unroll
        for (int d = 0; d < 3; ++d)
          *reinterpret_cast<uint32_t*>(dst + 32 * d) =
              e4m3_word(c.d[d][h], c.d[d][h + 2], c.d[d][h + 4], c.d[d][h + 6]);
      }
    }
    // E8M0 scale of A lane (row 4 t + d, K group lg): 2^(e_t - 14 + 10 - 5 d),
    // written by lane (token t, 4 d + lg); 2^0 for token slots past M
    {
      const int d = l16 >> 2, lg = l16 & 3;
      sSc[wave][4 * quarter + d + 16 * lg] = (uint8_t)(d < 3 && xreal ? 123 + c.e - 5 * d : 127);
    }
    if (l16 == 0) sCorr[wave][quarter] = xreal ? c.corr : 0.0f;
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. the second half of the code loads
#pragma unroll
  for (int g = kHalf; g < GSMAX; ++g) {
    const int gl = g < ng ? g : ng - 1;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      w[g][b] = __builtin_nontemporal_load(wsrc + (int64_t)gl * (4 * kTile) + b * 32);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 5. the scales of rows 16 b + col (lane l loaded row l)
  float sc[GSMAX][kBlocks];
#pragma unroll
  for (int g = 0; g < GSMAX; ++g)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      sc[g][b] = h2f((uint16_t)__builtin_amdgcn_ds_bpermute((16 * b + col) << 2, (int)sraw[g]));
  __syncthreads();

  // 6. one MFMA per group and row block, the four of a group issued together
  float acc[kBlocks] = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < GSMAX; ++g) {
    if (g < ng) {
      const uint4* ap = reinterpret_cast<const uint4*>(sA[g] + lane * 32);
      const uint4 a0 = ap[0], a1 = ap[1];
      const i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                       (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const int sa = sSc[g][lane];
      const float corr = sCorr[g][kg];
      f32x4 D[kBlocks];
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        const uint32_t lo = w[g][b].x, hi = w[g][b].y;
        const i32x8 B = {(int)(lo & 0x33333333u), (int)((lo >> 2) & 0x33333333u),
                         (int)(hi & 0x33333333u), (int)((hi >> 2) & 0x33333333u), 0, 0, 0, 0};
        D[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, 0, sa, 0, 128);
      }
#pragma unroll
      for (int b = 0; b < kBlocks; ++b)
        acc[b] = fmaf(sc[g][b], (D[b][0] + D[b][1]) + (D[b][2] - corr), acc[b]);
    }
  }

  // 7. lane (token kg, rows 16 b + col)
  if (live && kg < a.M) store_rows(a, kg, ltile, tile, col, acc);
}

// ---------------------------------------------------------------------------
// PQ2_0, one token: k_mxv1_pq2.  A workgroup takes TPW 64-row tiles and a
// K range of GW groups; its 8 waves split that range (GPW groups each) and
// cover all TPW tiles, so no wave shares activations with another: wave w
// encodes its own groups (four per pass, 16 lanes each; only A rows 0-2,
// the three digits, are non-zero, so its LDS keeps just those) in the middle
// of issuing its weight loads, and the waves meet only for the final
// fixed-order reduction in LDS.  With one K range per row range there is no
// row word at all; else the ranges are added through the row words.
// ---------------------------------------------------------------------------
template <int GPW, int TPW>
__global__ void __launch_bounds__(64 * kWaves) k_mxv1_pq2(MxvArgs a) {
  constexpr int kPasses = (GPW + 3) / 4;
  constexpr int kRows = TPW * kTile;
  // digit rows 0-2 of each group's A operand: [digit][lane group][32 bytes]
  __shared__ __attribute__((aligned(16))) uint8_t sA[kWaves][GPW][3 * 4 * 32];
  __shared__ uint8_t sSc[kWaves][GPW][4];   // E8M0 of digits 0-2 (byte 3 unused)
  __shared__ float sCorr[kWaves][GPW];
  __shared__ float red[kWaves][kRows];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int l16 = lane & 15, quarter = lane >> 4;
  const int64_t rr = blockIdx.x % a.RR, sl = blockIdx.x / a.RR;
  const int64_t gw0 = sl * a.GS;                                  // the workgroup's K range
  const int ngw = (int)(a.G - gw0 < a.GS ? a.G - gw0 : a.GS);
  const int gpw = (ngw + kWaves - 1) / kWaves;                     // groups per wave (<= GPW)
  const int gb = wave * gpw;                                       // this wave's first group
  const int ng = ngw - gb < 0 ? 0 : (ngw - gb < gpw ? ngw - gb : gpw);
  const int64_t g0 = gw0 + (ng > 0 ? gb : 0);                      // (a wave without groups re-reads)
  const int ngl = ng > 0 ? ng : 1;
  int64_t tiles[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t lt = rr * TPW + t;
    tiles[t] = a.tile0 + (lt < a.NTl ? lt : a.NTl - 1);
  }

  // 1. x of the wave's groups (pass p, quarter q: group 4 p + q)
  uint4 xraw[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int gi = 4 * p + quarter;
    xraw[p] = *reinterpret_cast<const uint4*>(a.x + (g0 + (gi < ngl ? gi : 0)) * kGroup + 8 * l16);
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. scales (lane l: row l of each tile), then the first half of the codes
  uint32_t sraw[TPW][GPW];
  u32x2 w[TPW][kBlocks][GPW];
  constexpr int kHalf = (GPW + 1) / 2;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const uint16_t* ssrc =
        reinterpret_cast<const uint16_t*>(a.packed + a.scale_offset) + (tiles[t] * a.G + g0) * kTile + lane;
#pragma unroll
    for (int g = 0; g < GPW; ++g) sraw[t][g] = ssrc[(int64_t)(g < ngl ? g : ngl - 1) * kTile];
  }
#pragma unroll
  for (int g = 0; g < kHalf; ++g)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const u32x2* wsrc = reinterpret_cast<const u32x2*>(a.packed) +
                          ((tiles[t] * a.C + 2 * g0 + (kg >> 1)) * kTile + col) * 2 + (kg & 1);
#pragma unroll
      for (int b = 0; b < kBlocks; ++b)
        w[t][b][g] = __builtin_nontemporal_load(wsrc + (int64_t)(g < ngl ? g : ngl - 1) * (4 * kTile) + b * 32);
    }
  __builtin_amdgcn_sched_barrier(0);

  // 3. encode the wave's groups: digit rows 0-2 of A
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int gi = 4 * p + quarter;
    if (4 * p < ng) {
      const BlockCode16 c = encode_block16(xraw[p], a.rotate, l16);
      if (gi < ng) {
        uint8_t* ab = sA[wave][gi];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k0 = pq2_run_k0(l16, h);
          // lane group of A = (k0 & 63) >> 4, bytes 16 (k0 >> 6) + (k0 & 15)
          uint8_t* dst = ab + ((k0 & 63) >> 4) * 32 + ((k0 >> 6) << 4) + (k0 & 15);
#pragma unroll
          for (int d = 0; d < 3; ++d)
            *reinterpret_cast<uint32_t*>(dst + 128 * d) =
                e4m3_word(c.d[d][h], c.d[d][h + 2], c.d[d][h + 4], c.d[d][h + 6]);
        }
        if (l16 < 3) sSc[wave][gi][l16] = (uint8_t)(123 + c.e - 5 * l16);
        if (l16 == 0) sCorr[wave][gi] = c.corr;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 4. the second half of the codes
#pragma unroll
  for (int g = kHalf; g < GPW; ++g)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const u32x2* wsrc = reinterpret_cast<const u32x2*>(a.packed) +
                          ((tiles[t] * a.C + 2 * g0 + (kg >> 1)) * kTile + col) * 2 + (kg & 1);
#pragma unroll
      for (int b = 0; b < kBlocks; ++b)
        w[t][b][g] = __builtin_nontemporal_load(wsrc + (int64_t)(g < ngl ? g : ngl - 1) * (4 * kTile) + b * 32);
    }
  __builtin_amdgcn_sched_barrier(0);

  // 5. MFMAs: A lanes of rows 0-2 read their digits, the rest are zero
  float acc[TPW][kBlocks];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[t][b] = 0.0f;
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const int arow = lane & 15;
#pragma unroll
  for (int g = 0; g < GPW; ++g) {
    if (g < ng) {
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
      int sa = 127;
      if (arow < 3) {
        const uint4* ap = reinterpret_cast<const uint4*>(sA[wave][g] + arow * 128 + kg * 32);
        a0 = ap[0];
        a1 = ap[1];
        sa = sSc[wave][g][arow];
      }
      const i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                       (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const float corr = sCorr[wave][g];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        f32x4 D[kBlocks];
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
          const uint32_t lo = w[t][b][g].x, hi = w[t][b][g].y;
          const i32x8 B = {(int)(lo & 0x33333333u), (int)((lo >> 2) & 0x33333333u),
                           (int)(hi & 0x33333333u), (int)((hi >> 2) & 0x33333333u), 0, 0, 0, 0};
          D[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, 0, sa, 0, 128);
        }
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
          const float s = h2f((uint16_t)__builtin_amdgcn_ds_bpermute((16 * b + col) << 2, (int)sraw[t][g]));
          acc[t][b] = fmaf(s, (D[b][0] + D[b][1]) + (D[b][2] - corr), acc[t][b]);
        }
      }
    }
  }

  // 6. the waves' partial rows, added in wave order
  if (kg == 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) red[wave][t * kTile + 16 * b + col] = acc[t][b];
  }
  __syncthreads();
  for (int r = threadIdx.x; r < kRows; r += 64 * kWaves) {
    float v = red[0][r];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) v += red[q][r];
    const int64_t lt = rr * TPW + r / kTile;
    if (lt >= a.NTl) continue;
    const int64_t lrow = lt * kTile + r % kTile;
    const int64_t row = a.tile0 * kTile + lrow;
    if (row >= a.N) continue;
    if (a.P == 1) {
      a.y[row] = f2h(v);
    } else {
      const uint64_t term = partial_term(a.rw, 0, lrow, v);
      const uint64_t old = arrive(a.rw, 0, lrow, term);
      finish_row(a.rw, 0, lrow, a.P, old, term, a.y + row);
    }
  }
}

// ---------------------------------------------------------------------------
// PTQ1_0 kernel
//
// Unit = one 16-byte chunk of a row (80 trits): lane (col, kg) of row block
// b reads bytes 4 kg .. 4 kg + 3 of the chunk (one dword; a wave instruction
// reads 16 rows x 16 bytes, contiguous) and turns each byte into one B
// register through the LDS table: the byte's five trits as e2m1 nibbles 0-4
// (-1 -> 0xA, 0 -> 0, +1 -> 0x2), nibbles 5-7 zero.  Logical K 32 kg + 8 r +
// n (n < 5) is trit 5 (4 kg + r) + n of the chunk.  A chunk touches at most
// two 128-groups (group ends fall inside bytes 25, 51, 76 and 102 of every
// 128-byte period); A holds one quad per (token, group of the chunk), M <= 2
// per MFMA set.  The table: 256 entries, 32 copies each (entry v of copy c at
// byte v 256 + 4 c; lane l reads copy l % 32, so the 32 lanes the LDS serves
// at once never share a bank, and the address is one v_perm of the packed
// word).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ptq1_t_nibbles(uint32_t b) {
  if (b >= 243) return 0u;  // no trits: reads as five zero trits
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t c = b % 3u;  // t + 1
    b /= 3u;
    r |= (c == 0 ? 0xAu : c == 2 ? 0x2u : 0u) << (4 * i);
  }
  return r;
}

template <int MT2>
__global__ void __launch_bounds__(64 * kWaves) k_mxv_ptq1(MxvArgs a) {
  constexpr int kUnits = kPeriodChunks;  // chunks per slice: one period
  constexpr int kGroups = kPeriodGroups;
  constexpr int kTok = 2 * MT2;
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * (kLutRowBytes / 4)];
  __shared__ __attribute__((aligned(16))) uint8_t sA[kUnits * MT2][64 * 32];
  __shared__ __attribute__((aligned(16))) uint8_t sSc[kUnits * MT2][64];
  __shared__ float sCorr[kUnits * MT2][4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int64_t rr = blockIdx.x % a.RR, sl = blockIdx.x / a.RR;
  const int64_t g0 = sl * kPeriodGroups, c0 = sl * kPeriodChunks;  // the slice is period sl
  const int ng = (int)(a.G - g0 < kGroups ? a.G - g0 : kGroups);
  const int nu = (int)(a.C - c0 < kUnits ? a.C - c0 : kUnits);
  const int64_t ltile = rr * kWaves + wave;
  const bool live = ltile < a.NTl;
  // (unconditional loads, as in k_mxv_pq2: a wave past the last tile reads
  // the last tile, a chunk or group past the slice the slice's last one)
  const int64_t tile = a.tile0 + (live ? ltile : a.NTl - 1);

  // 1. loads: x of the group this wave encodes (wave w < 5: group w, every
  //    token), the scales, the packed bytes
  const bool enc = wave < ng;
  const int64_t xg = g0 + (enc ? wave : 0);
  uint32_t xraw[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t)
    xraw[t] = *reinterpret_cast<const uint32_t*>(a.x + (int64_t)(t < a.M ? t : 0) * a.K + xg * kGroup + 2 * lane);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t w[kUnits][kBlocks];
  uint32_t sraw[kGroups];
  {
    const uint32_t* wsrc = reinterpret_cast<const uint32_t*>(a.packed) +
                           ((tile * a.C + c0) * kTile + col) * 4 + kg;
    const uint16_t* ssrc =
        reinterpret_cast<const uint16_t*>(a.packed + a.scale_offset) + (tile * a.G + g0) * kTile + lane;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) sraw[g] = ssrc[(int64_t)(g < ng ? g : ng - 1) * kTile];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int ul = u < nu ? u : nu - 1;
#pragma unroll
      for (int b = 0; b < kBlocks; ++b)
        w[u][b] = __builtin_nontemporal_load(wsrc + (int64_t)ul * (4 * kTile) + b * 64);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
    if (g >= ng) sraw[g] = 0u;

  // 2. the table; A / scale / NaN-term areas to zero / 2^0 / 0
  {
    const int e = threadIdx.x >> 1, half = threadIdx.x & 1;
    const uint32_t v = ptq1_t_nibbles((uint32_t)e);
    uint4* dst = reinterpret_cast<uint4*>(lut + e * (kLutRowBytes / 4) + 16 * half);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(v, v, v, v);
    uint4* az = reinterpret_cast<uint4*>(&sA[0][0]);
    for (int i = threadIdx.x; i < kUnits * MT2 * 64 * 2; i += 64 * kWaves) az[i] = make_uint4(0, 0, 0, 0);
    uint32_t* sz = reinterpret_cast<uint32_t*>(&sSc[0][0]);
    for (int i = threadIdx.x; i < kUnits * MT2 * 16; i += 64 * kWaves) sz[i] = 0x7F7F7F7Fu;
    float* cz = &sCorr[0][0];
    for (int i = threadIdx.x; i < kUnits * MT2 * 4; i += 64 * kWaves) cz[i] = 0.0f;
  }
  __syncthreads();

  // 3. encode: group `wave`'s positions go to the chunks they fall in
  if (enc) {
    const int gr = wave;
    const int ulo = (kGroup * gr) / kChunkTrits, uhi = (kGroup * gr + kGroup - 1) / kChunkTrits;
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      if (t < a.M) {
        const BlockCode c = encode_block(xraw[t], a.rotate, lane);
        const int set = t >> 1, tq = t & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int T = kGroup * gr + 2 * lane + j;
          const int u = T / kChunkTrits, tau = T % kChunkTrits;
          const int h = gr - (kChunkTrits * u) / kGroup;  // 0 or 1
          const int k = 32 * (tau / 20) + 8 * ((tau % 20) / 5) + tau % 5;
          uint8_t* dst = sA[u * MT2 + set] + (a_lane_of_k(k) + 4 * (2 * tq + h)) * 32 + a_byte_of_k(k);
#pragma unroll
          for (int d = 0; d < 3; ++d) dst[32 * d] = (uint8_t)e4m3_of(c.d[d][j]);
        }
        // scale bytes and NaN terms of the quads this group has in its chunks
        for (int u = ulo; u <= uhi; ++u) {
          const int q = 2 * tq + gr - (kChunkTrits * u) / kGroup;
          if (lane < 16) {
            const int d = lane >> 2, lg = lane & 3;
            sSc[u * MT2 + set][4 * q + d + 16 * lg] = (uint8_t)(d < 3 ? 123 + c.e - 5 * d : 127);
          }
          if (lane == 0) sCorr[u * MT2 + set][q] = c.corr != c.corr ? c.corr : 0.0f;
        }
      }
    }
  }
  __syncthreads();

  // 4. per chunk and row block: 4 table reads -> B; MT2 MFMAs
  float sc[kGroups][kBlocks];
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      sc[g][b] = h2f((uint16_t)__builtin_amdgcn_ds_bpermute((16 * b + col) << 2, (int)sraw[g]));
  float acc[MT2][kBlocks];
#pragma unroll
  for (int s = 0; s < MT2; ++s)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[s][b] = 0.0f;
  if (live) {
    const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t lane_off = lut_lane_off(lane);
    const bool hq = kg & 1;  // which group of the chunk this lane's quad holds
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      if (u < nu) {
        const int glo = (kChunkTrits * u) / kGroup;
        const int ghi = glo + 1 < kGroups ? glo + 1 : glo;
        i32x8 A[MT2];
        int sa[MT2];
        float corr[MT2];
#pragma unroll
        for (int s = 0; s < MT2; ++s) {
          const uint4* ap = reinterpret_cast<const uint4*>(sA[u * MT2 + s] + lane * 32);
          const uint4 a0 = ap[0], a1 = ap[1];
          A[s] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                       (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          sa[s] = sSc[u * MT2 + s][lane];
          corr[s] = sCorr[u * MT2 + s][kg];
        }
        i32x8 B[kBlocks];
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
          const uint32_t wd = w[u][b];
          B[b] = i32x8{(int)lut[lut_addr<0>(wd, lane_off) >> 2], (int)lut[lut_addr<1>(wd, lane_off) >> 2],
                       (int)lut[lut_addr<2>(wd, lane_off) >> 2], (int)lut[lut_addr<3>(wd, lane_off) >> 2],
                       0, 0, 0, 0};
        }
#pragma unroll
        for (int s = 0; s < MT2; ++s) {
          f32x4 D[kBlocks];
#pragma unroll
          for (int b = 0; b < kBlocks; ++b)
            D[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[s], B[b], zero, 0, 4, 0, sa[s], 0, 127);
#pragma unroll
          for (int b = 0; b < kBlocks; ++b)
            acc[s][b] = fmaf(hq ? sc[ghi][b] : sc[glo][b], (D[b][0] + D[b][1]) + (D[b][2] + corr[s]), acc[s][b]);
        }
      }
    }
  }

  // 5. a token's two group quads sit in lane groups 2 tq and 2 tq + 1 of its
  //    set: add them; lanes of even lane groups store
#pragma unroll
  for (int s = 0; s < MT2; ++s)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      acc[s][b] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(acc[s][b]), 0x401F));
  if (live && !(kg & 1)) {
#pragma unroll
    for (int s = 0; s < MT2; ++s) {
      const int t = 2 * s + (kg >> 1);
      if (t < a.M) store_rows(a, t, ltile, tile, col, acc[s]);
    }
  }
}

// ---------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------
constexpr int64_t kTargetWgs = 160;  // workgroups per launch the slicing aims at

}  // namespace

namespace bgg {

bool mxv_supported(const bgg_weights_desc* d, int64_t M) {
  return d->format == BGG_FMT_PQ2_0 && M >= 1 && M <= 4;
}

uint64_t mxv_workspace_bytes() { return 2 * kRowWordBytes; }

int mxv_kernel_name(const bgg_weights_desc* d, int64_t M, char* out, size_t cap) {
  if (M == 1) return snprintf(out, cap, "k_mxv1_pq2<5, %d>", d->row_tiles >= 2 * 128 ? 2 : 1);
  return snprintf(out, cap, "k_mxv_pq2<%d>", kPqGsMax);
}

bgg_status mxv_launch(const bgg_weights_desc* d, const void* packed, const void* x, void* y,
                      int64_t M, int rotate, void* workspace, hipStream_t st) {
  MxvArgs a{};
  a.packed = (const uint8_t*)packed;
  a.scale_offset = d->scale_offset;
  a.C = d->chunks;
  a.G = d->groups;
  a.N = d->N;
  a.M = (int)M;
  a.rotate = rotate;
  a.x = (const uint16_t*)x;
  a.K = d->K;
  a.rw = row_words_of(workspace);
  a.y = (uint16_t*)y;
  const int64_t NT = d->row_tiles;
  const bool pq2 = d->format == BGG_FMT_PQ2_0;
  if (pq2 && M == 1) {
    // one token: workgroups of TPW tiles x one K range of up to 8 x GPW groups
    constexpr int kGpw = 5;
    const int tpw = NT >= 2 * 128 ? 2 : 1;
    const int64_t RR = ceil_div(NT, tpw);
    // K ranges: each one costs the returning row-word atomics at the end
    // (about 2-3 us of tail), so as few as keep a range within 40 groups
    // (24 beyond K = 5120, where three groups per wave stream better) and
    // give at least kMinWgs workgroups
    constexpr int64_t kMinWgs = 96;
    const int64_t gmax = a.G <= kWaves * kGpw ? kWaves * kGpw : 24;
    int64_t P = std::max(ceil_div(a.G, gmax), ceil_div(kMinWgs, RR));
    P = std::min(P, a.G);
    const int64_t GW = ceil_div(a.G, P);
    P = ceil_div(a.G, GW);
    if (P > kMaxSlices) return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: K = %lld is too long", (long long)d->K);
    a.GS = (int)GW;
    a.P = (int)P;
    const int64_t rr_per = P > 1 ? kRowWordRows / (tpw * kTile) : RR;
    for (int64_t r0 = 0; r0 < RR; r0 += rr_per) {
      a.RR = std::min(rr_per, RR - r0);
      a.tile0 = r0 * tpw;
      a.NTl = std::min<int64_t>(a.RR * tpw, NT - a.tile0);
      const dim3 grid((unsigned)(a.RR * a.P)), block(64 * kWaves);
      if (tpw == 2)
        hipLaunchKernelGGL((k_mxv1_pq2<kGpw, 2>), grid, block, 0, st, a);
      else
        hipLaunchKernelGGL((k_mxv1_pq2<kGpw, 1>), grid, block, 0, st, a);
    }
    return hip_check("bgg_ternary_gemv");
  }
  const int64_t RRall = ceil_div(NT, kWaves);
  // units per row: groups (PQ2_0) or periods (PTQ1_0); slices of GS units
  const int64_t units = pq2 ? a.G : ceil_div(a.G, kPeriodGroups);
  const int gsmax = pq2 ? kPqGsMax : kPtqPsMax;
  int GS = gsmax;
  while (GS > 1 && RRall * ceil_div(units, GS) < kTargetWgs) GS = GS > 2 ? GS / 2 : 1;
  while (ceil_div(units, GS) > kMaxSlices) ++GS;
  if (GS > gsmax) return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: K = %lld is too long", (long long)d->K);
  a.GS = GS;
  a.P = (int)ceil_div(units, GS);
  // one launch per kRowWordRows rows when K is split (row words per slot)
  const int64_t rr_per = a.P > 1 ? kRowWordRows / (kWaves * kTile) : RRall;
  for (int64_t r0 = 0; r0 < RRall; r0 += rr_per) {
    a.RR = std::min(rr_per, RRall - r0);
    a.tile0 = r0 * kWaves;
    a.NTl = std::min<int64_t>(a.RR * kWaves, NT - a.tile0);
    const dim3 grid((unsigned)(a.RR * a.P)), block(64 * kWaves);
    if (pq2) {
      hipLaunchKernelGGL((k_mxv_pq2<kPqGsMax>), grid, block, 0, st, a);
    } else if (M <= 2) {
      hipLaunchKernelGGL((k_mxv_ptq1<1>), grid, block, 0, st, a);
    } else {
      hipLaunchKernelGGL((k_mxv_ptq1<2>), grid, block, 0, st, a);
    }
  }
  return hip_check("bgg_ternary_gemv");
}

}  // namespace bgg
