// Decode-time GEMV y[M][N] = x'[M][K] . (S*T)[N][K]^T on the gfx950 matrix
// cores, for 1 <= M <= 4 tokens (PQ2_0) or 1 <= M <= 2 (PTQ1_0): one launch
// per call, which also applies the block-128 Walsh-Hadamard transform to x.
//
// What is computed: allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), method
// paragraph (trits, one FP16 scale per 128 weights, block-Hadamard-rotated
// storage), runtime paragraph (the activations get the matching transform at
// run time) and packing paragraph (PQ2_0: one trit per 2-bit slot; PTQ1_0:
// five trits per byte);
// 10100.com/article/156675786 ("Bonsai 2，把27B压进6个G"), section 它怎么做到的.
//
// Work split (one MI355X: 256 CUs, 64-lane waves):
//   * one token (k_mxv1_pq2): a workgroup of 8 waves takes one or two 64-row
//     tiles and a K range of up to 40 groups, split over its waves; each wave
//     encodes the activations of its own groups in the middle of issuing
//     its weight loads, and the waves meet only for the final fixed-order
//     reduction in LDS;
//   * two to four tokens (k_mxv_pq2): wave w owns one 64-row tile and all 8
//     waves work on the same K slice, so the slice's activations are
//     transformed and encoded once per 512 rows and shared through LDS;
//   * PTQ1_0 (k_mxv_ptq1, one or two tokens): the same split with one
//     period of K per workgroup; the bytes become fp4 operands through an
//     LDS table (described with the kernel);
//   * every wave issues all of its weight loads before it waits for
//     anything (the x loads of its encode share go first, so that encoding
//     waits for x only);
//   * slices of one row range are added in fixed-point row words
//     (bgg_rowsum.h: deterministic, independent of the order of arrival).
//
// Arithmetic (exact up to one rounding per group and the final sum):
//   * x' = H128 x / sqrt(128) in fp32; per 128-block an exponent e with
//     max |x'| < 2^e and q = rint(x' 2^(14-e)), |q| <= 2^14, split into three
//     balanced base-32 digits q = 1024 d0 + 32 d1 + d2, d in [-16, 16], each
//     an exact e4m3 value;
//   * one v_mfma_scale_f32_16x16x128_f8f6f4 per 16 weight rows and group:
//     A (fp8, 16 rows) = four row quads, each quad (d0, d1, d2, 0) of one
//     token (rows whose outputs are dropped may hold anything: the
//     one-token kernel repeats digit row 0 there), with A's E8M0 block
//     scale 2^(e-14+10-5k) on digit k; B (fp4, 16
//     columns) = the codes c = t + 1 of 16 weight rows as nibbles (value
//     c/2, B scale 2);
//   * output lane (quad G, row j) adds its quad's three digit rows: every
//     partial is a multiple of 2^(e-14) below 2^23 of them, so the sum is
//     exact; it subtracts 2^(e-14) sum q (c - 1 = t); the group's fp16 scale
//     multiplies it into an fp32 accumulator (one rounding per group);
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp4 B operand of v_mfma_scale_f32_16x16x128_f8f6f4: for fp4 elements the
// instruction reads only the first four of the eight operand registers (32
// nibbles per lane), so the other four are left undefined instead of being
// filled with zeros before every operation.
__device__ __forceinline__ i32x8 fp4_b(int r0, int r1, int r2, int r3) {
  const i32x4 v = {r0, r1, r2, r3};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

// A constant in one VGPR for the whole kernel: the block-scale operands of
// the matrix operations are VGPRs, and a literal there would be moved into
// a register again before every operation.
__device__ __forceinline__ int vgpr_const(int v) {
  int r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

constexpr int kWaves = 8;       // waves per workgroup, one 64-row tile each
constexpr int kBlocks = 4;      // 16-row blocks per tile
constexpr int kPqGsMax = 8;     // PQ2_0: groups per slice (compile-time bound)

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
  int TW;         // PTQ1_0: row tiles per workgroup (at most its waves)
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

// The matrix-core instructions read their operands from all 64 lanes, also
// from lanes whose results the kernel then drops; `pin` makes a result an
// input of an empty (convergent) asm statement in uniform control flow, so
// the compiler cannot move the instructions that produce it into a branch
// that switches some lanes off (those lanes would then feed the matrix
// operation stale operand registers).
__device__ __forceinline__ void pin(float v) { asm volatile("" : : "v"(v)); }

// ---------------------------------------------------------------------------
// Activation encoding: one 128-block of one token per 16 lanes (lane l16
// holding positions 8 l16 .. 8 l16 + 7): four blocks per wave at once, all
// lane moves in DPP.
// ---------------------------------------------------------------------------
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

// Four integer-valued |d| <= 16 (exact e4m3 values) as e4m3 bytes.
__device__ __forceinline__ uint32_t e4m3_word(float a, float b, float c, float d) {
  // v_cvt_pk_fp8_f32 (OCP e4m3 on gfx950; the digits are exact e4m3 values)
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// v of lane l ^ m across the whole wave (m = 1 .. 32): DPP within 16-lane
// rows, a swizzle within 32 lanes (bit-mask mode: and 31, xor 16), a
// permute across the halves.
template <int m>
__device__ __forceinline__ float xor64_f(float v, int lane) {
  if constexpr (m <= 8) return xor16_f<m>(v);
  else if constexpr (m == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  else return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v)));
}
template <int m>
__device__ __forceinline__ void fwht64_stage(float (&v)[2], int lane) {
  const float sgn = (lane & m) ? -1.0f : 1.0f;
  const float p0 = xor64_f<m>(v[0], lane), p1 = xor64_f<m>(v[1], lane);
  v[0] = fmaf(sgn, v[0], p0);  // low lane: v + p; high lane: p - v
  v[1] = fmaf(sgn, v[1], p1);
}
template <int m>
__device__ __forceinline__ float max64_step(float a, int lane) { return fmaxf(a, xor64_f<m>(a, lane)); }
template <int m>
__device__ __forceinline__ float sum64_step(float a, int lane) { return a + xor64_f<m>(a, lane); }

// The same encoding as encode_block16 with one 128-block per wave, lane l
// holding positions 2 l and 2 l + 1 (raw: their two fp16 values).  The
// butterflies run over the strides in the same order (1 within the lane,
// then 2 .. 64 across lanes), so the codes are the same bits.
struct BlockCode64 {
  float d[3][2];
  float corr;
  int e;
};
__device__ __forceinline__ BlockCode64 encode_block64(uint32_t raw, int rotate, int lane) {
  float v[2] = {h2f((uint16_t)(raw & 0xFFFF)), h2f((uint16_t)(raw >> 16))};
  if (rotate) {
    const float a = v[0] + v[1], b = v[0] - v[1];
    v[0] = a;
    v[1] = b;
    fwht64_stage<1>(v, lane);
    fwht64_stage<2>(v, lane);
    fwht64_stage<4>(v, lane);
    fwht64_stage<8>(v, lane);
    fwht64_stage<16>(v, lane);
    fwht64_stage<32>(v, lane);
  }
  const float norm = rotate ? kHadamardNorm : 1.0f;
  const float a0 = fabsf(v[0]), a1 = fabsf(v[1]);
  float amax = fmaxf(a0 < INFINITY ? a0 : INFINITY, a1 < INFINITY ? a1 : INFINITY);  // NaN counts as inf
  amax = max64_step<1>(amax, lane);
  amax = max64_step<2>(amax, lane);
  amax = max64_step<4>(amax, lane);
  amax = max64_step<8>(amax, lane);
  amax = max64_step<16>(amax, lane);
  amax = max64_step<32>(amax, lane);
  amax *= norm;  // max |x'| (inf for a non-finite block)
  BlockCode64 r;
  const bool nf = !(amax < INFINITY);
  const bool ok = !nf && amax > 0.0f;
  int e = 0;
  if (ok) frexpf(amax, &e);  // amax = f 2^e, f in [0.5, 1): |x'| < 2^e
  const float up = ok ? ldexpf(norm, 14 - e) : 0.0f;
  float qs = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float q = rintf(v[j] * up);          // |q| <= 2^14 (0 for a non-finite block)
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
  r.corr = nf ? __builtin_nanf("") : qs * ldexpf(1.0f, r.e - 14);
  return r;
}

// A-operand placement (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4): lane
// (row i, group kg) holds K 16 kg .. 16 kg + 15 in bytes 0-15 and 64 + 16 kg
// .. 64 + 16 kg + 15 in bytes 16-31; lane index i + 16 kg, 32 bytes each.
__device__ __forceinline__ int a_lane_of_k(int k) { return ((k & 63) >> 4) * 16; }  // + row
__device__ __forceinline__ int a_byte_of_k(int k) { return ((k >> 6) << 4) + (k & 15); }

// B-operand (fp4) of PQ2_0: lane (col, kg) holds K 32 kg .. 32 kg + 31 of
// column col; the kernel feeds it (w0 & m, (w0 >> 2) & m, w1 & m, (w1 >> 2) & m)
// of the lane's two code words, so logical K 32 kg + 8 r + n carries group
// position 32 kg + 16 (r >> 1) + 2 n + (r & 1).  So position 8 l16 + j of
// the 16-lane encoding goes to logical K
// pq2_run_k0(l16, j & 1) + (j >> 1): two runs of four consecutive K (even and
// odd j), each one 32-bit word of one A lane.
__device__ __forceinline__ int pq2_run_k0(int l16, int h) {
  return 32 * (l16 >> 2) + 16 * ((l16 >> 1) & 1) + 8 * h + 4 * (l16 & 1);
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
  __shared__ __attribute__((aligned(16))) uint16_t sS[kWaves][GSMAX * kTile];  // each wave's scales

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

  // 2. scales: the slice's ng blocks of 64 fp16 scales of the tile lie one
  //    after the other (ng x 128 bytes), one 16-byte load per lane (lanes
  //    past the end re-read the first piece); then the first half of the
  //    code loads: lane (col, kg) loads the whole 16-byte chunk 2 g + kg / 2
  //    of row 16 (2 p + kg % 2) + col for block pair p (blocks 2 p, 2 p + 1),
  //    and lanes kg = 0, 1 (2, 3) later swap halves, so that each holds its
  //    8 bytes of both blocks; a group past the slice re-reads its last
  constexpr int kHalf = (GSMAX + 1) / 2;
  uint4 w[GSMAX][kBlocks / 2];
  const uint4 sraw =
      reinterpret_cast<const uint4*>(a.packed + a.scale_offset)[(tile * a.G + g0) * 8 + (lane < 8 * ng ? lane : 0)];
  const uint4* wsrc = reinterpret_cast<const uint4*>(a.packed) +
                      (tile * a.C + 2 * g0 + (kg >> 1)) * kTile + 16 * (kg & 1) + col;
#pragma unroll
  for (int g = 0; g < kHalf; ++g) {
    const int gl = g < ng ? g : ng - 1;
#pragma unroll
    for (int p = 0; p < kBlocks / 2; ++p) w[g][p] = ld_stream(wsrc + (int64_t)gl * (2 * kTile) + p * 32);
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
    for (int p = 0; p < kBlocks / 2; ++p) w[g][p] = ld_stream(wsrc + (int64_t)gl * (2 * kTile) + p * 32);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 5. the scales into LDS, where lane (col, kg) reads those of rows 16 b + col
  if (lane < GSMAX * 8) reinterpret_cast<uint4*>(sS[wave])[lane] = sraw;
  __syncthreads();

  // 6. one MFMA per group and row block, the four of a group issued together
  float acc[kBlocks] = {0.0f, 0.0f, 0.0f, 0.0f};
  const int bsc = vgpr_const(128);  // B scale 2: codes c/2 -> c
#pragma unroll
  for (int g = 0; g < GSMAX; ++g) {
    if (g < ng) {
      const uint4* ap = reinterpret_cast<const uint4*>(sA[g] + lane * 32);
      const uint4 a0 = ap[0], a1 = ap[1];
      const i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                       (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const int sa = sSc[g][lane];
      // digit row 2 of the lane's token starts at -2^(e-14) sum q (an exact
      // integer multiple of 2^(e-14), as every partial sum is)
      const f32x4 cz = {0.0f, 0.0f, -sCorr[g][kg], 0.0f};
      // block 2 p: bytes 0-7 of the chunk on lanes kg = 0, 2, bytes 8-15 on
      // kg = 1, 3; block 2 p + 1 likewise (v_permlane16_swap: odd 16-lane
      // rows of the first operand with even rows of the second)
      uint32_t cw[kBlocks][2];
#pragma unroll
      for (int p = 0; p < kBlocks / 2; ++p) {
        const auto s0 = __builtin_amdgcn_permlane16_swap(w[g][p].x, w[g][p].z, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(w[g][p].y, w[g][p].w, false, false);
        cw[2 * p][0] = s0[0];
        cw[2 * p][1] = s1[0];
        cw[2 * p + 1][0] = s0[1];
        cw[2 * p + 1][1] = s1[1];
      }
      f32x4 D[kBlocks];
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        const uint32_t lo = cw[b][0], hi = cw[b][1];
        const i32x8 B = fp4_b((int)(lo & 0x33333333u), (int)((lo >> 2) & 0x33333333u),
                               (int)(hi & 0x33333333u), (int)((hi >> 2) & 0x33333333u));
        D[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, cz, 0, 4, 0, sa, 0, bsc);
      }
#pragma unroll
      for (int b = 0; b < kBlocks; ++b)
        acc[b] = fmaf(h2f(sS[wave][g * kTile + 16 * b + col]), (D[b][0] + D[b][1]) + D[b][2], acc[b]);
    }
  }

  // 7. lane (token kg, rows 16 b + col)
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) pin(acc[b]);
  if (live && kg < a.M) store_rows(a, kg, ltile, tile, col, acc);
}

// ---------------------------------------------------------------------------
// PQ2_0, one token: k_mxv1_pq2.  A workgroup takes TPW 64-row tiles and a
// K range of GW groups; its 8 waves split that range (GPW groups each) and
// cover all TPW tiles, so no wave shares activations with another: wave w
// encodes its own groups (four per pass, 16 lanes each; only A rows 0-2,
// the three digits, feed kept outputs, so its LDS keeps just those) in the middle
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
  __shared__ __attribute__((aligned(16))) uint16_t sS[kWaves][TPW][GPW * kTile];  // the wave's scales

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
  // 2. scales: per tile the wave's ngl groups of 64 fp16 scales lie one
  //    after the other (ngl x 128 bytes), one 16-byte load per lane (lanes
  //    past the end re-read the first piece); then the first half of the codes
  static_assert(TPW == 1 || TPW == 2, "one or two tiles");
  const uint4* sbase = reinterpret_cast<const uint4*>(a.packed + a.scale_offset) + (lane < 8 * ngl ? lane : 0);
  const uint4 sraw0 = sbase[(tiles[0] * a.G + g0) * 8];
  const uint4 sraw1 = TPW == 2 ? sbase[(tiles[TPW - 1] * a.G + g0) * 8] : sraw0;
  // codes: lane (col, kg) loads the whole 16-byte chunk 2 g + (kg >> 1) of
  // row 16 (2 p + (kg & 1)) + col for block pair p (blocks 2 p, 2 p + 1),
  // and lanes kg = 0, 1 (2, 3) later swap halves, so that each holds its 8
  // bytes of both blocks (one load instruction per two blocks)
  uint4 w[TPW][kBlocks / 2][GPW];
  constexpr int kHalf = (GPW + 1) / 2;
#pragma unroll
  for (int g = 0; g < kHalf; ++g)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint4* wsrc = reinterpret_cast<const uint4*>(a.packed) +
                          (tiles[t] * a.C + 2 * g0 + (kg >> 1)) * kTile + 16 * (kg & 1) + col;
#pragma unroll
      for (int p = 0; p < kBlocks / 2; ++p)
        w[t][p][g] = ld_stream(wsrc + (int64_t)(g < ngl ? g : ngl - 1) * (2 * kTile) + p * 32);
    }
  __builtin_amdgcn_sched_barrier(0);

  // the scales into LDS, where each output lane reads its rows' scales:
  // with one tile after the encoding (which need not wait for them), with
  // two before it (measured faster; the two tiles' weight registers leave
  // none to keep the scales through the encoding)
  auto scales_to_lds = [&]() {
    if (lane < GPW * 8) {
      reinterpret_cast<uint4*>(sS[wave][0])[lane] = sraw0;
      if (TPW == 2) reinterpret_cast<uint4*>(sS[wave][TPW - 1])[lane] = sraw1;
    }
  };
  if (TPW == 2) scales_to_lds();
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
  if (TPW == 1) scales_to_lds();
  wave_lds_sync();
  // 4. MFMAs: A lanes of rows 0-2 read their digits.
  //    The second half of the codes is issued in the first iterations, one
  //    group per iteration ahead of that iteration's matrix operations: a
  //    wave that queues loads waits until the CU has room for them, and the
  //    first groups' operations need not wait with it.
  float acc[TPW][kBlocks];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[t][b] = 0.0f;
  const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const int arow3 = (lane & 15) < 3 ? (lane & 15) : 0;
  const int bsc = vgpr_const(128);  // B scale 2: codes c/2 -> c
#pragma unroll
  for (int g = 0; g < GPW; ++g) {
    if (kHalf + g < GPW) {
      const int gh = kHalf + g;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint4* wsrc = reinterpret_cast<const uint4*>(a.packed) +
                            (tiles[t] * a.C + 2 * g0 + (kg >> 1)) * kTile + 16 * (kg & 1) + col;
#pragma unroll
        for (int p = 0; p < kBlocks / 2; ++p)
          w[t][p][gh] = ld_stream(wsrc + (int64_t)(gh < ngl ? gh : ngl - 1) * (2 * kTile) + p * 32);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g < ng) {
      // (A rows 3-15 feed only output rows that are dropped: their lanes
      // read digit row 0 again, with no branch and no zero fill)
      const uint4* ap = reinterpret_cast<const uint4*>(sA[wave][g] + arow3 * 128 + kg * 32);
      const uint4 a0 = ap[0], a1 = ap[1];
      const int sa = sSc[wave][g][arow3];
      const i32x8 A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                       (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const float corr = sCorr[wave][g];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        // block 2 p: bytes 0-7 of the chunk on lanes kg = 0, 2, bytes 8-15 on
        // kg = 1, 3; block 2 p + 1 likewise: the odd lane rows' first halves
        // trade places with the even rows' second halves
        // (v_permlane16_swap: odd 16-lane rows of the first operand with even
        // rows of the second)
        uint32_t cw[kBlocks][2];
#pragma unroll
        for (int p = 0; p < kBlocks / 2; ++p) {
          const auto s0 = __builtin_amdgcn_permlane16_swap(w[t][p][g].x, w[t][p][g].z, false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(w[t][p][g].y, w[t][p][g].w, false, false);
          cw[2 * p][0] = s0[0];
          cw[2 * p][1] = s1[0];
          cw[2 * p + 1][0] = s0[1];
          cw[2 * p + 1][1] = s1[1];
        }
        f32x4 D[kBlocks];
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
          const uint32_t lo = cw[b][0], hi = cw[b][1];
          const i32x8 B = fp4_b((int)(lo & 0x33333333u), (int)((lo >> 2) & 0x33333333u),
                               (int)(hi & 0x33333333u), (int)((hi >> 2) & 0x33333333u));
          D[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, 0, sa, 0, bsc);
        }
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
          const float s = h2f(sS[wave][t][g * kTile + 16 * b + col]);
          acc[t][b] = fmaf(s, (D[b][0] + D[b][1]) + (D[b][2] - corr), acc[t][b]);
        }
      }
    }
  }

  // 5. the waves' partial rows, added in wave order
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) pin(acc[t][b]);
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
// PTQ1_0, one or two tokens: k_mxv_ptq1<NW, MT>.  A workgroup of NW waves
// takes TW <= NW 64-row tiles (one per wave; the waves past them only help
// with the table and the encoding) and one period of K (640 trits = 5
// groups = 128 row bytes = 8 chunks).  After issuing its loads every wave
// writes its share of the byte table, and the lanes of the first waves
// encode the MT tokens' activations straight into matrix-core operands in
// LDS; one barrier, then the waves multiply.  The table words (B) serve
// every token: a token adds four matrix operations per step and two LDS
// reads, not table lookups.  (Three and more tokens take the two-step
// kernels, whose cost hardly depends on the token count: here the encoding,
// the matrix phase and the row stores of a workgroup all grow with it, and
// from two tokens on a CU holds only one workgroup, for its registers.)
//
// Weights (B, fp4): lane (col, kg) loads chunk 4 h + kg of row 16 b + col
// for each half h of the period (one 16-byte load); dword u of it feeds
// matrix operation u of (h, b): B lane (col, kg), dword r, nibble n is trit
// n of byte 4 u + r of that chunk, looked up in an LDS table of e2m1
// nibbles (t = +-1 -> +-1.0, t = 0 and nibbles 5-7 -> 0; B scale 1).  So K
// 32 kg + 8 r + n of operation (h, u) is trit 80 (4 h + kg) + 20 u + 5 r + n
// of the period.
//
// Activations (A, fp8), per token: lane (row i, kgA) bytes 0-15 are K
// 16 kgA .. +15, i.e. the ten trits of piece j = 32 h + 8 (kgA >> 1) + 2 u +
// (kgA & 1) of the period (trits 10 j .. 10 j + 4 in bytes 0-4, 10 j + 5 ..
// 10 j + 9 in bytes 8-12, the rest zero), bytes 16-31 those of piece j + 16.
// A half of a period spans three groups, 2 h .. 2 h + 2: row 4 s + d (s, d
// < 3) carries digit d of the trits of group 2 h + s and zero elsewhere,
// with that group's E8M0 scale 2^(e - 14 + 10 - 5 d).  The four operations
// u of (h, b) chain their accumulators; output lane (col, s < 3) then holds
// in its rows 4 s .. 4 s + 2 the digit sums of group 2 h + s for weight row
// 16 b + col, which add up exactly (multiples of 2^(e-14) below 2^21 of
// them); the group's fp16 scale multiplies the sum into an fp32 accumulator
// (group 2 of a period, cut by the half boundary, once per half).
//
// LDS: the e2m1 table, 256 rows of 256 bytes (bytes 0-127 of row v hold 32
// copies of entry v), and operand areas of 81 "hole rows" of 128 bytes per
// token in the free upper halves of the table rows: token 0 in rows 0-80,
// token 1 in rows 96-176.  In a token's area:
//   * A operands: unit U = 4 h + u in rows 10 U .. 10 U + 8: row
//     q = 3 d + s holds digit plane d of slot s, the half hf of lane group
//     kgA in the 16 bytes at (32 kgA + 16 hf + 16 q) mod 128 -- rotated by
//     row, so that the lanes of one A column read different banks; row 9
//     stays zero and serves the lanes of the unused rows (s = 3 or d = 3),
//     rotated by 2 (rows 0-7 of A) or 1 (rows 8-15) for the same reason;
//   * row 80: the groups' exponents e (5 ints) and NaN terms (5 floats).
// ---------------------------------------------------------------------------
constexpr int kPtqMetaRow = 80;
constexpr int kPtqMaxTokens = 2;

// LDS byte address of row `row` of token m's operand area.
__device__ __forceinline__ uint32_t tok_addr(int m, int row) {
  return (uint32_t)(96 * m + row) * kLutRowBytes + 128u;
}

template <int NW, int MT>
__global__ void __launch_bounds__(64 * NW) k_mxv_ptq1(MxvArgs a) {
  static_assert(NW >= 2 && NW <= 16, "2 to 16 waves");
  static_assert(MT >= 1 && MT <= kPtqMaxTokens, "one or two tokens");
  constexpr int kEnc = kPeriodGroups * MT;             // blocks to encode
  // encoding: one block per wave ("wide") where the waves take every block
  // in one pass, else one block per 16-lane quarter (fewer, longer passes)
  constexpr bool kWide = kEnc <= NW;
  constexpr int kPasses = kWide ? (kEnc + NW - 1) / NW : (kEnc + 4 * NW - 1) / (4 * NW);
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * kLutRowBytes / 4];
  char* const lds = reinterpret_cast<char*>(lut);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const int64_t rr = blockIdx.x % a.RR, sl = blockIdx.x / a.RR;  // row range, period
  // waves from a.TW on take no tile: they build their share of the table
  // and encode, then leave (the test is uniform over the wave).  Their
  // loads stay (a branch around them would make the compiler wait for every
  // load at its end) but read wave 0's tile, one piece per instruction
  const bool active = wave < a.TW;
  const int64_t lt = rr * a.TW + (active ? wave : 0);
  const int64_t tile = a.tile0 + (lt < a.NTl ? lt : a.NTl - 1);

  // 1. x of the blocks this thread encodes.  Wide form: pass p, block
  //    gb = NW p + wave (token gb / 5, group gb % 5 of the period), two values
  //    per lane; quarter form: block gb = 4 NW p + 4 wave + kg, eight values
  //    per lane.  Every wave loads (the rest re-read token 0's group 0), so
  //    that the load counts are uniform.
  uint32_t xw[kWide ? kPasses : 1];
  uint4 xq[kWide ? 1 : kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int gb = kWide ? NW * p + wave : 4 * NW * p + 4 * wave + kg;
    const int m = gb / kPeriodGroups;
    const int64_t egg = sl * kPeriodGroups + gb % kPeriodGroups;
    const bool xval = gb < kEnc && egg < a.G;
    const uint16_t* xs = a.x + (xval ? m * a.K + egg * kGroup : 0);
    if constexpr (kWide)
      xw[p] = *reinterpret_cast<const uint32_t*>(xs + 2 * lane);
    else
      xq[p] = *reinterpret_cast<const uint4*>(xs + 8 * col);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. scales: lane (col, q) of half h, block b takes row 16 b + col, group
  //    2 h + q of the period (q < 3); then the weights: chunk 4 h + kg of
  //    row 16 b + col (chunks past the row re-read the last one)
  const uint16_t* sbase = reinterpret_cast<const uint16_t*>(a.packed + a.scale_offset) + tile * a.G * kTile;
  uint32_t sraw[2][kBlocks];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t g = sl * kPeriodGroups + 2 * h + (kg < 3 ? kg : 2);
    const uint16_t* srow = sbase + (g < a.G ? g : a.G - 1) * kTile;
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) sraw[h][b] = ld_scale_pair(srow + 16 * b, col);
  }
  // (the second half's weights are issued after the barrier, between the
  // first half's matrix operations: a wave that queues loads waits until the
  // CU has room for them, and its table and encoding work should not wait)
  uint4 w[2][kBlocks];
  const uint4* wsrc[2];
  // (a helper wave's lanes all read one 16-byte piece per instruction)
  const int wkg = active ? kg : 0, wcol = active ? col : 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int64_t c = sl * kPeriodChunks + 4 * h + wkg;
    c = c < a.C ? c : a.C - 1;
    wsrc[h] = reinterpret_cast<const uint4*>(a.packed) + (tile * a.C + c) * kTile + wcol;
  }
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) w[0][b] = ld_stream(wsrc[0] + 16 * b);
  __builtin_amdgcn_sched_barrier(0);

  // 3. the table: job j = t, t + 64 NW, ... < 512 writes copies 16 (j & 1) ..
  //    16 (j & 1) + 15 of entry j / 2 (the 16-byte pieces of a row in an
  //    order rotated by the entry, so that the lanes of one store, 256 bytes
  //    apart, spread over the banks)
  for (int j = threadIdx.x; j < 512; j += 64 * NW) {
    const int e = j >> 1;
    const uint32_t v = ptq1_lut_entry<kLutE2m1>((uint32_t)e);
#pragma unroll
    for (int q = 0; q < kLutCopies32 / 8; ++q)
      reinterpret_cast<uint4*>(lut)[e * (kLutRowBytes / 16) + (j & 1) * (kLutCopies32 / 8) +
                                    ((q + e) & (kLutCopies32 / 8 - 1))] = make_uint4(v, v, v, v);
  }
  // the zero row of every unit of every token
  for (int t = threadIdx.x; t < 64 * MT; t += 64 * NW)
    *reinterpret_cast<uint4*>(lds + tok_addr(t / 64, 10 * ((t / 8) % 8) + 9) + 16 * (t % 8)) =
        make_uint4(0, 0, 0, 0);
  // 4. encode: the lanes of block (m, eg) clear the rows of its slots (slot
  //    eg of half 0 for eg <= 2, slot eg - 2 of half 1 for eg >= 2: 4 units x
  //    3 planes each, 96 pieces of 16 bytes per half), then write its
  //    digits: trit P = 128 eg + V l + j of the period (lane l of the
  //    block's L lanes, V = 128 / L values each) goes to half h = P / 320,
  //    piece jp = (P - 320 h) / 10, byte pr = (P - 320 h) % 10 of it (bytes
  //    0-4 and 8-12)
  constexpr int L = kWide ? 64 : 16, V = kGroup / L;
  const int bl = kWide ? lane : col;  // lane within the block
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int gb = kWide ? NW * p + wave : 4 * NW * p + 4 * wave + kg;
    if (gb >= kEnc) continue;
    const int m = gb / kPeriodGroups, eg = gb % kPeriodGroups;
    const bool xval = sl * kPeriodGroups + eg < a.G;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = eg - 2 * h;
      if (s < 0 || s > 2) continue;
#pragma unroll
      for (int k = 0; k < (96 + L - 1) / L; ++k) {
        const int i = bl + L * k, row = i / 8, u = row / 3, d = row % 3;
        if (i < 96)
          *reinterpret_cast<uint4*>(lds + tok_addr(m, 10 * (4 * h + u) + 3 * d + s) + 16 * (i % 8)) =
              make_uint4(0, 0, 0, 0);
      }
    }
    uint32_t wd[3][V / 4 > 0 ? V / 4 : 1];
    int ce;
    float ccorr;
    if constexpr (kWide) {
      const BlockCode64 c = encode_block64(xval ? xw[p] : 0u, a.rotate, lane);
#pragma unroll
      for (int d = 0; d < 3; ++d) wd[d][0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c.d[d][0], c.d[d][1], 0, false);
      ce = c.e;
      ccorr = c.corr;
    } else {
      const BlockCode16 c = encode_block16(xval ? xq[p] : make_uint4(0, 0, 0, 0), a.rotate, col);
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        wd[d][0] = e4m3_word(c.d[d][0], c.d[d][1], c.d[d][2], c.d[d][3]);
        wd[d][1] = e4m3_word(c.d[d][4], c.d[d][5], c.d[d][6], c.d[d][7]);
      }
      ce = c.e;
      ccorr = c.corr;
    }
    wave_lds_sync();  // (the clears land before the digits)
    const int P0 = kGroup * eg + V * bl;
    const int h = P0 / 320, s = eg - 2 * h, Q0 = P0 - 320 * h;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int Q = Q0 + j, jp = Q / 10, pr = Q % 10;
      const int hf = jp >> 4, r = jp & 15, u = (r >> 1) & 3, kgA = 2 * (r >> 3) + (r & 1);
      const int at = 32 * kgA + 16 * hf + pr + (pr >= 5 ? 3 : 0);
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        const int q = 3 * d + s;
        lds[tok_addr(m, 10 * (4 * h + u) + q) + ((at + 16 * q) & 127)] = (char)(wd[d][j >> 2] >> (8 * (j & 3)));
      }
    }
    if (bl == 0) {
      int* meta = reinterpret_cast<int*>(lds + tok_addr(m, kPtqMetaRow));
      meta[eg] = ce;
      reinterpret_cast<float*>(meta)[kPeriodGroups + eg] = ccorr != ccorr ? ccorr : 0.0f;
    }
  }
  __syncthreads();
  if (!active) return;

  // 5. per half: four chained operations per row block and token, then lane
  //    (col, s < 3) scales its group's sums.  The operands of step k + 1 (the
  //    tokens' A columns and the table words) are fetched before the
  //    operations of step k are issued, so that LDS latency overlaps the
  //    matrix cores.
  float acc[MT][kBlocks];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[m][b] = 0.0f;
  {
    const int bsc = vgpr_const(127);  // B scale 1
    const int arow = lane & 15, as = arow >> 2, ad = arow & 3;
    const bool aon = as < 3 && ad < 3;
    const int aq = aon ? 3 * ad + as : 9, rot = aon ? aq : (arow < 8 ? 2 : 1);
    const uint32_t aoff0 = (32 * kg + 16 * rot) & 127, aoff1 = (32 * kg + 16 + 16 * rot) & 127;
    const uint32_t loff = lut_lane_off(lane);
    int sa[MT][2];
    float fl[MT][2];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int* meta = reinterpret_cast<const int*>(lds + tok_addr(m, kPtqMetaRow));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sa[m][h] = aon ? 123 + meta[2 * h + as] - 5 * ad : 127;
        fl[m][h] = kg < 3 ? reinterpret_cast<const float*>(meta)[kPeriodGroups + 2 * h + kg] : 0.0f;
      }
    }
    i32x8 A[2][MT];
    i32x4 B[2][kBlocks];
    auto fetch = [&](int k, i32x8 (&Ak)[MT], i32x4 (&Bk)[kBlocks]) {
      const int h = k >> 2, u = k & 3;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const char* ar = lds + tok_addr(m, aq) + 10 * k * kLutRowBytes;
        const uint4 a0 = *reinterpret_cast<const uint4*>(ar + aoff0);
        const uint4 a1 = *reinterpret_cast<const uint4*>(ar + aoff1);
        Ak[m] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      }
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        const uint32_t wd = u == 0 ? w[h][b].x : u == 1 ? w[h][b].y : u == 2 ? w[h][b].z : w[h][b].w;
        Bk[b] = i32x4{*reinterpret_cast<const int*>(lds + lut_addr<0>(wd, loff)),
                      *reinterpret_cast<const int*>(lds + lut_addr<1>(wd, loff)),
                      *reinterpret_cast<const int*>(lds + lut_addr<2>(wd, loff)),
                      *reinterpret_cast<const int*>(lds + lut_addr<3>(wd, loff))};
      }
    };
    f32x4 D[MT][kBlocks];
    fetch(0, A[0], B[0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int cur = k & 1, h = k >> 2, u = k & 3;
      if (k < 4) w[1][k] = ld_stream(wsrc[1] + 16 * k);
      if (k + 1 < 8 && k != 3) fetch(k + 1, A[cur ^ 1], B[cur ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        const i32x8 Bv = fp4_b(B[cur][b][0], B[cur][b][1], B[cur][b][2], B[cur][b][3]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f32x4 C = u == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : D[m][b];
          D[m][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[cur][m], Bv, C, 0, 4, 0, sa[m][h], 0, bsc);
        }
      }
      if (k == 3) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(4, A[0], B[0]);  // (waits for the second half's weights)
      }
      if (u == 3) {
        const bool gon = kg < 3 && sl * kPeriodGroups + 2 * h + kg < a.G;
#pragma unroll
        for (int b = 0; b < kBlocks; ++b) {
          const float s = gon ? scale_half(sraw[h][b], col) : 0.0f;
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[m][b] = fmaf(s, (D[m][b][0] + D[m][b][1]) + (D[m][b][2] + fl[m][h]), acc[m][b]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // 6. the wave's rows: its four lane groups' partials (slots) added, so
  //    that every lane holds the sums of its column's four row blocks; lane
  //    (col, kg) stores row 16 kg + col (all of a lane's row-word arrivals
  //    issued before any is checked)
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      pin(acc[m][b]);
      acc[m][b] += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, __float_as_int(acc[m][b])));
      acc[m][b] += __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(acc[m][b])));
    }
  const int64_t lrow = lt * kTile + 16 * kg + col;
  const int64_t row = a.tile0 * kTile + lrow;
  if (lt >= a.NTl || row >= a.N) return;
  float v[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) v[m] = kg == 0 ? acc[m][0] : kg == 1 ? acc[m][1] : kg == 2 ? acc[m][2] : acc[m][3];
  if (a.P == 1) {
#pragma unroll
    for (int m = 0; m < MT; ++m) a.y[(int64_t)m * a.N + row] = f2h(v[m]);
    return;
  }
  uint64_t term[MT], old[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) term[m] = partial_term(a.rw, m, lrow, v[m]);
#pragma unroll
  for (int m = 0; m < MT; ++m) old[m] = arrive(a.rw, m, lrow, term[m]);
#pragma unroll
  for (int m = 0; m < MT; ++m) finish_row(a.rw, m, lrow, a.P, old[m], term[m], a.y + (int64_t)m * a.N + row);
}

// ---------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------
constexpr int64_t kTargetWgs = 160;  // workgroups per launch the slicing aims at

// One-token kernel: 64-row tiles per workgroup.
int mxv1_tpw(const bgg_weights_desc* d) { return d->row_tiles >= 2 * 128 ? 2 : 1; }

// One-token kernel: how many K ranges (each a row-word arrival; a range
// costs the returning atomics at the end, about 2-3 us of tail) for `units`
// groups of K of which a workgroup takes at most `umax`:
// as few as keep a range within umax and give at least min_wgs workgroups
// (160 for one-tile workgroups, measured: q 6.2 -> 5.8 us, k/v 4.5 -> 4.1;
// 96 for two-tile ones, whose projections would otherwise split K: gate/up
// 9.0 -> 12.1 us with 160).
struct K1Split {
  int64_t P, GW;
};
K1Split k1_split(int64_t units, int64_t umax, int64_t RR, int64_t min_wgs) {
  int64_t P = std::max(ceil_div(units, umax), ceil_div(min_wgs, RR));
  // (at most one range per group, and no more ranges than the row words
  // count; ceil(units / umax) itself stays within that for every K the
  // kernel takes)
  P = std::min({P, units, (int64_t)kMaxSlices});
  const int64_t GW = ceil_div(units, P);
  return K1Split{ceil_div(units, GW), GW};
}

// PTQ1_0 kernel: row tiles per workgroup (tw), the fewest that leave at
// most one workgroup per CU, and waves per workgroup (nw), one per tile but
// at least kPtqMinWaves (5 for one token: the five blocks of a period are
// encoded in one pass; 3 for two), the waves past the tiles only helping
// with the table and the encoding.  A CU that holds two workgroups takes
// them in about 1.3x the time of one and so sets the launch's end
// (measured: gate/up 17408x5120 at one token 9.4 us with 8 tiles = 272
// workgroups on 256 CUs, 8.0 us with 9 tiles = 248; at two tokens 16.3 and
// 11.5 us); small projections spread over more CUs with fewer tiles each.
constexpr int kPtqMaxWaves[3] = {0, 16, 12};  // (two tokens: registers for 3 waves per SIMD)
constexpr int kPtqMinWaves[3] = {0, 5, 3};
struct PtqPlan {
  int nw, tw;
};
PtqPlan ptq1_plan(const bgg_weights_desc* d, int64_t M) {
  const int64_t P = ceil_div(d->groups, kPeriodGroups), cus = device_cus();
  int tw = kPtqMaxWaves[M];
  for (int t = 1; t < kPtqMaxWaves[M]; ++t)
    if (ceil_div(d->row_tiles, t) * P <= cus) {
      tw = t;
      break;
    }
  return PtqPlan{std::max(tw, kPtqMinWaves[M]), tw};
}

template <int NW>
void launch_ptq1(int M, dim3 grid, hipStream_t st, const MxvArgs& a) {
  const dim3 block(64 * NW);
  if (M == 1) {
    if constexpr (NW >= kPtqMinWaves[1]) hipLaunchKernelGGL((k_mxv_ptq1<NW, 1>), grid, block, 0, st, a);
  } else {
    if constexpr (NW <= kPtqMaxWaves[2]) hipLaunchKernelGGL((k_mxv_ptq1<NW, 2>), grid, block, 0, st, a);
  }
}
template <int NW>
void launch_ptq1_nw(int nw, int M, dim3 grid, hipStream_t st, const MxvArgs& a) {
  if constexpr (NW <= 16) {
    if (nw == NW)
      launch_ptq1<NW>(M, grid, st, a);
    else
      launch_ptq1_nw<NW + 1>(nw, M, grid, st, a);
  }
}

}  // namespace

namespace bgg {

bool mxv_supported(const bgg_weights_desc* d, int64_t M) {
  // (K short enough for the row words' arrival count at the widest ranges)
  if (d->format == BGG_FMT_PTQ1_0)
    return M >= 1 && M <= kPtqMaxTokens && ceil_div(d->groups, kPeriodGroups) <= kMaxSlices;
  return d->format == BGG_FMT_PQ2_0 && M >= 1 && M <= 4 && d->groups <= (M == 1 ? 24 : kPqGsMax) * kMaxSlices;
}

uint64_t mxv_workspace_bytes() { return 2 * kRowWordBytes; }

int mxv_kernel_name(const bgg_weights_desc* d, int64_t M, char* out, size_t cap) {
  if (d->format == BGG_FMT_PTQ1_0) return snprintf(out, cap, "k_mxv_ptq1<%d, %d>", ptq1_plan(d, M).nw, (int)M);
  if (M == 1) return snprintf(out, cap, "k_mxv1_pq2<5, %d>", mxv1_tpw(d));
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
  if (d->format == BGG_FMT_PTQ1_0) {
    // workgroups of tw tiles x one period, nw waves
    const PtqPlan pl = ptq1_plan(d, M);
    const int nw = pl.nw;
    if (nw < kPtqMinWaves[M] || nw > kPtqMaxWaves[M] || pl.tw < 1 || pl.tw > nw)  // (instantiated counts)
      return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: no kernel for %d waves", nw);
    a.TW = pl.tw;
    const int64_t RRall = ceil_div(NT, a.TW);
    a.P = (int)ceil_div(a.G, kPeriodGroups);
    if (a.P > kMaxSlices) return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: K = %lld is too long", (long long)d->K);
    a.GS = 1;
    const int64_t rr_per = a.P > 1 ? kRowWordRows / (a.TW * kTile) : RRall;
    for (int64_t r0 = 0; r0 < RRall; r0 += rr_per) {
      a.RR = std::min(rr_per, RRall - r0);
      a.tile0 = r0 * a.TW;
      a.NTl = std::min<int64_t>(a.RR * a.TW, NT - a.tile0);
      const dim3 grid((unsigned)(a.RR * a.P));
      launch_ptq1_nw<kPtqMinWaves[2]>(nw, (int)M, grid, st, a);
    }
    return hip_check("bgg_ternary_gemv");
  }
  if (M == 1) {
    // one token: workgroups of TPW tiles x one K range of up to 8 x 5
    // groups (8 x 3 beyond K = 5120, where three groups per wave stream
    // better), split over the waves
    const int tpw = mxv1_tpw(d);
    const int64_t RR = ceil_div(NT, tpw);
    constexpr int kGpw = 5;
    const K1Split sp = k1_split(a.G, a.G <= kWaves * kGpw ? kWaves * kGpw : 24, RR, tpw == 2 ? 96 : 160);
    if (sp.P > kMaxSlices) return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: K = %lld is too long", (long long)d->K);
    a.GS = (int)sp.GW;
    a.P = (int)sp.P;
    const int64_t rr_per = a.P > 1 ? kRowWordRows / (tpw * kTile) : RR;
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
  // two to four tokens (PQ2_0): workgroups of kWaves tiles x GS groups
  const int64_t RRall = ceil_div(NT, kWaves);
  int GS = kPqGsMax;
  while (GS > 1 && RRall * ceil_div(a.G, GS) < kTargetWgs) GS = GS > 2 ? GS / 2 : 1;
  while (ceil_div(a.G, GS) > kMaxSlices) ++GS;
  if (GS > kPqGsMax) return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: K = %lld is too long", (long long)d->K);
  a.GS = GS;
  a.P = (int)ceil_div(a.G, GS);
  // one launch per kRowWordRows rows when K is split (row words per slot)
  const int64_t rr_per = a.P > 1 ? kRowWordRows / (kWaves * kTile) : RRall;
  for (int64_t r0 = 0; r0 < RRall; r0 += rr_per) {
    a.RR = std::min(rr_per, RRall - r0);
    a.tile0 = r0 * kWaves;
    a.NTl = std::min<int64_t>(a.RR * kWaves, NT - a.tile0);
    const dim3 grid((unsigned)(a.RR * a.P)), block(64 * kWaves);
    hipLaunchKernelGGL((k_mxv_pq2<kPqGsMax>), grid, block, 0, st, a);
  }
  return hip_check("bgg_ternary_gemv");
}

}  // namespace bgg
