// Decode-time GEMV y[M][N] = x'[M][K] . (S*T)[N][K]^T for 1 <= M <= 16 on
// gfx950, for both packings.
//
// What is computed: allhereai.com/news/1346 ("27B 模型压到 5.95GB…"), method
// paragraph (trits, one FP16 scale per 128 weights, block-Hadamard-rotated
// storage), runtime paragraph (the activations get the Hadamard transform at
// run time) and packing paragraph (PQ2_0 and PTQ1_0; decoding PTQ1_0 costs
// arithmetic); 10100.com/article/156675786, section "它怎么做到的".
//
// Design (one MI355X: 256 CUs in 8 XCDs, 64-lane waves, HBM3E):
//   * activation prep (one small kernel per call): x -> x' in fp32 -> per
//     128-group a power-of-two scale 2^(e-14) with max|x'| < 2^e and
//     q = rint(x' 2^(14-e)), |q| <= 2^14, cut into four signed 4-bit digits
//     packed eight to a word in the order the trit codes will meet them;
//   * one lane per weight row: a wave reads a 64-row tile chunk by chunk
//     with coalesced 16-byte loads (1 KiB per instruction), so all lanes sit
//     at the same K and the digit words are wave-uniform: they live in
//     scalar registers and cost no LDS or vector-cache bandwidth;
//   * trits are never turned into floats: PQ2_0 codes c = t + 1 are spread
//     into 4-bit lanes with one mask (even positions) or a shift and a mask
//     (odd), PTQ1_0 bytes go through a base-3 LUT in LDS to five 4-bit codes,
//     and v_dot8_i32_i4 multiplies 8 codes by 8 digits.  Per group the exact
//     integer sum of c*q minus the sum of q is the sum of t*q; it is scaled
//     by s * 2^(e-14) and accumulated in fp32;
//   * K is split over the eight waves of a workgroup (reduced in LDS, fixed
//     order) and, when the tiles alone cannot fill the chip, over
//     workgroups, which add their partial rows as fixed-point integers with
//     one 64-bit atomic per row; the atomic also counts the arrivals, and
//     the last workgroup to arrive at a row writes it (deterministic: integer
//     addition does not depend on the order; one launch, no waiting on other
//     workgroups).
#include "bgg_device.h"
#include "bgg_rowsum.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>

using namespace bgg;

namespace {

// Digit words of one PQ2_0 chunk (64 trits): 4 code words x {even, odd}
// positions x 4 digits.
constexpr int kPqFragWords = 32;
// Digit words of one PTQ1_0 period: 4 per byte, plus 4 for the upper part
// of each of the 4 bytes that straddle a group end.
constexpr int kPtqFragWords = kPeriodBytes * 4 + 4 * 4;  // 528

// Token counts one GEMV kernel handles at once; a larger M runs in groups of
// kGemvTokens tokens (each group reads the weights again).
constexpr int kGemvTokens = 4;
__host__ __device__ inline int gemv_m_bucket(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }

// ---------------------------------------------------------------------------
// activation encoding, one wave at a time
//
// wave_encode: NG consecutive 128-blocks g0 .. g0+NG-1 of one token row,
// 16 lanes per block, four blocks per pass.  x -> x' (fp32 FWHT) -> the
// block's exponent e (max|x'| < 2^e) -> q = rint(x' 2^(14-e)), |q| <= 2^14
// -> the four signed 4-bit digits of q (q = d0 + 16 d1 + 256 d2 + 4096 d3,
// d in [-8, 7]) packed into one 16-bit value, the nibbles of
// (q + 0x8888) ^ 0x8888: adding 8 to every digit makes each nibble of the
// sum d + 8 in [0, 15] without carries, and flipping bit 3 of each nibble
// gives d's own 4-bit two's complement.  The packed values go to sd[] (this
// wave's LDS staging area) and the block's sum of q and 2^(e-14) to
// metaQ/metaF (zero for an all-zero block and for blocks past G).
// ---------------------------------------------------------------------------
// The raw fp16 values of the NG blocks, 16 bytes per lane and pass; a
// kernel that also streams weights issues these loads first, so that waiting
// for them does not wait for the weights (loads complete in issue order).
template <int NG>
struct EncodeRaw {
  uint4 v[(NG + 3) / 4];
};
// What wave_encode_finish leaves in registers: per pass, the sum of q and
// 2^(e-14) of the block that the lane worked on (all 16 lanes of a block
// hold them).
template <int NG>
struct EncodeMeta {
  int q[(NG + 3) / 4];
  float f[(NG + 3) / 4];
  // block i's values, wave-uniform (read from lane 16 (i % 4))
  __device__ __forceinline__ int q_of(int i) const {
    return __builtin_amdgcn_readlane(q[i / 4], 16 * (i % 4));
  }
  __device__ __forceinline__ float f_of(int i) const {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f[i / 4]), 16 * (i % 4)));
  }
};
template <int NG>
__device__ __forceinline__ EncodeRaw<NG> wave_encode_load(const uint16_t* __restrict__ x, int64_t G,
                                                          int64_t g0, bool token_valid, int lane) {
  const int gl = lane >> 4, lane16 = lane & 15;
  EncodeRaw<NG> r;
#pragma unroll
  for (int pass = 0; pass < (NG + 3) / 4; ++pass) {
    const int gi = pass * 4 + gl;
    const int64_t g = g0 + gi;
    r.v[pass] = gi < NG && g < G && token_valid
                    ? *reinterpret_cast<const uint4*>(x + g * kGroup + lane16 * 8)
                    : make_uint4(0, 0, 0, 0);
  }
  return r;
}
template <int NG>
__device__ __forceinline__ EncodeMeta<NG> wave_encode_finish(const EncodeRaw<NG>& r, int64_t g0,
                                                             int rotate, uint16_t* sd, int lane,
                                                             int32_t* __restrict__ metaQ,
                                                             float* __restrict__ metaF,
                                                             int64_t gpad) {
  const int gl = lane >> 4, lane16 = lane & 15;
  EncodeMeta<NG> meta;
#pragma unroll
  for (int pass = 0; pass < (NG + 3) / 4; ++pass) {
    const int gi = pass * 4 + gl;  // block within the NG
    const int64_t g = g0 + gi;
    const bool in_set = gi < NG;
    float v[8];
    unpack8h(r.v[pass], v);
    if (rotate) {
      fwht128_unscaled(v, lane16);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= kHadamardNorm;
    }
    float amax = 0.0f;
    int nf = 0;  // a non-finite x' in the block
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      amax = fmaxf(amax, fabsf(v[j]));
      nf |= !(fabsf(v[j]) <= 3.0e38f);
    }
    amax = fmaxf(amax, xor16_f<1>(amax));
    amax = fmaxf(amax, xor16_f<2>(amax));
    amax = fmaxf(amax, xor16_f<4>(amax));
    amax = fmaxf(amax, xor16_f<8>(amax));
    nf |= xor16_i<1>(nf);
    nf |= xor16_i<2>(nf);
    nf |= xor16_i<4>(nf);
    nf |= xor16_i<8>(nf);
    if (nf) amax = 0.0f;  // digits 0; the block's scale below is NaN
    int e = 0;
    frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1): |x'| < 2^e
    int qsum = 0;
    uint32_t nib[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = amax > 0.0f ? (int)rintf(ldexpf(v[j], 14 - e)) : 0;
      nib[j] = ((uint32_t)(q + 0x8888) ^ 0x8888u) & 0xFFFFu;
      qsum += q;
    }
    if (in_set)
      *reinterpret_cast<uint4*>(sd + gi * kGroup + lane16 * 8) =
          make_uint4(nib[0] | nib[1] << 16, nib[2] | nib[3] << 16, nib[4] | nib[5] << 16,
                     nib[6] | nib[7] << 16);
    qsum += xor16_i<1>(qsum);
    qsum += xor16_i<2>(qsum);
    qsum += xor16_i<4>(qsum);
    qsum += xor16_i<8>(qsum);
    // a block with a non-finite x' scales its groups by NaN: every row of
    // the token becomes NaN, as 0 * inf and NaN do in the fp64 product
    const float f = nf ? __builtin_nanf("") : amax > 0.0f ? ldexpf(1.0f, e - 14) : 0.0f;
    meta.q[pass] = qsum;
    meta.f[pass] = f;
    if (metaQ && in_set && lane16 == 0 && g < gpad) {
      metaQ[g] = qsum;
      metaF[g] = f;
    }
  }
  return meta;
}

// PQ2_0 digit words of chunks c0 .. c0+2*NG-1 (those below C) from sd:
// word (d, par, L) of chunk c holds in nibble n digit L of q at chunk
// position 16 d + 2 n + par.  Lane item (chunk, d, par) packs the four words
// L = 0..3, which sit next to each other (one 16-byte store).
template <int NG>
__device__ __forceinline__ void wave_pack_pq2(const uint16_t* sd, uint32_t* __restrict__ out,
                                              int64_t c0, int64_t C, int lane,
                                              int64_t cout0 = 0) {
#pragma unroll
  for (int it0 = 0; it0 < NG * 16; it0 += 64) {
    const int it = it0 + lane;
    const int cl = it >> 3, d = (it >> 1) & 3, par = it & 1;
    const int64_t c = c0 + cl;
    if (it < NG * 16 && c < C) {
      uint32_t wd[4] = {0, 0, 0, 0};
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint32_t v = sd[cl * 64 + 16 * d + 2 * n + par];
#pragma unroll
        for (int L = 0; L < 4; ++L) wd[L] |= ((v >> (4 * L)) & 15u) << (4 * n);
      }
      *reinterpret_cast<uint4*>(out + (c - cout0) * kPqFragWords + d * 8 + par * 4) =
          make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  }
}

// Where word i of a wave's PTQ1_0 digit words sits: contiguous (global
// workspace), or (HOLES) in the unused upper halves of the LUT's 256-byte
// rows, 32 words per row -- the one-launch kernel keeps them in LDS there.
template <bool HOLES>
__device__ __forceinline__ int ptq1_word(int i) {
  return HOLES ? (i >> 5) * (kLutRowBytes / 4) + (i & 31) : i;
}
constexpr int kPtqHoleRows = (kPtqFragWords + 31) / 32;  // LUT rows per wave

// PTQ1_0 digit words of one period (528 words per token) from sd.  Word
// (byte jb, L), jb < 128: nibble i = digit L of q at period position
// 5 jb + i, kept only if that position is in the same group as 5 jb.  Word
// (128 + s, L): the upper part of the s-th straddling byte (positions in
// the next group).  Tokens are interleaved within their GEMV token group of
// b slots (b = 1, 2 or 4): word (r, L) of slot t sits at (r b + t) 4 + L, so
// the words one wave needs for a few consecutive bytes are contiguous.
// Lane jb packs the four words of byte jb (and the upper four of a
// straddling byte), two bytes per lane.
template <bool HOLES = false>
__device__ __forceinline__ void wave_pack_ptq1(const uint16_t* sd, uint32_t* __restrict__ out,
                                               int b, int slot, int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int jb = h * 64 + lane;
    const int first_group = (5 * jb) / kGroup;
    uint32_t lo[4] = {0, 0, 0, 0}, hi[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int pos = 5 * jb + i;
      const uint32_t v = sd[pos];
      const bool upper = pos / kGroup != first_group;
#pragma unroll
      for (int L = 0; L < 4; ++L) {
        const uint32_t nib = ((v >> (4 * L)) & 15u) << (4 * i);
        if (upper)
          hi[L] |= nib;
        else
          lo[L] |= nib;
      }
    }
    *reinterpret_cast<uint4*>(out + ptq1_word<HOLES>((jb * b + slot) * 4)) =
        make_uint4(lo[0], lo[1], lo[2], lo[3]);
    if ((5 * jb + 4) / kGroup != first_group)  // bytes 25, 51, 76, 102: s = first_group
      *reinterpret_cast<uint4*>(out + ptq1_word<HOLES>(((kPeriodBytes + first_group) * b + slot) * 4)) =
          make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

// Blocks per prep unit: one PTQ1_0 period, or five PQ2_0 groups.
constexpr int kPrepGroups = 5;

// The PTQ1_0 token group of token m: its base slot, its slot count b, and
// m's slot within it.
__device__ __forceinline__ void ptq1_token_slot(int m, int Mreal, int* tg0, int* b, int* slot) {
  const int tg = m / kGemvTokens;
  *tg0 = tg * kGemvTokens;
  *slot = m % kGemvTokens;
  *b = gemv_m_bucket(Mreal - *tg0 < kGemvTokens ? Mreal - *tg0 : kGemvTokens);
}

// ---------------------------------------------------------------------------
// activation prep kernel: one wave per unit of five blocks and token slot.
// grid: (ceil(Gpad / 5), token slots); block: 64 threads.  Tokens past Mreal
// get zeros.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ void __launch_bounds__(64)
    k_gemv_prep(const uint16_t* __restrict__ x, int64_t K, int Mreal, int rotate,
                uint32_t* __restrict__ frag, int64_t frag_words_per_token,
                int32_t* __restrict__ metaQ, float* __restrict__ metaF, int64_t gpad) {
  __shared__ __attribute__((aligned(16))) uint16_t sd[kPrepGroups * kGroup];
  const int lane = threadIdx.x;
  const int m = blockIdx.y;
  const int64_t G = K / kGroup;
  const int64_t g0 = (int64_t)blockIdx.x * kPrepGroups;
  const EncodeRaw<kPrepGroups> raw = wave_encode_load<kPrepGroups>(x + (int64_t)m * K, G, g0,
                                                                   m < Mreal, lane);
  wave_encode_finish<kPrepGroups>(raw, g0, rotate, sd, lane, metaQ + (int64_t)m * gpad,
                                  metaF + (int64_t)m * gpad, gpad);
  wave_lds_sync();
  if (FMT == BGG_FMT_PQ2_0) {
    wave_pack_pq2<kPrepGroups>(sd, frag + (int64_t)m * frag_words_per_token, 2 * g0, K / 64, lane);
  } else {
    int tg0, b, slot;
    ptq1_token_slot(m, Mreal, &tg0, &b, &slot);
    if (slot >= b) return;  // a slot no GEMV token group reads
    wave_pack_ptq1(sd, frag + (int64_t)tg0 * frag_words_per_token +
                           (g0 / kPeriodGroups) * kPtqFragWords * b, b, slot, lane);
  }
}

// ---------------------------------------------------------------------------
// Workgroup end: the W waves' partial sums are added in wave order in LDS and
// wave 0 writes y when the workgroup covers all of K; otherwise (Sg
// workgroups per tile) each lane adds its row's partial sum into the row
// words at the start of the workspace (bgg_rowsum.h: fixed point, exact and
// order-independent, NaN sticky), and the workgroup that completes a row
// writes y.  A launch covers at most kSumRows rows of split tiles.
// ---------------------------------------------------------------------------
// Zeroes n16 16-byte words (bgg_gemv_workspace_reset).
__global__ void __launch_bounds__(256) k_fill_zero16(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxSumSlices = kMaxSlices;  // arrivals the row words count
constexpr int64_t kSumRows = kRowWordRows;
constexpr uint64_t kSumBytes = 2 * kRowWordBytes;  // fine and coarse words

template <int M, int W>
__device__ __forceinline__ void wg_finish(const float (&acc)[M], float (*red)[M][64], int wave,
                                          int lane, int64_t row, int64_t N, int Mreal, int Sg,
                                          int64_t local_row, unsigned long long* __restrict__ sums,
                                          uint16_t* __restrict__ y) {
#pragma unroll
  for (int m = 0; m < M; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave != 0) return;
  float s[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    s[m] = red[0][m][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) s[m] += red[w][m][lane];
  }
  if (Sg == 1) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (m < Mreal && row < N) y[(int64_t)m * N + row] = f2h(s[m]);
    return;
  }
  if (row >= N) return;
  const RowWords rw = row_words_of(sums);
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (m < Mreal) add_partial(rw, m, local_row, Sg, s[m], y + (int64_t)m * N + row);
}

// ---------------------------------------------------------------------------
// Which tile and K slice a workgroup takes.  The first nta tiles of a launch
// are cut into sga slices of W waves each.  The tiles after them -- left
// over when the tile count is just above a multiple of the CU count, e.g.
// 272 tiles on 256 CUs -- are cut into sgb slices of one wave each: those
// workgroups are light and sit beside the full ones on the CUs, instead of
// giving a few CUs twice the work of the rest.
// ---------------------------------------------------------------------------
struct WgSlot {
  int64_t tile, local;  // tile index, and its index within the launch
  int wgs, Sg;          // slice of the tile, slices of the tile
  bool one;             // a one-wave slice (only wave 0 works)
};
__device__ __forceinline__ WgSlot wg_slot(int64_t tile0, int64_t ntl, int64_t nta, int sga,
                                          int sgb, bool light_last) {
  // Light workgroups come first in launch order, so the dispatcher spreads
  // them over the CUs before the full ones: the one-wave slices, and (with
  // light_last) the last slice of every tile when it has fewer waves than
  // the others.
  // (32-bit arithmetic: block and tile counts of a launch fit, and it keeps
  // the divisions short)
  const uint32_t b = blockIdx.x, nb = (uint32_t)(ntl - nta) * (uint32_t)sgb;
  const uint32_t na = (uint32_t)nta, ga = (uint32_t)sga, gb = (uint32_t)sgb;
  WgSlot s;
  s.one = false;
  if (b < nb) {
    s.local = na + b / gb, s.wgs = (int)(b % gb), s.Sg = sgb, s.one = true;
  } else if (ga == 1) {
    s.local = b - nb, s.wgs = 0, s.Sg = 1;
  } else if (light_last) {
    const uint32_t r = b - nb;
    if (r < na)
      s.local = r, s.wgs = sga - 1;
    else
      s.local = (r - na) / (ga - 1), s.wgs = (int)((r - na) % (ga - 1));
    s.Sg = sga;
  } else {
    const uint32_t r = b - nb;
    s.local = r / ga, s.wgs = (int)(r % ga), s.Sg = sga;
  }
  s.tile = tile0 + s.local;
  return s;
}

// ---------------------------------------------------------------------------
// One-launch GEMV for one token: every wave first encodes the activation
// blocks of its own K slice (the same digit words the prep kernel writes,
// laid out the same way) into LDS and reads them from there: PQ2_0 into a
// per-wave array, PTQ1_0 into the unused upper halves of the LUT's rows.
// No global round trip: a wait for the wave's own global stores
// (s_waitcnt vmcnt(0)) would also wait for every weight load issued before
// them.  The per-block meta comes from the registers of the lanes that
// computed it.
// ---------------------------------------------------------------------------
struct FuseArgs {
  const uint16_t* x;  // the token row, K fp16 values
  int rotate;
};
// ---------------------------------------------------------------------------
// PQ2_0, the second step of bgg_gemv_prepare + bgg_gemv_run for one token
// (one launch serves one token through bgg_mxv.hip): wave = 64 rows x BPS
// groups; workgroup = W consecutive K slices.  grid: NT * Sg workgroups of
// 64*W threads.
// ---------------------------------------------------------------------------
template <int M, int BPS, int W>
__global__ void __launch_bounds__(64 * W)
    k_gemv_pq2(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t C, int64_t G,
               int64_t N, int Sg, int Mreal, const uint32_t* __restrict__ frag,
               int64_t frag_words_per_token, const int32_t* __restrict__ metaQ,
               const float* __restrict__ metaF, int64_t gpad, unsigned long long* __restrict__ sums,
               int64_t tile0, int64_t ntl, int64_t nta, int sgb, int light_last,
               uint16_t* __restrict__ y) {
  __shared__ float red[W][M][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const WgSlot ws = wg_slot(tile0, ntl, nta, Sg, sgb, light_last != 0);
  const int64_t tile = ws.tile;
  const int64_t gbeg =
      ws.one ? (wave == 0 ? (int64_t)ws.wgs * BPS : G) : ((int64_t)ws.wgs * W + wave) * BPS;

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  if (gbeg < G) {
    const uint4* tdata = reinterpret_cast<const uint4*>(packed) + (tile * C) * kTile + lane;
    const uint16_t* sdata =
        reinterpret_cast<const uint16_t*>(packed + scale_offset) + (tile * G) * kTile;
    // Every load of the slice is issued before any is used, without branches
    // (a group past G re-reads group G-1 and gets a zero weight below).
    uint4 w[2 * BPS];
    uint32_t sc[BPS];
#pragma unroll
    for (int i = 0; i < BPS; ++i) {
      const int64_t g = gbeg + i < G ? gbeg + i : G - 1;
      w[2 * i] = ld_stream(tdata + (2 * g) * kTile);
      w[2 * i + 1] = ld_stream(tdata + (2 * g + 1) * kTile);
      sc[i] = ld_scale_pair(sdata + g * kTile, lane);
    }
    // per-group activation scale and digit sum, for every token
    float gf[BPS][M];
    int gq[BPS][M];
#pragma unroll
    for (int i = 0; i < BPS; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const bool gv = gbeg + i < G;
        const int64_t g = gv ? gbeg + i : G - 1;
        gf[i][m] = gv ? metaF[(int64_t)m * gpad + g] : 0.0f;
        gq[i][m] = metaQ[(int64_t)m * gpad + g];
      }
    // keep the scheduler from sinking the loads towards their uses
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < BPS; ++i) {
      const int64_t g = gbeg + i < G ? gbeg + i : G - 1;
      const float s = scale_half(sc[i], lane);
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
        const uint32_t* xf = frag + (int64_t)m * frag_words_per_token + (2 * g) * kPqFragWords;
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
        const int p = a0 + (a1 << 4) + (a2 << 8) + (a3 << 12) - gq[i][m];
        acc[m] = fmaf(s * gf[i][m], (float)p, acc[m]);
      }
    }
  }
  wg_finish<M, W>(acc, red, wave, lane, tile * kTile + lane, N, Mreal, ws.Sg,
                  ws.local * kTile + lane, sums, y);
}

// ---------------------------------------------------------------------------
// PTQ1_0: wave = 64 rows x one part of one period (a period is 5 groups =
// 128 row bytes, cut into H parts); workgroup = W consecutive parts of one
// tile sharing a 32-copy LUT.
//
// The LUT yields the trits t themselves as signed nibbles, so a group's
// integer sum is sum t*q directly (no digit-sum correction), and a group
// cut by a part boundary is finished by each part for its own trits.
// ---------------------------------------------------------------------------
template <int M>
__device__ __forceinline__ void ptq1_close(int (&a)[M][4], float (&acc)[M], const float (&gf)[M],
                                           float s) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int p = a[m][0] + (a[m][1] << 4) + (a[m][2] << 8) + (a[m][3] << 12);
    acc[m] = fmaf(s * gf[m], (float)p, acc[m]);
#pragma unroll
    for (int L = 0; L < 4; ++L) a[m][L] = 0;
  }
}

// Bytes [B0, B0 + 128/H) of one period for all M tokens.
//
// Software pipeline over batches of BB = 4/M bytes (16 digit words): the LUT
// reads and digit-word loads of batch b+1 are issued, then batch b is
// computed, then both are awaited.  Without the explicit wait the compiler
// waits for everything at the first use of batch b, i.e. right after issuing
// batch b+1, and the scalar-load latency is paid once per batch.
template <int M, int H, int PART, bool HOLES>
__device__ __forceinline__ void ptq1_part(const uint4 (&w)[8 / H], const float (&sc)[kPeriodGroups],
                                          const float (&gf)[kPeriodGroups][M],
                                          const uint32_t* __restrict__ fp, const char* lbase, uint32_t lane_off, float (&acc)[M]) {
  constexpr int BP = kPeriodBytes / H, B0 = PART * BP, B1 = B0 + BP;
  constexpr int BB = 4 / M, NB = BP / BB;
  static_assert(BP % BB == 0, "batch size");
  int a[M][4];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int L = 0; L < 4; ++L) a[m][L] = 0;

  uint32_t lv[2][BB];           // LUT words of the batch's bytes
  uint32_t fr[2][BB][M][4];     // digit words of the batch's bytes
  uint32_t up[2][M][4];         // digit words of a straddling byte's upper trits
  auto issue = [&](int nb, int buf) {
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      const int jb = B0 + nb * BB + j;
      const uint4& ch = w[(jb - B0) >> 4];
      const uint32_t word = (jb >> 2 & 3) == 0 ? ch.x : (jb >> 2 & 3) == 1 ? ch.y
                            : (jb >> 2 & 3) == 2 ? ch.z : ch.w;
      uint32_t addr;
      switch (jb & 3) {
        case 0: addr = lut_addr<0>(word, lane_off); break;
        case 1: addr = lut_addr<1>(word, lane_off); break;
        case 2: addr = lut_addr<2>(word, lane_off); break;
        default: addr = lut_addr<3>(word, lane_off); break;
      }
      lv[buf][j] = *reinterpret_cast<const uint32_t*>(lbase + addr);
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int L = 0; L < 4; ++L) fr[buf][j][m][L] = fp[ptq1_word<HOLES>((jb * M + m) * 4 + L)];
      const int k_first = (5 * jb) / kGroup;
      if ((5 * jb + 4) / kGroup != k_first) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int L = 0; L < 4; ++L)
            up[buf][m][L] = fp[ptq1_word<HOLES>((kPeriodBytes * M + k_first * M + m) * 4 + L)];
      }
    }
  };

  issue(0, 0);
#pragma clang loop unroll(full)
  for (int nb = 0; nb < NB; ++nb) {
    const int buf = nb & 1;
    wait_lgkm0();
    __builtin_amdgcn_sched_barrier(0);
    if (nb + 1 < NB) issue(nb + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      const int jb = B0 + nb * BB + j;
      const int codes = (int)lv[buf][j];
#pragma unroll
      for (int m = 0; m < M; ++m)
#pragma unroll
        for (int L = 0; L < 4; ++L)
          a[m][L] = __builtin_amdgcn_sdot8(codes, (int)fr[buf][j][m][L], a[m][L], false);
      const int k_first = (5 * jb) / kGroup, k_last = (5 * jb + 4) / kGroup;
      if (k_last != k_first) {
        // this byte's trits cross a group end: close the lower group and
        // start the next one with the byte's upper trits
        ptq1_close<M>(a, acc, gf[k_first], sc[k_first]);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int L = 0; L < 4; ++L)
            a[m][L] = __builtin_amdgcn_sdot8(codes, (int)up[buf][m][L], a[m][L], false);
      } else if ((5 * jb + 5) % kGroup == 0) {
        ptq1_close<M>(a, acc, gf[k_first], sc[k_first]);
      }
    }
  }
  // a group still open at the part's end is finished here for this part
  constexpr int last = B1 - 1;
  if ((5 * last + 5) % kGroup != 0) {
    constexpr int k = (5 * last + 4) / kGroup;
    ptq1_close<M>(a, acc, gf[k], sc[k]);
  }
}

template <int M, int H, int W, bool FUSE>
__global__ void __launch_bounds__(64 * W)
    k_gemv_ptq1(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t C, int64_t G,
                int64_t N, int Sg, int Mreal, const uint32_t* __restrict__ frag,
                int64_t frag_words_per_token, const int32_t* __restrict__ metaQ,
                const float* __restrict__ metaF, int64_t gpad, unsigned long long* __restrict__ sums,
                int64_t tile0, int64_t ntl, int64_t nta, int sgb, int light_last, FuseArgs fa,
                uint16_t* __restrict__ y) {
  constexpr int CH = kPeriodChunks / H;  // chunks per part
  static_assert(W * 64 >= 256, "the LUT build needs 256 threads");
  static_assert(!FUSE || M == 1, "the one-launch GEMV is for one token");
  __shared__ uint32_t lut[256 * kLutRowBytes / 4];
  __shared__ uint32_t lut_seed[256];
  __shared__ float red[W][M][64];
  __shared__ __attribute__((aligned(16))) uint16_t sd_stage[FUSE ? W * kPeriodGroups * kGroup : 8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const WgSlot ws = wg_slot(tile0, ntl, nta, Sg, sgb, light_last != 0);
  const int64_t tile = ws.tile;
  const int64_t P = ceil_div(G, kPeriodGroups);
  // (period, part) of this wave
  const int64_t item = ws.one ? (wave == 0 ? ws.wgs : P * H) : (int64_t)ws.wgs * W + wave;
  const int64_t p = item / H;
  const int part = (int)(item % H);
  const bool active = p < P;
  const uint4* tdata = reinterpret_cast<const uint4*>(packed) + (tile * C) * kTile + lane;
  const uint16_t* sdata =
      reinterpret_cast<const uint16_t*>(packed + scale_offset) + (tile * G) * kTile;
  // The part's loads first -- before the LUT is built, so they are in flight
  // meanwhile -- without bounds checks: chunks past the row and groups past
  // G read the next tile's bytes or the buffer's zero slack.  Their trits
  // meet digit words and activation scales that are zero (the prep writes
  // zeros for positions past K), so they add nothing.
  uint4 w[CH];
  uint32_t sr[kPeriodGroups];
  EncodeRaw<kPeriodGroups> xraw;
  if (FUSE && active) xraw = wave_encode_load<kPeriodGroups>(fa.x, G, p * kPeriodGroups, true, lane);
  if (active) {
    // scales first: all of them are needed before the first byte
#pragma unroll
    for (int k = 0; k < kPeriodGroups; ++k)
      sr[k] = ld_scale_pair(sdata + (p * kPeriodGroups + k) * kTile, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) w[c] = ld_stream(tdata + (p * kPeriodChunks + part * CH + c) * kTile);
  }
  __builtin_amdgcn_sched_barrier(0);
  // one-launch: the wave's digit words in LDS, in the unused upper halves
  // of LUT rows wave * kPtqHoleRows ..
  constexpr bool kHoles = FUSE;
  static_assert(W * kPtqHoleRows <= 256, "the waves' digit words fit the LUT rows");
  uint32_t* holes = lut + wave * kPtqHoleRows * (kLutRowBytes / 4) + kLutRowBytes / 8;
  // the LUT is built while the loads are in flight (with FUSE: while x is)
  build_lut32(lut, lut_seed);
  __syncthreads();
  // (after the barrier: each wave goes on to its loop as soon as its own
  // encoding is done)
  EncodeMeta<kPeriodGroups> em;
  if (FUSE && active) {
    uint16_t* sdw = sd_stage + wave * (kPeriodGroups * kGroup);
    em = wave_encode_finish<kPeriodGroups>(xraw, p * kPeriodGroups, fa.rotate, sdw, lane, nullptr,
                                           nullptr, gpad);
    wave_lds_sync();
    wave_pack_ptq1<true>(sdw, holes, 1, 0, lane);
    wave_lds_sync();
  }

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  if (active) {
    const int64_t gp = p * kPeriodGroups;
    // group scales (zero past G) and the activations' group meta
    float sc[kPeriodGroups], gf[kPeriodGroups][M];
#pragma unroll
    for (int k = 0; k < kPeriodGroups; ++k) {
      sc[k] = scale_half(sr[k], lane);
      // fused: from the registers (other periods' meta share its cache lines)
#pragma unroll
      for (int m = 0; m < M; ++m) gf[k][m] = FUSE ? em.f_of(k) : metaF[(int64_t)m * gpad + gp + k];
    }
    const uint32_t* fp = kHoles ? holes : frag + p * kPtqFragWords * M;
    const uint32_t lane_off = lut_lane_off(lane);
    const char* lbase = reinterpret_cast<const char*>(lut);
    static_assert(H == 1 || H == 2, "one or two parts per period");
    if (H == 1 || part == 0)
      ptq1_part<M, H, 0, kHoles>(w, sc, gf, fp, lbase, lane_off, acc);
    else
      ptq1_part<M, H, H - 1, kHoles>(w, sc, gf, fp, lbase, lane_off, acc);
  }
  wg_finish<M, W>(acc, red, wave, lane, tile * kTile + lane, N, Mreal, ws.Sg,
                  ws.local * kTile + lane, sums, y);
}

// ---------------------------------------------------------------------------
// PQ2_0 for 2..16 tokens on the matrix cores, with the same integer
// arithmetic as the kernels above: for each 128-group the exact sum
// p = sum t q over the group's weights, then acc = fma(s 2^(e-14), p, acc)
// in fp32 (the rows of a token come out bit for bit as with one token).
//
// The VALU kernels spend dot8 work per code word per token and read the
// weights once per four tokens; here one v_mfma_scale_f32_16x16x128_f8f6f4
// per row block multiplies a 128-group of 16 weight rows with 16 token
// slots (slots past M repeat the last token; their results are dropped):
//   * B (weights) in fp4 (e2m1): a code c in {0, 1, 2} (trit c - 1) is the
//     nibble c, whose e2m1 value is c / 2; B's block scale 2 makes it c.
//     Two operations per 16 codes: the codes of even positions are w & 0x3..,
//     of odd positions (w >> 2) & 0x3...
//   * A (activations) in fp8 (e4m3): q = 1024 d0 + 32 d1 + d2 with balanced
//     base-32 digits d in [-16, 16], each an e4m3 integer; one MFMA per
//     digit with A's block scale 2^(e-14+10-5k) for digit k, accumulating
//     into the same registers.  Started from -2^(e-14) sum q (written by the
//     prep kernel), the accumulator ends at 2^(e-14) sum (c-1) q: every
//     partial sum is a multiple of 2^(e-14) below 2^24 of them, so fp32
//     holds it exactly.
// Operand layouts (gfx950): B lane (col, g) holds K 32 g .. 32 g + 31 of
// column col as nibbles, A lane (row, g) holds K 16 g + (0..15) in bytes
// 0-15 and K 64 + 16 g + (0..15) in bytes 16-31; the scale byte of lane
// (row, g) covers K block 32 g.  The prep kernel stores the A digits in the
// order the B nibbles take, for each lane 32 contiguous bytes.
//
// Work split as the VALU kernel (wg_slot, same slices): a wave takes BPS
// groups of one 64-row tile (row blocks rb: rows col + 16 rb), W waves of a
// workgroup consecutive slices; the waves' 16 x 64 results are added in
// wave order in LDS, the workgroups of a tile in the fixed-point row sums
// (one slot per token).
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// fp4 B operand of v_mfma_scale_f32_16x16x128_f8f6f4: for fp4 elements the
// instruction reads only the first four of the eight operand registers (32
// nibbles per lane), so the other four are left undefined instead of being
// filled with zeros before every operation.
__device__ __forceinline__ i32x8 fp4_b(int r0, int r1, int r2, int r3) {
  const i32x4 v = {r0, r1, r2, r3};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

constexpr int kMmaSlots = 16;      // token slots of the A operand
constexpr int kMmaRedStride = 68;  // floats per token row in LDS (64 rows + 4: no bank conflicts)
constexpr int kMxDigits = 3;       // base-32 digits of q

// Group position (0..127) of the weight that B element K (= 32 g + n, nibble n
// of lane group g) carries: dword j = n / 8 of the lane's four holds the
// codes of word j / 2 at even (j even) or odd (j odd) positions.
__host__ __device__ constexpr int mx_pos_of_k(int K) {
  return (K & ~31) + 16 * ((K >> 4) & 1) + 2 * (K & 7) + ((K >> 3) & 1);
}
// K of byte e of an A lane in lane group g.
__host__ __device__ constexpr int mx_k_of_a(int g, int e) {
  return e < 16 ? 16 * g + e : 64 + 16 * g + (e - 16);
}
// e4m3 byte of an integer |d| <= 16 (exact).
__device__ __forceinline__ uint32_t e4m3_of_int(int d) {
  const uint32_t a = (uint32_t)(d < 0 ? -d : d);
  if (a == 0) return 0;
  const int p = 31 - __builtin_clz(a);
  return (d < 0 ? 0x80u : 0u) | ((uint32_t)(p + 7) << 3) | (((a << 3) >> p) - 8);
}

// One 128-group for the lane's four row blocks: B operands from the code
// words (lo: K 32 kg .. +15, hi: K 32 kg + 16 .. +31 of the group), the
// three digit MFMAs issued digit by digit across the row blocks (four
// independent accumulators, so no MFMA waits for the one before it), then
// acc[rb] += s[rb] * (2^(e-14) p) per row block.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void mx_group(const i32x8 (&A)[kMxDigits], uint32_t sa, f32x4 c0,
                                         const u32x2 (&wv)[4], const float (&s)[4],
                                         f32x4 (&acc)[4]) {
  i32x8 B[4];
  f32x4 ag[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const uint32_t lo = wv[rb].x, hi = wv[rb].y;
    B[rb] = fp4_b((int)(lo & 0x33333333u), (int)((lo >> 2) & 0x33333333u),
                  (int)(hi & 0x33333333u), (int)((hi >> 2) & 0x33333333u));
    ag[rb] = c0;
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], B[rb], ag[rb], 0, 4, 0, (int)sa, 0, 128);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], B[rb], ag[rb], 0, 4, 1, (int)sa, 0, 128);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[2], B[rb], ag[rb], 0, 4, 2, (int)sa, 0, 128);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[rb][e] = fmaf(s[rb], ag[rb][e], acc[rb][e]);
}

// Q1_0: one 32-bit word of sign bits (K 32 kg .. +31 of the group, bit i =
// K 32 kg + i) -> four B words of fp4 nibbles in natural K order: nibble n
// of word j = bit 8 j + n, as the nibble value 0 or 1 (e2m1 0 or 0.5; B's
// block scale 4 makes it 0 or 2, so 2 b - 1 = the weight after the -sum q
// start).  Each byte's bits are moved to the nibbles' low bits in three
// shift-or-mask steps.
__device__ __forceinline__ uint32_t q1_spread8(uint32_t b) {
  uint32_t x = (b | (b << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  return (x | (x << 3)) & 0x11111111u;
}
__device__ __forceinline__ void mx_group_q1(const i32x8 (&A)[kMxDigits], uint32_t sa, f32x4 c0,
                                            const uint32_t (&wv)[4], const float (&s)[4],
                                            f32x4 (&acc)[4]) {
  i32x8 B[4];
  f32x4 ag[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const uint32_t w = wv[rb];
    B[rb] = fp4_b((int)q1_spread8(w & 0xFFu), (int)q1_spread8((w >> 8) & 0xFFu),
                  (int)q1_spread8((w >> 16) & 0xFFu), (int)q1_spread8(w >> 24));
    ag[rb] = c0;
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], B[rb], ag[rb], 0, 4, 0, (int)sa, 0, 129);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], B[rb], ag[rb], 0, 4, 1, (int)sa, 0, 129);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[2], B[rb], ag[rb], 0, 4, 2, (int)sa, 0, 129);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[rb][e] = fmaf(s[rb], ag[rb][e], acc[rb][e]);
}
// Q2_0_g64: the PQ2_0 operands, but a scale per 64 weights: lane groups 0-1
// hold the group's first 64 weights (chunk 2 g), 2-3 the second; each half
// is summed by its own MFMAs (B zero in the other half's lanes) from its
// own start value -2^(e-14) sum q over the half, and takes its own scale.
__device__ __forceinline__ void mx_group_g64(const i32x8 (&A)[kMxDigits], uint32_t sa,
                                             const f32x4 (&c0)[2], const u32x2 (&wv)[4],
                                             const float (&s)[2][4], bool upper, f32x4 (&acc)[4]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool mine = (h == 1) == upper;
    i32x8 B[4];
    f32x4 ag[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      // (the other half's lanes feed nibble 0, the value 0)
      const uint32_t lo = mine ? wv[rb].x : 0u, hi = mine ? wv[rb].y : 0u;
      B[rb] = fp4_b((int)(lo & 0x33333333u), (int)((lo >> 2) & 0x33333333u),
                  (int)(hi & 0x33333333u), (int)((hi >> 2) & 0x33333333u));
      ag[rb] = c0[h];
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], B[rb], ag[rb], 0, 4, 0, (int)sa, 0, 128);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], B[rb], ag[rb], 0, 4, 1, (int)sa, 0, 128);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      ag[rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[2], B[rb], ag[rb], 0, 4, 2, (int)sa, 0, 128);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[rb][e] = fmaf(s[h][rb], ag[rb][e], acc[rb][e]);
  }
}

template <int FMT, int BPS, int W>
__device__ __forceinline__ void mx_gemv_body(const uint8_t* __restrict__ packed,
                                             uint64_t scale_offset, int64_t C, int64_t G,
                                             int64_t N, int Sg, int Mreal,
                                             const uint4* __restrict__ xa,
                                             const uint32_t* __restrict__ xs,
                                             const float* __restrict__ xc,
                                             const float* __restrict__ xh,
                                             unsigned long long* __restrict__ sums, int64_t tile0,
                                             int64_t ntl, int64_t nta, int sgb, int light_last,
                                             uint16_t* __restrict__ y) {
  constexpr bool kQ1 = FMT == BGG_FMT_Q1_0, kG64 = FMT == BGG_FMT_Q2_0_G64;
  __shared__ float red[W][kMmaSlots * kMmaRedStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const WgSlot ws = wg_slot(tile0, ntl, nta, Sg, sgb, light_last != 0);
  const int64_t tile = ws.tile;
  const int64_t gbeg =
      ws.one ? (wave == 0 ? (int64_t)ws.wgs * BPS : G) : ((int64_t)ws.wgs * W + wave) * BPS;

  f32x4 acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  if (gbeg < G) {
    // PQ2_0 / Q2_0_g64: K 32 kg .. 32 kg + 31 of group g, row r: 8 bytes at
    // chunk 2 g + kg / 2, half kg % 2 -- uint2 index ((tile C + c) 64 + r) 2
    // + half.  Q1_0: the group is chunk g; word kg -- dword index
    // ((tile C + g) 64 + r) 4 + kg.
    const u32x2* wsrc =
        reinterpret_cast<const u32x2*>(packed) + ((tile * C + (kg >> 1)) * kTile + col) * 2 + (kg & 1);
    const uint32_t* wsrc1 = reinterpret_cast<const uint32_t*>(packed) + ((tile * C) * kTile + col) * 4 + kg;
    // scales per row: G (one per group), or 2 G for Q2_0_g64
    constexpr int kSc = kG64 ? 2 : 1;
    const uint16_t* ssrc =
        reinterpret_cast<const uint16_t*>(packed + scale_offset) + tile * (kSc * G) * kTile + col;
    // The slice runs in batches of NB groups (all BPS groups, or two halves
    // of eight; Q2_0_g64, with two start values and two scales per group
    // and row, batches of two: the registers hold one batch).  A batch's loads are issued
    // first, group by group (A digits, scale word, start values, weights,
    // weight scales), with no branch between them and their use: loads
    // complete in issue order, so group i waits only for its own loads and
    // those of the groups before it.  A group past G re-reads group G - 1
    // and gets a zero scale.  Lanes of token slots past M load no A bytes
    // and multiply zeros (their rows are dropped), so a few tokens cost few
    // A bytes.
    constexpr int NB = kG64 ? (BPS >= 8 ? 2 : BPS) : BPS <= 5 ? BPS : BPS / 2;
    static_assert(BPS % NB == 0, "whole batches");
    const bool aload = col < Mreal;
    const int aslot = aload ? col : Mreal - 1;
    const uint4* asrc = xa + (aslot + 16 * kg) * 2;
    // (a loop, not unrolled: the second batch's loads must not move above
    // the first batch's work)
#pragma unroll 1
    for (int b0 = 0; b0 < BPS; b0 += NB) {
      __builtin_amdgcn_sched_barrier(0);
      uint4 a[NB][kMxDigits][2];
      uint32_t sa[NB];
      f32x4 c0[NB][kSc];
      u32x2 w[NB][4];
      uint32_t w1[NB][4];
      uint16_t sc[NB][kSc][4];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int64_t g = gbeg + b0 + i < G ? gbeg + b0 + i : G - 1;
#pragma unroll
        for (int k = 0; k < kMxDigits; ++k) {
          a[i][k][0] = aload ? asrc[(g * kMxDigits + k) * 128] : make_uint4(0, 0, 0, 0);
          a[i][k][1] = aload ? asrc[(g * kMxDigits + k) * 128 + 1] : make_uint4(0, 0, 0, 0);
        }
        sa[i] = xs[g * kMmaSlots + aslot];
        if constexpr (kG64) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            c0[i][h] = *reinterpret_cast<const f32x4*>(xh + (g * 2 + h) * kMmaSlots + 4 * kg);
        } else {
          c0[i][0] = *reinterpret_cast<const f32x4*>(xc + g * kMmaSlots + 4 * kg);
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if constexpr (kQ1)
            w1[i][rb] = __builtin_nontemporal_load(wsrc1 + g * (4 * kTile) + rb * 64);
          else
            w[i][rb] = __builtin_nontemporal_load(wsrc + g * (4 * kTile) + rb * 32);
#pragma unroll
          for (int h = 0; h < kSc; ++h) sc[i][h][rb] = ssrc[(g * kSc + h) * kTile + 16 * rb];
        }
      }
      // keep the scheduler from sinking the loads towards their uses
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        i32x8 A[kMxDigits];
#pragma unroll
        for (int k = 0; k < kMxDigits; ++k) {
          A[k] = i32x8{(int)a[i][k][0].x, (int)a[i][k][0].y, (int)a[i][k][0].z,
                       (int)a[i][k][0].w, (int)a[i][k][1].x, (int)a[i][k][1].y,
                       (int)a[i][k][1].z, (int)a[i][k][1].w};
        }
        const bool live = gbeg + b0 + i < G;
        if constexpr (kG64) {
          float s2[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) s2[h][rb] = live ? h2f(sc[i][h][rb]) : 0.0f;
          mx_group_g64(A, sa[i], c0[i], w[i], s2, kg >= 2, acc);
        } else {
          float s[4];
#pragma unroll
          for (int rb = 0; rb < 4; ++rb) s[rb] = live ? h2f(sc[i][0][rb]) : 0.0f;
          if constexpr (kQ1)
            mx_group_q1(A, sa[i], c0[i][0], w1[i], s, acc);
          else
            mx_group(A, sa[i], c0[i][0], w[i], s, acc);
        }
      }
    }
  }
  // D layout: lane holds weight row 16 rb + col and token slots 4 kg + e
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      red[wave][(4 * kg + e) * kMmaRedStride + 16 * rb + col] = acc[rb][e];
  __syncthreads();
  for (int it = threadIdx.x; it < kMmaSlots * kTile; it += 64 * W) {
    const int t = it >> 6, r = it & 63;
    if (t >= Mreal) break;  // t only grows with it
    float v = red[0][t * kMmaRedStride + r];
#pragma unroll
    for (int q = 1; q < W; ++q) v += red[q][t * kMmaRedStride + r];
    const int64_t row = tile * kTile + r;
    if (ws.Sg == 1) {
      if (row < N) y[(int64_t)t * N + row] = f2h(v);
      continue;
    }
    if (row < N) add_partial(row_words_of(sums), t, ws.local * kTile + r, ws.Sg, v, y + (int64_t)t * N + row);
  }
}

#define BGG_MX_PARAMS                                                                         \
  const uint8_t *__restrict__ packed, uint64_t scale_offset, int64_t C, int64_t G, int64_t N,  \
      int Sg, int Mreal, const uint4 *__restrict__ xa, const uint32_t *__restrict__ xs,        \
      const float *__restrict__ xc, const float *__restrict__ xh,                              \
      unsigned long long *__restrict__ sums, int64_t tile0, int64_t ntl, int64_t nta, int sgb, \
      int light_last, uint16_t *__restrict__ y
#define BGG_MX_ARGS \
  packed, scale_offset, C, G, N, Sg, Mreal, xa, xs, xc, xh, sums, tile0, ntl, nta, sgb, light_last, y
// one kernel per format, so that a profiler names them apart
template <int BPS, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_pq2_mx(BGG_MX_PARAMS) {
  mx_gemv_body<BGG_FMT_PQ2_0, BPS, W>(BGG_MX_ARGS);
}
template <int BPS, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_q1_mx(BGG_MX_PARAMS) {
  mx_gemv_body<BGG_FMT_Q1_0, BPS, W>(BGG_MX_ARGS);
}
template <int BPS, int W>
__global__ void __launch_bounds__(64 * W) k_gemv_q2g64_mx(BGG_MX_PARAMS) {
  mx_gemv_body<BGG_FMT_Q2_0_G64, BPS, W>(BGG_MX_ARGS);
}
#undef BGG_MX_PARAMS
#undef BGG_MX_ARGS

// ---------------------------------------------------------------------------
// PTQ1_0 for several tokens on the matrix cores.  A wave takes one period
// (five groups, 128 row bytes) of one 64-row tile, as the VALU kernel with
// one part per period does, and gives the same bits:
//   1. each lane decodes its own row's 128 bytes through the LUT (entries in
//      the 2-bit code form, ten bits per byte) into the PQ2_0 code layout --
//      16 bytes are 80 positions, exactly five 32-bit words -- and stores
//      the 40 words of the period in LDS;
//   2. the MFMA loop of k_gemv_pq2_mx reads each lane's operand words (K
//      32 kg .. 32 kg + 31 of a group, rows col + 16 rb) from there.
// LDS: the LUT (64 KiB), the waves' code words (44 words per row), and the
// final reduction, which reuses the code words' space.
// ---------------------------------------------------------------------------
constexpr int kPtqCodeStride = 44;  // words per row in LDS: 40 + 4 against bank conflicts

template <int W>
__global__ void __launch_bounds__(64 * W)
    k_gemv_ptq1_mx(const uint8_t* __restrict__ packed, uint64_t scale_offset, int64_t C, int64_t G,
                   int64_t N, int Sg, int Mreal, const uint4* __restrict__ xa,
                   const uint32_t* __restrict__ xs, const float* __restrict__ xc,
                   unsigned long long* __restrict__ sums, int64_t tile0, int64_t ntl, int64_t nta,
                   int sgb, int light_last, uint16_t* __restrict__ y) {
  static_assert(W * 64 >= 256, "the LUT build needs 256 threads");
  static_assert(kMmaSlots * kMmaRedStride <= kTile * kPtqCodeStride, "red fits in a wave's codes");
  constexpr int PRE = 2;  // groups whose A operands are in flight
  __shared__ uint32_t lut[256 * kLutRowBytes / 4];
  __shared__ uint32_t lut_seed[256];
  __shared__ __attribute__((aligned(16))) uint32_t codes[W][kTile * kPtqCodeStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kg = lane >> 4;
  const WgSlot ws = wg_slot(tile0, ntl, nta, Sg, sgb, light_last != 0);
  const int64_t tile = ws.tile;
  const int64_t P = ceil_div(G, kPeriodGroups);
  const int64_t p = ws.one ? (wave == 0 ? ws.wgs : P) : (int64_t)ws.wgs * W + wave;
  const bool active = p < P;
  const int64_t g0 = p * kPeriodGroups;

  // Loads first, before the LUT is built: the row's 8 chunks of the period
  // (past the row they read the next tile's bytes or the buffer's zero
  // slack; those positions are in groups past G, which get a zero scale),
  // the weight scales, and the A operands of the first PRE groups.
  const bool aload = col < Mreal;
  const int aslot = aload ? col : Mreal - 1;
  const uint4* asrc = xa + (aslot + 16 * kg) * 2;
  uint4 wch[kPeriodChunks];
  uint16_t sc[kPeriodGroups][4];
  uint4 a[PRE][kMxDigits][2];
  uint32_t sa[PRE];
  f32x4 c0[PRE];
#define BGG_MX_LOAD_A(SLOT, I)                                                  \
  do {                                                                          \
    const int64_t g_ = g0 + (I) < G ? g0 + (I) : G - 1;                         \
    _Pragma("unroll") for (int k = 0; k < kMxDigits; ++k) {                    \
      a[SLOT][k][0] = aload ? asrc[(g_ * kMxDigits + k) * 128] : make_uint4(0, 0, 0, 0); \
      a[SLOT][k][1] = aload ? asrc[(g_ * kMxDigits + k) * 128 + 1] : make_uint4(0, 0, 0, 0); \
    }                                                                           \
    sa[SLOT] = xs[g_ * kMmaSlots + aslot];                                      \
    c0[SLOT] = *reinterpret_cast<const f32x4*>(xc + g_ * kMmaSlots + 4 * kg);   \
  } while (0)
  if (active) {
    const uint4* tdata = reinterpret_cast<const uint4*>(packed) + (tile * C) * kTile + lane;
#pragma unroll
    for (int c = 0; c < kPeriodChunks; ++c) wch[c] = ld_stream(tdata + (p * kPeriodChunks + c) * kTile);
    const uint16_t* ssrc =
        reinterpret_cast<const uint16_t*>(packed + scale_offset) + tile * G * kTile + col;
#pragma unroll
    for (int gi = 0; gi < kPeriodGroups; ++gi) {
      const int64_t g = g0 + gi < G ? g0 + gi : G - 1;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) sc[gi][rb] = ssrc[g * kTile + 16 * rb];
    }
#pragma unroll
    for (int i = 0; i < PRE; ++i) BGG_MX_LOAD_A(i, i);
  }
  __builtin_amdgcn_sched_barrier(0);
  build_lut32<kLutCodes>(lut, lut_seed);
  __syncthreads();

  uint32_t* cw = codes[wave];
  if (active) {
    // 1. decode: chunk c (bytes 16c .. 16c+15 of the period) -> words
    //    5c .. 5c+4 (byte j's ten code bits at bit 10 j of the 160)
    const uint32_t lane_off = lut_lane_off(lane);
    const char* lbase = reinterpret_cast<const char*>(lut);
#pragma unroll
    for (int c = 0; c < kPeriodChunks; ++c) {
      const uint32_t wd[4] = {wch[c].x, wch[c].y, wch[c].z, wch[c].w};
      uint32_t v[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[4 * q + 0] = *reinterpret_cast<const uint32_t*>(lbase + lut_addr<0>(wd[q], lane_off));
        v[4 * q + 1] = *reinterpret_cast<const uint32_t*>(lbase + lut_addr<1>(wd[q], lane_off));
        v[4 * q + 2] = *reinterpret_cast<const uint32_t*>(lbase + lut_addr<2>(wd[q], lane_off));
        v[4 * q + 3] = *reinterpret_cast<const uint32_t*>(lbase + lut_addr<3>(wd[q], lane_off));
      }
      uint32_t o[5];
      o[0] = v[0] | (v[1] << 10) | (v[2] << 20) | (v[3] << 30);
      o[1] = (v[3] >> 2) | (v[4] << 8) | (v[5] << 18) | (v[6] << 28);
      o[2] = (v[6] >> 4) | (v[7] << 6) | (v[8] << 16) | (v[9] << 26);
      o[3] = (v[9] >> 6) | (v[10] << 4) | (v[11] << 14) | (v[12] << 24);
      o[4] = (v[12] >> 8) | (v[13] << 2) | (v[14] << 12) | (v[15] << 22);
#pragma unroll
      for (int d = 0; d < 5; ++d) cw[lane * kPtqCodeStride + 5 * c + d] = o[d];
    }
  }
  wave_lds_sync();  // a wave reads only its own code words

  f32x4 acc[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (active) {
    // 2. per group: 3 MFMAs per row block, then acc += s * (2^(e-14) p)
#pragma unroll
    for (int gi = 0; gi < kPeriodGroups; ++gi) {
      const int slot = gi % PRE;
      i32x8 A[kMxDigits];
#pragma unroll
      for (int k = 0; k < kMxDigits; ++k) {
        A[k] = i32x8{(int)a[slot][k][0].x, (int)a[slot][k][0].y, (int)a[slot][k][0].z,
                     (int)a[slot][k][0].w, (int)a[slot][k][1].x, (int)a[slot][k][1].y,
                     (int)a[slot][k][1].z, (int)a[slot][k][1].w};
      }
      const uint32_t sac = sa[slot];
      const f32x4 cc = c0[slot];
      if (gi + PRE < kPeriodGroups) BGG_MX_LOAD_A(slot, gi + PRE);
      const bool live = g0 + gi < G;
      u32x2 wv[4];
      float s[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        wv[rb] = *reinterpret_cast<const u32x2*>(&cw[(col + 16 * rb) * kPtqCodeStride + 8 * gi + 2 * kg]);
        s[rb] = live ? h2f(sc[gi][rb]) : 0.0f;
      }
      mx_group(A, sac, cc, wv, s, acc);
    }
  }
#undef BGG_MX_LOAD_A
  // every wave is done with its code words before they become red
  __syncthreads();
  float* red = reinterpret_cast<float*>(codes[0]);
  constexpr int kRedWave = kTile * kPtqCodeStride;  // floats between waves' red rows
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      red[wave * kRedWave + (4 * kg + e) * kMmaRedStride + 16 * rb + col] = acc[rb][e];
  __syncthreads();
  for (int it = threadIdx.x; it < kMmaSlots * kTile; it += 64 * W) {
    const int t = it >> 6, r = it & 63;
    if (t >= Mreal) break;  // t only grows with it
    float v = red[t * kMmaRedStride + r];
#pragma unroll
    for (int q = 1; q < W; ++q) v += red[q * kRedWave + t * kMmaRedStride + r];
    const int64_t row = tile * kTile + r;
    if (ws.Sg == 1) {
      if (row < N) y[(int64_t)t * N + row] = f2h(v);
      continue;
    }
    if (row < N) add_partial(row_words_of(sums), t, ws.local * kTile + r, ws.Sg, v, y + (int64_t)t * N + row);
  }
}

// Activations for the matrix-core kernels.  Per 128-group and token slot:
// the same x', e and q as the encoding above; q's three base-32 digits as
// e4m3 bytes in the A operand order (xa: per group and digit, 64 lanes x 32
// bytes), the scale bytes 127 + e - 14 + 10 - 5 k of digit k (xs: one word
// per group and slot) and -2^(e-14) sum q (xc), and with xh the same over
// each 64-weight half (xh[group][half][slot], for Q2_0_g64).  Only the
// slots below M rounded up to four are written (slots past M-1 repeat token
// M - 1): the GEMV's lanes of slots past M load nothing, and their rows are
// dropped.  NATURAL: the B nibbles carry K in natural order (Q1_0), else in
// the PQ2_0 word order (mx_pos_of_k).  grid: (G, ceil(M / 4)) blocks of 64
// threads, four slots of one group per block, 16 lanes per slot.
constexpr int kPrepMxSlots = 4;
template <bool NATURAL>
__global__ void __launch_bounds__(64)
    k_gemv_prep_mx(const uint16_t* __restrict__ x, int64_t K, int M, int rotate,
                   uint32_t* __restrict__ xa, uint32_t* __restrict__ xs, float* __restrict__ xc,
                   float* __restrict__ xh) {
  // the e4m3 bytes of every digit, slot and group position
  __shared__ __attribute__((aligned(16))) uint8_t dig[kMxDigits][kPrepMxSlots][kGroup];
  const int64_t blk = blockIdx.x;
  const int ts = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  const int t = (int)blockIdx.y * kPrepMxSlots + ts;
  const int src = t < M ? t : M - 1;
  float v[8];
  load8h(x + (int64_t)src * K + blk * kGroup + 8 * l16, v);
  if (rotate) {
    fwht128_unscaled(v, l16);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= kHadamardNorm;
  }
  float amax = 0.0f;
  int nf = 0;  // a non-finite x' in the block
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    amax = fmaxf(amax, fabsf(v[j]));
    nf |= !(fabsf(v[j]) <= 3.0e38f);
  }
  amax = fmaxf(amax, xor16_f<1>(amax));
  amax = fmaxf(amax, xor16_f<2>(amax));
  amax = fmaxf(amax, xor16_f<4>(amax));
  amax = fmaxf(amax, xor16_f<8>(amax));
  nf |= xor16_i<1>(nf);
  nf |= xor16_i<2>(nf);
  nf |= xor16_i<4>(nf);
  nf |= xor16_i<8>(nf);
  if (nf) amax = 0.0f;  // digits 0; the correction terms below are NaN
  const float nanf_ = __builtin_nanf("");
  int e = 0;
  frexpf(amax, &e);
  int qsum = 0;
  uint32_t b[kMxDigits][2] = {{0, 0}, {0, 0}, {0, 0}};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = amax > 0.0f ? (int)rintf(ldexpf(v[j], 14 - e)) : 0;
    qsum += q;
    const int d2 = ((q + 16) & 31) - 16;
    const int r = (q - d2) >> 5;
    const int d1 = ((r + 16) & 31) - 16;
    const int d0 = (r - d1) >> 5;
    b[0][j >> 2] |= e4m3_of_int(d0) << (8 * (j & 3));
    b[1][j >> 2] |= e4m3_of_int(d1) << (8 * (j & 3));
    b[2][j >> 2] |= e4m3_of_int(d2) << (8 * (j & 3));
  }
#pragma unroll
  for (int k = 0; k < kMxDigits; ++k)
    *reinterpret_cast<uint2*>(&dig[k][ts][8 * l16]) = make_uint2(b[k][0], b[k][1]);
  qsum += xor16_i<1>(qsum);
  qsum += xor16_i<2>(qsum);
  qsum += xor16_i<4>(qsum);
  // lanes 0-7 (positions 0-63) and 8-15 (64-127) now hold their half's sum
  if (xh && (l16 & 7) == 0)
    xh[(blk * 2 + (l16 >> 3)) * kMmaSlots + t] =
        nf ? nanf_ : amax > 0.0f ? -(float)qsum * ldexpf(1.0f, e - 14) : 0.0f;
  qsum += xor16_i<8>(qsum);
  if (l16 == 0) {
    const int eb = amax > 0.0f ? e : 0;
    xs[blk * kMmaSlots + t] = (uint32_t)(123 + eb) | ((uint32_t)(118 + eb) << 8) |
                              ((uint32_t)(113 + eb) << 16) | (127u << 24);
    // a block with a non-finite x' starts its groups' sums at NaN: every
    // row of the token becomes NaN, as 0 * inf and NaN do in the fp64 product
    xc[blk * kMmaSlots + t] = nf ? nanf_ : amax > 0.0f ? -(float)qsum * ldexpf(1.0f, e - 14) : 0.0f;
  }
  __syncthreads();
  // this block's words: 3 digits x 4 lane groups x 4 slots x 8 words; word
  // dd of lane (slot tt, lane group ga) holds A bytes e = 4 dd .. 4 dd + 3,
  // i.e. the digits at the group positions that the B nibbles of those K
  // carry.  Those four K are consecutive from K0 = mx_k_of_a(ga, 4 dd), a
  // multiple of 4: in natural order four consecutive bytes (one 32-bit
  // read); in PQ2_0 order the positions p0, p0 + 2, p0 + 4, p0 + 6 with p0
  // = mx_pos_of_k(K0), all in the 8-byte block at p0 & ~7 (p0 % 8 is 0 or
  // 1): one 64-bit read and a byte select.
#pragma unroll
  for (int it0 = 0; it0 < kMxDigits * 4 * kPrepMxSlots * 8; it0 += 64) {
    const int it = it0 + threadIdx.x;
    const int k = it >> 7, ga = (it >> 5) & 3, tl = (it >> 3) & 3, dd = it & 7;
    const uint8_t* row = dig[k][tl];
    const int k0 = mx_k_of_a(ga, 4 * dd);
    uint32_t word;
    if (NATURAL) {
      word = *reinterpret_cast<const uint32_t*>(row + k0);
    } else {
      const int p0 = mx_pos_of_k(k0);
      const uint2 blk8 = *reinterpret_cast<const uint2*>(row + (p0 & ~7));
      word = __builtin_amdgcn_perm(blk8.y, blk8.x, 0x06040200u + (uint32_t)(p0 & 1) * 0x01010101u);
    }
    const int l = 16 * ga + (int)blockIdx.y * kPrepMxSlots + tl;
    xa[((blk * kMxDigits + k) * 64 + l) * 8 + dd] = word;
  }
}

// ---------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------
// Token slots of the prepared activations: padding tokens are zero.
inline int64_t gemv_m_slots(int64_t M) {
  return M <= 2 ? M : ((M + kGemvTokens - 1) / kGemvTokens) * kGemvTokens;
}

// Split of K: units along K (PQ2_0: groups, PTQ1_0: periods of 5 groups),
// units per wave slice, waves per workgroup W, slices S, workgroup slices
// Sg = ceil(S / W) (Sg > 1: the workgroups of a tile add their rows into
// 64-bit row sums), and the workspace layout.
struct GemvPlan {
  int64_t G, gpad, units, per_slice, W, S, Sg, NT, slots, frag_words_per_token;
  uint64_t off_frag, off_meta_q, off_meta_f, off_sums, total;
  int64_t nta, sgb;  // tiles with Sg slices; one-wave slices of the rest
  bool mma;          // PQ2_0 with several tokens: the matrix-core kernel
};

// The fewest tokens that run on the matrix-core kernels of this file: two
// (they measured faster than the VALU kernels from two tokens on, for both
// packings: the VALU kernels spend dot8 work per packed word or byte and
// token); every token count for the sister formats.
int64_t gemv_mma_min_tokens(int format) {
  return format == BGG_FMT_Q1_0 || format == BGG_FMT_Q2_0_G64 ? 1 : 2;
}

// Wave counts the K split aims at (measured on the projection shapes).
constexpr int64_t kTargetWaves = 2048;     // the split of K aims at this many waves
constexpr int64_t kMinSingleWaves = 1024;  // one workgroup per tile from this many waves

GemvPlan plan_gemv(const bgg_weights_desc* d, int64_t M) {
  GemvPlan p{};
  p.G = d->groups;
  p.NT = d->row_tiles;
  p.slots = gemv_m_slots(M);
  p.W = 8;
  p.mma = M >= gemv_mma_min_tokens(d->format);
  if (d->format != BGG_FMT_PTQ1_0) {
    p.gpad = p.G;
    p.units = p.G;
    p.frag_words_per_token = (d->K / 64) * kPqFragWords;
    // one workgroup per tile (no partial rows) when that still fills the
    // chip: the smallest groups-per-wave with all of K in 8 waves
    // (Q2_0_g64 has no five-group slices: its batches hold two groups)
    const int64_t one_wg[] = {2, 4, 5, 8};
    p.per_slice = 0;
    for (int64_t b : one_wg)
      if (ceil_div(p.units, b) <= p.W && p.NT * p.W >= kMinSingleWaves &&
          !(b == 5 && d->format == BGG_FMT_Q2_0_G64)) {
        p.per_slice = b;
        break;
      }
    if (!p.per_slice) {
      // else the largest groups-per-wave that gives the target wave count
      p.per_slice = 8;
      // (as long as the slices of a tile stay within what a row word counts)
      while (p.per_slice > 2 && p.NT * p.W * ceil_div(ceil_div(p.units, p.per_slice), p.W) < kTargetWaves &&
             ceil_div(ceil_div(p.units, p.per_slice / 2), p.W) <= kMaxSumSlices)
        p.per_slice /= 2;
    }
    p.S = ceil_div(p.units, p.per_slice);
  } else {
    // units are period parts: H parts per period, H = 2 only for one token
    // and only when whole periods give fewer waves than the target (more
    // parts mean more per-wave and per-workgroup overhead); 8 waves per
    // workgroup (16 measured slower: the LUT barrier waits for more waves)
    const int64_t P = ceil_div(p.G, kPeriodGroups);
    p.gpad = P * kPeriodGroups;
    p.frag_words_per_token = P * kPtqFragWords;
    p.per_slice = 1;
    while (p.per_slice < 2 && !p.mma && p.NT * P * p.per_slice < kTargetWaves &&
           ceil_div(P * 2, p.W) <= kMaxSumSlices)
      p.per_slice *= 2;
    p.units = P * p.per_slice;
    p.S = p.units;
  }
  p.Sg = ceil_div(p.S, p.W);
  if (p.Sg > kMaxSumSlices) return GemvPlan{};  // K beyond what a row sum counts
  // tiles left over above a multiple of the CU count: one-wave slices
  p.nta = p.NT;
  p.sgb = 1;
  if (p.Sg == 1 && p.S <= kMaxSumSlices && p.NT * kTile <= kSumRows) {
    const int64_t ncu = device_cus(), r = p.NT % ncu;
    if (p.NT > ncu && r != 0 && r * p.S <= 2 * ncu) {
      p.nta = p.NT - r;
      p.sgb = p.S;
    }
  }
  // [row sums][digit words][group Q][group F]: the row sums are the same for
  // every call, the rest depends only on the format, K and M
  // (the frag region also holds the matrix-core kernels' A digits, and the
  // group-Q region their scale words and start values: reserved for every
  // M, so that the size does not depend on which kernel runs)
  uint64_t frag_bytes = (uint64_t)p.slots * p.frag_words_per_token * 4;
  uint64_t meta_q_bytes = (uint64_t)p.slots * p.gpad * 4;
  frag_bytes = std::max<uint64_t>(frag_bytes, (uint64_t)p.G * kMxDigits * 64 * 32);
  meta_q_bytes = std::max<uint64_t>(meta_q_bytes, (uint64_t)p.G * kMmaSlots * 16);
  p.off_sums = 0;
  p.off_frag = std::max<uint64_t>(kSumBytes, mxv_workspace_bytes());
  uint64_t off = align256(p.off_frag + frag_bytes);
  p.off_meta_q = off;
  off = align256(off + meta_q_bytes);
  p.off_meta_f = off;
  off = align256(off + (uint64_t)p.slots * p.gpad * 4);
  p.total = off;
  return p;
}

void launch_prep(const bgg_weights_desc* d, const GemvPlan& p, const uint16_t* x, int64_t M,
                 int rotate, uint8_t* ws, hipStream_t st) {
  uint32_t* frag = reinterpret_cast<uint32_t*>(ws + p.off_frag);
  int32_t* mq = reinterpret_cast<int32_t*>(ws + p.off_meta_q);
  float* mf = reinterpret_cast<float*>(ws + p.off_meta_f);
  if (p.mma) {
    // [xs: G x 16 words][xc: G x 16][xh: G x 2 x 16 (Q2_0_g64)]
    uint32_t* xs = reinterpret_cast<uint32_t*>(ws + p.off_meta_q);
    float* xc = reinterpret_cast<float*>(xs + p.G * kMmaSlots);
    float* xh = d->format == BGG_FMT_Q2_0_G64 ? xc + p.G * kMmaSlots : nullptr;
    uint32_t* xa = reinterpret_cast<uint32_t*>(ws + p.off_frag);
    const dim3 grid((unsigned)p.G, (unsigned)ceil_div(M, kPrepMxSlots));
    if (d->format == BGG_FMT_Q1_0)
      hipLaunchKernelGGL(k_gemv_prep_mx<true>, grid, dim3(64), 0, st, x, d->K, (int)M, rotate, xa,
                         xs, xc, xh);
    else
      hipLaunchKernelGGL(k_gemv_prep_mx<false>, grid, dim3(64), 0, st, x, d->K, (int)M, rotate,
                         xa, xs, xc, xh);
    return;
  }
  const dim3 grid((unsigned)ceil_div(p.gpad, kPrepGroups), (unsigned)p.slots);
  if (d->format == BGG_FMT_PQ2_0)
    hipLaunchKernelGGL(k_gemv_prep<BGG_FMT_PQ2_0>, grid, dim3(64), 0, st, x, d->K, (int)M,
                       rotate, frag, p.frag_words_per_token, mq, mf, p.gpad);
  else
    hipLaunchKernelGGL(k_gemv_prep<BGG_FMT_PTQ1_0>, grid, dim3(64), 0, st, x, d->K,
                       (int)M, rotate, frag, p.frag_words_per_token, mq, mf, p.gpad);
}

// The VALU GEMV for one token (one launch, or one per kSumRows rows of split
// tiles).  FUSE (PTQ1_0 only): the kernel also encodes the activations from
// fa.x; else it reads the preparation in the workspace.
template <bool FUSE>
void launch_gemv1(const bgg_weights_desc* d, const GemvPlan& p, const uint8_t* packed, uint16_t* y,
                  uint8_t* ws, const FuseArgs& fa, hipStream_t st) {
  const uint32_t* frag = reinterpret_cast<const uint32_t*>(ws + p.off_frag);
  const int32_t* mq = reinterpret_cast<const int32_t*>(ws + p.off_meta_q);
  const float* mf = reinterpret_cast<const float*>(ws + p.off_meta_f);
  unsigned long long* sums = reinterpret_cast<unsigned long long*>(ws + p.off_sums);
  const int Sg = (int)p.Sg;
  const dim3 block((unsigned)(64 * p.W));
  // split tiles add into the row sums, which hold kSumRows rows: one launch
  // per kSumRows / 64 tiles (one-wave slices only in a single launch)
  const int64_t chunk = Sg > 1 ? kSumRows / kTile : p.NT;
  for (int64_t t0 = 0; t0 < p.NT; t0 += chunk) {
    const int64_t ntl = p.NT - t0 < chunk ? p.NT - t0 : chunk;
    // with one-wave slices (p.sgb > 1): nta full tiles, the rest in one-wave
    // slices; else every tile has Sg slices
    const int64_t nta = p.sgb > 1 ? p.nta : ntl;
    const int sgb = (int)p.sgb;
    // (with split tiles whose slices do not fill the last workgroup: that
    // light workgroup is dispatched first)
    const int light = p.Sg > 1 && p.S % p.W != 0 ? 1 : 0;
    const dim3 grid((unsigned)(nta * Sg + (ntl - nta) * sgb));
    if constexpr (!FUSE) {
      if (d->format == BGG_FMT_PQ2_0) {
#define BGG_PQ2(BPS)                                                                              \
  hipLaunchKernelGGL((k_gemv_pq2<1, BPS, 8>), grid, block, 0, st, packed, d->scale_offset, d->chunks, \
                     p.G, d->N, Sg, 1, frag, p.frag_words_per_token, mq, mf, p.gpad, sums, t0, ntl,  \
                     nta, sgb, light, y)
        switch (p.per_slice) {
          case 8: BGG_PQ2(8); break;
          case 5: BGG_PQ2(5); break;
          case 4: BGG_PQ2(4); break;
          default: BGG_PQ2(2); break;
        }
#undef BGG_PQ2
        continue;
      }
    }
#define BGG_PTQ1(H)                                                                                    \
  hipLaunchKernelGGL((k_gemv_ptq1<1, H, 8, FUSE>), grid, block, 0, st, packed, d->scale_offset,    \
                     d->chunks, p.G, d->N, Sg, 1, frag, p.frag_words_per_token, mq, mf, p.gpad, sums, \
                     t0, ntl, nta, sgb, light, fa, y)
    if (p.per_slice == 2)
      BGG_PTQ1(2);
    else
      BGG_PTQ1(1);
#undef BGG_PTQ1
  }
}

// The matrix-core GEMV for several tokens (one launch, or one per kSumRows
// rows of split tiles); the plan's work split is the VALU kernels'.
void launch_gemv_mma(const bgg_weights_desc* d, const GemvPlan& p, const uint8_t* packed,
                     uint16_t* y, int Mreal, uint8_t* ws, hipStream_t st) {
  const uint4* xa = reinterpret_cast<const uint4*>(ws + p.off_frag);
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(ws + p.off_meta_q);
  const float* xc = reinterpret_cast<const float*>(xs + p.G * kMmaSlots);
  const float* xh = d->format == BGG_FMT_Q2_0_G64 ? xc + p.G * kMmaSlots : nullptr;
  unsigned long long* sums = reinterpret_cast<unsigned long long*>(ws + p.off_sums);
  const int Sg = (int)p.Sg;
  const dim3 block(64 * 8);
  const int64_t chunk = Sg > 1 ? kSumRows / kTile : p.NT;
  for (int64_t t0 = 0; t0 < p.NT; t0 += chunk) {
    const int64_t ntl = p.NT - t0 < chunk ? p.NT - t0 : chunk;
    const int64_t nta = p.sgb > 1 ? p.nta : ntl;
    const int sgb = (int)p.sgb;
    const int light = p.Sg > 1 && p.S % p.W != 0 ? 1 : 0;
    const dim3 grid((unsigned)(nta * Sg + (ntl - nta) * sgb));
    if (d->format == BGG_FMT_PTQ1_0) {
      hipLaunchKernelGGL((k_gemv_ptq1_mx<8>), grid, block, 0, st, packed, d->scale_offset,
                         d->chunks, p.G, d->N, Sg, Mreal, xa, xs, xc, sums, t0, ntl, nta, sgb,
                         light, y);
      continue;
    }
#define BGG_MMA_ONE(KERN, BPS)                                                                 \
  hipLaunchKernelGGL((KERN<BPS, 8>), grid, block, 0, st, packed, d->scale_offset, d->chunks,    \
                     p.G, d->N, Sg, Mreal, xa, xs, xc, xh, sums, t0, ntl, nta, sgb, light, y)
#define BGG_MMA(KERN)                          \
  switch (p.per_slice) {                       \
    case 8: BGG_MMA_ONE(KERN, 8); break;       \
    case 5: BGG_MMA_ONE(KERN, 5); break;       \
    case 4: BGG_MMA_ONE(KERN, 4); break;       \
    default: BGG_MMA_ONE(KERN, 2); break;      \
  }
    if (d->format == BGG_FMT_Q1_0) {
      BGG_MMA(k_gemv_q1_mx);
    } else if (d->format == BGG_FMT_Q2_0_G64) {
      switch (p.per_slice) {  // (never 5)
        case 8: BGG_MMA_ONE(k_gemv_q2g64_mx, 8); break;
        case 4: BGG_MMA_ONE(k_gemv_q2g64_mx, 4); break;
        default: BGG_MMA_ONE(k_gemv_q2g64_mx, 2); break;
      }
    } else {
      BGG_MMA(k_gemv_pq2_mx);
    }
#undef BGG_MMA
#undef BGG_MMA_ONE
  }
}

bgg_status gemv_args_check(const char* who, const bgg_weights_desc* d, int64_t M,
                           const void* workspace, size_t workspace_bytes, GemvPlan* plan) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!workspace) return fail(BGG_ERR_NULL, "%s: NULL workspace", who);
  if (M < 1 || M > BGG_MAX_GEMV_M)
    return fail(BGG_ERR_SHAPE, "%s: M must be in 1..16 (got %lld)", who, (long long)M);
  if (!aligned16(workspace)) return fail(BGG_ERR_BUFFER, "%s: misaligned workspace", who);
  *plan = plan_gemv(d, M);
  if (plan->total == 0)
    return fail(BGG_ERR_SHAPE, "%s: K = %lld needs more K slices than a row sum counts", who,
                (long long)d->K);
  if (workspace_bytes < plan->total)
    return fail(BGG_ERR_BUFFER, "%s: workspace has %zu bytes, needs %llu", who, workspace_bytes,
                (unsigned long long)plan->total);
  return BGG_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

size_t bgg_gemv_workspace_size(const bgg_weights_desc* d, int64_t M) {
  if (check_desc(d) != BGG_OK || M < 1 || M > BGG_MAX_GEMV_M) return 0;
  return (size_t)plan_gemv(d, M).total;
}

bgg_status bgg_gemv_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(BGG_ERR_NULL, "bgg_gemv_workspace_reset: NULL workspace");
  if (!aligned16(workspace) || workspace_bytes % 16)
    return fail(BGG_ERR_BUFFER, "bgg_gemv_workspace_reset: workspace or size not a multiple of 16 bytes");
  const uint64_t n16 = std::min<uint64_t>(workspace_bytes, kSumBytes) / 16;
  if (n16 == 0) return BGG_OK;
  hipLaunchKernelGGL(k_fill_zero16, dim3((unsigned)std::min<uint64_t>(ceil_div(n16, 256), 2048)), dim3(256), 0,
                     (hipStream_t)stream, reinterpret_cast<uint4*>(workspace), (int64_t)n16);
  return hip_check("bgg_gemv_workspace_reset");
}

bgg_status bgg_gemv_kernel_name(const bgg_weights_desc* d, int64_t M, char* out, size_t cap) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!out) return fail(BGG_ERR_NULL, "bgg_gemv_kernel_name: NULL out");
  if (M < 1 || M > BGG_MAX_GEMV_M)
    return fail(BGG_ERR_SHAPE, "bgg_gemv_kernel_name: M must be in 1..16 (got %lld)", (long long)M);
  const GemvPlan p = plan_gemv(d, M);
  int n;
  if (mxv_supported(d, M)) {
    n = mxv_kernel_name(d, M, out, cap);
  } else if (p.mma && d->format == BGG_FMT_PTQ1_0) {
    n = snprintf(out, cap, "k_gemv_ptq1_mx<8>");
  } else if (p.mma) {
    const char* kn = d->format == BGG_FMT_Q1_0       ? "k_gemv_q1_mx"
                     : d->format == BGG_FMT_Q2_0_G64 ? "k_gemv_q2g64_mx"
                                                     : "k_gemv_pq2_mx";
    n = snprintf(out, cap, "%s<%d, 8>", kn, (int)p.per_slice);
  } else if (d->format == BGG_FMT_PQ2_0) {  // (K beyond the one-launch kernel's reach)
    n = snprintf(out, cap, "k_gemv_pq2<1, %d, 8>", (int)p.per_slice);
  } else {
    n = snprintf(out, cap, "k_gemv_ptq1<1, %d, 8, true>", p.per_slice == 2 ? 2 : 1);
  }
  if (n < 0 || (size_t)n >= cap)
    return fail(BGG_ERR_BUFFER, "bgg_gemv_kernel_name: %zu bytes are too few", cap);
  return BGG_OK;
}

bgg_status bgg_gemv_prepare(const bgg_weights_desc* d, const void* x_dev, int64_t M, uint32_t flags,
                            void* workspace, size_t workspace_bytes, void* stream) {
  GemvPlan p;
  bgg_status st = gemv_args_check("bgg_gemv_prepare", d, M, workspace, workspace_bytes, &p);
  if (st) return st;
  if (!x_dev) return fail(BGG_ERR_NULL, "bgg_gemv_prepare: NULL x");
  if (!aligned16(x_dev)) return fail(BGG_ERR_BUFFER, "bgg_gemv_prepare: misaligned x");
  if (flags & ~(uint32_t)BGG_ROTATE_INPUT)
    return fail(BGG_ERR_SHAPE, "bgg_gemv_prepare: unknown flags 0x%x", flags);
  launch_prep(d, p, (const uint16_t*)x_dev, M, (flags & BGG_ROTATE_INPUT) ? 1 : 0,
              (uint8_t*)workspace, (hipStream_t)stream);
  return hip_check("bgg_gemv_prepare");
}

bgg_status bgg_gemv_run(const bgg_weights_desc* d, const void* packed_dev, void* y_dev, int64_t M,
                        void* workspace, size_t workspace_bytes, void* stream) {
  GemvPlan p;
  bgg_status st = gemv_args_check("bgg_gemv_run", d, M, workspace, workspace_bytes, &p);
  if (st) return st;
  if (!packed_dev || !y_dev) return fail(BGG_ERR_NULL, "bgg_gemv_run: NULL buffer");
  if (!aligned16(packed_dev) || ((uintptr_t)y_dev & 1))
    return fail(BGG_ERR_BUFFER, "bgg_gemv_run: misaligned buffer");
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* pk = (const uint8_t*)packed_dev;
  uint8_t* ws = (uint8_t*)workspace;
  uint16_t* y = (uint16_t*)y_dev;
  if (p.mma) {
    launch_gemv_mma(d, p, pk, y, (int)M, ws, s);
    return hip_check("bgg_gemv_run");
  }
  launch_gemv1<false>(d, p, pk, y, ws, FuseArgs{}, s);  // (one token: the plan has no mma)
  return hip_check("bgg_gemv_run");
}

bgg_status bgg_ternary_gemv(const bgg_weights_desc* d, const void* packed_dev, const void* x_dev,
                            void* y_dev, int64_t M, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!packed_dev || !y_dev) return fail(BGG_ERR_NULL, "bgg_ternary_gemv: NULL buffer");
  if (!aligned16(packed_dev) || ((uintptr_t)y_dev & 1))
    return fail(BGG_ERR_BUFFER, "bgg_ternary_gemv: misaligned buffer");
  if (mxv_supported(d, M)) {
    GemvPlan p;
    st = gemv_args_check("bgg_ternary_gemv", d, M, workspace, workspace_bytes, &p);
    if (st) return st;
    if (!x_dev) return fail(BGG_ERR_NULL, "bgg_ternary_gemv: NULL x");
    if (!aligned16(x_dev)) return fail(BGG_ERR_BUFFER, "bgg_ternary_gemv: misaligned x");
    if (flags & ~(uint32_t)BGG_ROTATE_INPUT)
      return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: unknown flags 0x%x", flags);
    return mxv_launch(d, packed_dev, x_dev, y_dev, M, (flags & BGG_ROTATE_INPUT) ? 1 : 0, workspace,
                      (hipStream_t)stream);
  }
  // one PTQ1_0 token runs in one launch; everything else not served above
  // (several PTQ1_0 tokens, five and more PQ2_0 tokens, the sister formats,
  // PQ2_0 K beyond the one-launch kernel's reach) in two steps
  if (M != 1 || d->format != BGG_FMT_PTQ1_0) {
    st = bgg_gemv_prepare(d, x_dev, M, flags, workspace, workspace_bytes, stream);
    if (st) return st;
    return bgg_gemv_run(d, packed_dev, y_dev, M, workspace, workspace_bytes, stream);
  }
  // one token: a single launch that also encodes the activations
  GemvPlan p;
  st = gemv_args_check("bgg_ternary_gemv", d, M, workspace, workspace_bytes, &p);
  if (st) return st;
  if (!x_dev) return fail(BGG_ERR_NULL, "bgg_ternary_gemv: NULL x");
  if (!aligned16(x_dev)) return fail(BGG_ERR_BUFFER, "bgg_ternary_gemv: misaligned x");
  if (flags & ~(uint32_t)BGG_ROTATE_INPUT)
    return fail(BGG_ERR_SHAPE, "bgg_ternary_gemv: unknown flags 0x%x", flags);
  FuseArgs fa;
  fa.x = (const uint16_t*)x_dev;
  fa.rotate = (flags & BGG_ROTATE_INPUT) ? 1 : 0;
  launch_gemv1<true>(d, p, (const uint8_t*)packed_dev, (uint16_t*)y_dev, (uint8_t*)workspace, fa,
                     (hipStream_t)stream);
  return hip_check("bgg_ternary_gemv");
}

}  // extern "C"
