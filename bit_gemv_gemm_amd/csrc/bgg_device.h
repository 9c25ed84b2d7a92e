// Device helpers shared by the kernels of libbgg (gfx950).
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bgg_internal.h"

namespace bgg {

constexpr int kGroup = BGG_GROUP;   // 128 weights per scale / Hadamard block
constexpr int kTile = BGG_ROW_TILE;  // 64 weight rows per tile, one per lane

// PTQ1_0 period: 5 groups = 640 trits = 128 row bytes = 8 chunks.  Group
// ends fall inside bytes 25, 51, 76 and 102 of every period and at its end.
constexpr int kPeriodGroups = 5;
constexpr int kPeriodBytes = 128;
constexpr int kPeriodChunks = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of data that is read once (packed weights): non-temporal.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// The fp16 scale of lane `lane` from a row of 64 scales at p: each lane reads
// the aligned 32-bit word holding its scale and its neighbour's (neighbouring
// lanes read the same word; the access stays one coalesced 256-byte read) and
// keeps its half later with scale_half().  A 16-bit load would let the
// compiler pack two scales into one register right after the loads, which
// makes the wave wait for every load issued before them at that point.
__device__ __forceinline__ uint32_t ld_scale_pair(const uint16_t* row64, int lane) {
  return reinterpret_cast<const uint32_t*>(row64)[lane >> 1];
}
__device__ __forceinline__ float scale_half(uint32_t pair, int lane) {
  return h2f((uint16_t)(pair >> ((lane & 1) * 16)));
}
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// 1/sqrt(128) rounded to fp32.
constexpr float kHadamardNorm = 0.08838834764831845f;

// v of lane l ^ m within each group of 16 lanes (m = 1, 2, 4 or 8), with
// DPP lane moves, which cost no LDS trip: m = 1, 2 are quad permutations,
// m = 8 a rotation of the 16-lane row by 8, and m = 4 two row shifts that
// each write only the 4-lane banks that read in their direction.
template <int m>
__device__ __forceinline__ int xor16_i(int v) {
  static_assert(m == 1 || m == 2 || m == 4 || m == 8, "xor16: m in {1, 2, 4, 8}");
  if (m == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  if (m == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  if (m == 8) return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror:8
  // lanes 0-3, 8-11 (banks 0, 2) read l + 4 (row_shl:4); lanes 4-7, 12-15
  // (banks 1, 3) read l - 4 (row_shr:4)
  const int t = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);
  return __builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false);
}
template <int m>
__device__ __forceinline__ float xor16_f(float v) {
  return __int_as_float(xor16_i<m>(__float_as_int(v)));
}

// Fast Walsh-Hadamard transform (Sylvester order, unnormalised) of one
// 128-block held by 16 lanes, 8 consecutive values each (lane i of the 16
// holds positions 8i..8i+7).  Butterflies (a, b) -> (a + b, a - b) over
// strides 1..64, in fp32.
template <int m>
__device__ __forceinline__ void fwht_lane_stage(float v[8], int lane16) {
  const float sgn = (lane16 & m) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = xor16_f<m>(v[i]);
    v[i] = fmaf(sgn, v[i], p);  // low lane: v + p; high lane: p - v
  }
}
__device__ __forceinline__ void fwht128_unscaled(float v[8], int lane16) {
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & s)) {
        const float a = v[i], b = v[i + s];
        v[i] = a + b;
        v[i + s] = a - b;
      }
  }
  fwht_lane_stage<1>(v, lane16);
  fwht_lane_stage<2>(v, lane16);
  fwht_lane_stage<4>(v, lane16);
  fwht_lane_stage<8>(v, lane16);
}

__device__ __forceinline__ void unpack8h(const uint4 u, float v[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = h2f((uint16_t)(w[i] & 0xFFFF));
    v[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8h(const uint16_t* p, float v[8]) {
  unpack8h(*reinterpret_cast<const uint4*>(p), v);
}

// PQ2_0: 16 codes of one word -> codes of even positions in the low two
// bits of each nibble (E) and of odd positions likewise (O).
__device__ __forceinline__ uint32_t pq2_even(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t pq2_odd(uint32_t w) { return (w >> 2) & 0x33333333u; }

// PTQ1_0: the five base-3 digits of a byte (= t + 1 of five trits), one per
// nibble 0..4.  Bytes 243..255 come from no trits; they decode as five zero
// trits (digits 1).
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

// The GEMV's LUT holds the trits themselves, t = c - 1 as signed 4-bit
// nibbles (-1 = 0xF), five to a word.  Entry e occupies a 256-byte row at
// e * 256; copy c of it is the word at e * 256 + c * 4, and lane l reads copy
// l % 32, so the 32 lanes that the LDS serves together hit 32 different
// banks whatever entries they want.  The address of byte j of a packed word
// w is then one v_perm_b32: byte 0 = (l % 32) * 4 (from lane_off), byte 1 =
// byte j of w, bytes 2-3 = 0.  Only the first 128 bytes of each row are
// written (32 KiB of stores), but the rows span 64 KiB of LDS.  (64 copies,
// one per lane, were measured no faster to read and twice as slow to build.)
constexpr int kLutRowBytes = 256;
constexpr int kLutCopies32 = 32;
__device__ __forceinline__ uint32_t ptq1_trit_nibbles(uint32_t b) {
  const uint32_t c = ptq1_entry(b);
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) t |= ((((c >> (4 * i)) & 15u) + 15u) & 15u) << (4 * i);
  return t;
}
__device__ __forceinline__ uint32_t lut_lane_off(int lane) { return (uint32_t)(lane & 31) * 4u; }
// The same five trits as codes c = t + 1 in 2-bit fields (code i in bits
// 2i..2i+1): the PQ2_0 code form, ten bits per byte.
__device__ __forceinline__ uint32_t ptq1_codes10(uint32_t b) {
  const uint32_t c = ptq1_entry(b);
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) r |= ((c >> (4 * i)) & 3u) << (2 * i);
  return r;
}
// The same five trits as fp4 (e2m1) matrix-core operands, one per nibble
// 0..4: +1 = 0x2 (1.0), -1 = 0xA (-1.0), 0 = 0x0; nibbles 5..7 are zero.
__device__ __forceinline__ uint32_t ptq1_e2m1_nibbles(uint32_t b) {
  const uint32_t c = ptq1_entry(b);
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t ci = (c >> (4 * i)) & 15u;
    r |= (ci == 2u ? 0x2u : ci == 0u ? 0xAu : 0u) << (4 * i);
  }
  return r;
}
// Entry forms of the table below.
constexpr int kLutTrits = 0;  // signed trit nibbles (ptq1_trit_nibbles)
constexpr int kLutCodes = 1;  // 2-bit codes (ptq1_codes10)
constexpr int kLutE2m1 = 2;   // e2m1 nibbles (ptq1_e2m1_nibbles)
template <int FORM>
__device__ __forceinline__ uint32_t ptq1_lut_entry(uint32_t b) {
  return FORM == kLutCodes ? ptq1_codes10(b) : FORM == kLutE2m1 ? ptq1_e2m1_nibbles(b)
                                                                : ptq1_trit_nibbles(b);
}
// Built in two steps: the first 256 threads each decode one byte value into
// seed[], then (after a barrier) every thread copies entries out, 16 bytes
// per store.  Needs blockDim.x >= 256; the caller synchronises afterwards.
template <int FORM = kLutTrits>
__device__ __forceinline__ void build_lut32(uint32_t* lut, uint32_t* seed) {
  if (threadIdx.x < 256) seed[threadIdx.x] = ptq1_lut_entry<FORM>(threadIdx.x);
  __syncthreads();
  constexpr int kQuads = kLutCopies32 / 4, kRowQuads = kLutRowBytes / 16;
  for (int i = threadIdx.x; i < 256 * kQuads; i += blockDim.x) {
    const int e = i / kQuads, q = i % kQuads;
    const uint32_t v = seed[e];
    reinterpret_cast<uint4*>(lut)[e * kRowQuads + q] = make_uint4(v, v, v, v);
  }
}

// The wave's own LDS writes are visible to all its lanes after this: LDS
// executes a wave's instructions in order, and the fence keeps the compiler
// from moving the reads above the writes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// s_waitcnt lgkmcnt(0) with the other counters left alone (gfx9 encoding:
// vmcnt 63, expcnt 7).  LDS reads and scalar loads share this counter and
// scalar loads may return out of order, so a kernel that wants its scalar
// loads to overlap LDS work waits for both explicitly at the point it picks.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
template <int J>
__device__ __forceinline__ uint32_t lut_addr(uint32_t word, uint32_t lane_off) {
  return __builtin_amdgcn_perm(word, lane_off, 0x0C0C0000u | ((4u + J) << 8));
}

// fp16 matrix-core operands (v_mfma_f32_32x32x16_f16)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// The three values an fp16 scale s gives a PQ2_0 code c = t + 1, as a
// byte-select table for v_perm_b32: `lo` holds the low byte of the value of
// code c in byte c, `hi` its high byte in byte c.
// Code 0 is -s (s with the sign bit flipped), code 1 is 0, code 2 is +s;
// code 3, which no valid buffer holds, reads 0 like code 1.
struct Pq2Table {
  uint32_t lo, hi;
};
__device__ __forceinline__ Pq2Table pq2_table(uint32_t sbits) {
  const uint32_t l = sbits & 0xFFu, h = (sbits >> 8) & 0xFFu;
  return {l * 0x00010001u, (h ^ 0x80u) | (h << 16)};
}

// Eight consecutive PQ2_0 codes (bits `shift` .. `shift` + 15 of a code
// word: code i in bits 2i..2i+1 of that field) -> the fp16 MFMA operand
// (s*t_0, ..., s*t_7), bit for bit the value s*t (+-s or 0) -- no
// arithmetic, only byte moves.  t | t << 14 puts codes 0, 4 in bytes 0, 1
// and codes 1, 5 in bytes 2, 3 (two-bit fields at the byte starts); shifted
// down by four the same holds for codes 2, 6, 3, 7.  Those four codes, used
// as byte selectors as they are, read the low bytes of their values from
// the table's `lo` word and the high bytes from its `hi` word (one byte
// permute each); a third permute pairs each low byte with its high byte.
__device__ __forceinline__ f16x8 decode8_pq2(uint32_t word, uint32_t shift, Pq2Table tb) {
  const uint32_t t = __builtin_amdgcn_ubfe(word, shift, 16);
  uint32_t z;  // t | t << 14 in one instruction
  asm("v_lshl_or_b32 %0, %1, 14, %1" : "=v"(z) : "v"(t));
  const uint32_t ab = z & 0x03030303u, cd = (z >> 4) & 0x03030303u;  // codes (0, 4, 1, 5), (2, 6, 3, 7)
  const uint32_t lab = __builtin_amdgcn_perm(0u, tb.lo, ab), hab = __builtin_amdgcn_perm(0u, tb.hi, ab);
  const uint32_t lcd = __builtin_amdgcn_perm(0u, tb.lo, cd), hcd = __builtin_amdgcn_perm(0u, tb.hi, cd);
  uint32_t out[4];
  out[0] = __builtin_amdgcn_perm(hab, lab, 0x06020400u);  // values of codes 0, 1
  out[1] = __builtin_amdgcn_perm(hcd, lcd, 0x06020400u);  // 2, 3
  out[2] = __builtin_amdgcn_perm(hab, lab, 0x07030501u);  // 4, 5
  out[3] = __builtin_amdgcn_perm(hcd, lcd, 0x07030501u);  // 6, 7
  f16x8 r;
  __builtin_memcpy(&r, out, sizeof(r));
  return r;
}

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

inline bgg_status hip_check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BGG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return BGG_OK;
}

// Compute units of the current device (cached per device; 256 if the
// runtime cannot tell).
inline int64_t device_cus() {
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

// The matrix-core GEMV of bgg_mxv.hip (one launch that also transforms x;
// PQ2_0 for 1..4 tokens, PTQ1_0 for 1..2): whether it serves (format, M),
// the workspace bytes it uses at the start of a GEMV workspace (row words
// that every launch leaves zero), the name of the kernel it launches
// (snprintf's return), and the launch.
bool mxv_supported(const bgg_weights_desc* d, int64_t M);
uint64_t mxv_workspace_bytes();
int mxv_kernel_name(const bgg_weights_desc* d, int64_t M, char* out, size_t cap);
bgg_status mxv_launch(const bgg_weights_desc* d, const void* packed, const void* x, void* y,
                      int64_t M, int rotate, void* workspace, hipStream_t st);

}  // namespace bgg
