// Split-K row sums of the decode GEMVs: a launch that cuts K into P slices
// adds the slices' fp32 partial rows as 64-bit fixed-point integers with one
// device-scope atomic per row and token; the atomic also counts arrivals, and
// the arrival that completes a row writes y and clears its words.  Integer
// addition does not depend on the order of arrival, so y is deterministic.
// Every GEMV workspace starts with these words (fine words, then coarse
// words, 8 MiB each); every launch leaves the words it used at zero.
#pragma once
#include "bgg_device.h"

namespace bgg {

// ---------------------------------------------------------------------------
// Row words.  Word (slot m, row r) of a launch that splits K over P slices:
//   bits  0..55  sum over slices of (v + 2^48), v = rint(p 2^30) for a
//                partial |p| < 2^17 (else v = 0)
//   bit  56      a partial went to the coarse word (|p| >= 2^17)
//   bit  57      a partial was NaN (or inf)
//   bits 58..63  arrivals
// The coarse word (slot m, row r) holds sum rint(p 16) of the large partials
// (two's complement).  The workgroup whose atomic sees P - 1 arrivals writes y
// and sets both words back to zero.
// ---------------------------------------------------------------------------
constexpr int kRowWordRows = 65536;  // rows per slot; a launch covers at most this many
constexpr int kRowWordSlots = 16;
constexpr uint64_t kRowWordBytes = (uint64_t)kRowWordSlots * kRowWordRows * 8;
constexpr uint64_t kFineBias = 1ull << 48;
constexpr uint64_t kFineMask = (1ull << 56) - 1;
constexpr uint64_t kFlagCoarse = 1ull << 56;
constexpr uint64_t kFlagNaN = 1ull << 57;
constexpr int kArriveShift = 58;
constexpr int kMaxSlices = 63;
constexpr float kFineLimit = 131072.0f;  // 2^17
// a partial at or beyond 2^52 in magnitude (never reached from finite fp16
// inputs, whose partials stay below 2^48) or NaN marks the row NaN
constexpr float kCoarseLimit = 0x1p52f;

struct RowWords {
  unsigned long long* fine;  // kRowWordSlots x kRowWordRows
  long long* coarse;         // same shape
};

// The fine words of a workspace, then the coarse words.
inline __host__ __device__ RowWords row_words_of(void* workspace) {
  RowWords rw;
  rw.fine = reinterpret_cast<unsigned long long*>(workspace);
  rw.coarse = reinterpret_cast<long long*>((uint8_t*)workspace + kRowWordBytes);
  return rw;
}

// Phase 1 for partial p of (token slot m, local row lr): the rare cases
// (|p| >= 2^17: its value goes to the coarse word; NaN: a flag) touch the
// words now; the returned term is what the arrival adds to the row word.
__device__ __forceinline__ uint64_t partial_term(const RowWords& rw, int m, int64_t lr, float p) {
  if (fabsf(p) < kFineLimit)
    return (1ull << kArriveShift) + (uint64_t)((int64_t)llrint((double)p * 0x1p30) + (int64_t)kFineBias);
  unsigned long long* word = rw.fine + (int64_t)m * kRowWordRows + lr;
  if (!(fabsf(p) < kCoarseLimit)) {  // NaN or beyond the coarse range: NaN
    __hip_atomic_fetch_or(word, kFlagNaN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // the coarse add is complete before the flag is set (release), so the
    // last arrival, which reads the coarse word after seeing the flag, finds it
    __hip_atomic_fetch_add(rw.coarse + (int64_t)m * kRowWordRows + lr,
                           (long long)llrint((double)p * 16.0), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(word, kFlagCoarse, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  return (1ull << kArriveShift) + kFineBias;
}
__device__ __forceinline__ uint64_t arrive(const RowWords& rw, int m, int64_t lr, uint64_t term) {
  return __hip_atomic_fetch_add(rw.fine + (int64_t)m * kRowWordRows + lr, term, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
// Phase 2: the arrival that saw P - 1 before it holds the whole row: store y
// and clear the words.
__device__ __forceinline__ void finish_row(const RowWords& rw, int m, int64_t lr, int P, uint64_t old,
                                           uint64_t term, uint16_t* __restrict__ yrow) {
  if ((int)(old >> kArriveShift) != P - 1) return;
  const uint64_t tot = old + term;
  float y;
  if (tot & kFlagNaN) {
    y = __builtin_nanf("");
  } else {
    double v = (double)((int64_t)(tot & kFineMask) - (int64_t)P * (int64_t)kFineBias) * 0x1p-30;
    if (tot & kFlagCoarse) {
      long long* cw = rw.coarse + (int64_t)m * kRowWordRows + lr;
      const long long c = __hip_atomic_load(cw, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      v += (double)c * 0.0625;
      __hip_atomic_store(cw, 0ll, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    y = (float)v;
  }
  *yrow = f2h(y);
  __hip_atomic_store(rw.fine + (int64_t)m * kRowWordRows + lr, 0ull, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Partial p of (token slot m, local row lr) of a row cut into P slices, in
// one go: add it; the arrival that completes the row stores y at *yrow.
__device__ __forceinline__ void add_partial(const RowWords& rw, int m, int64_t lr, int P, float p,
                                            uint16_t* __restrict__ yrow) {
  const uint64_t term = partial_term(rw, m, lr, p);
  const uint64_t old = arrive(rw, m, lr, term);
  finish_row(rw, m, lr, P, old, term, yrow);
}

}  // namespace bgg
