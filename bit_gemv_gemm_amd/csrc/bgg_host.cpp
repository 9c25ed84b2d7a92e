// Host side of libbgg: descriptors, packing into the device layout,
// validation, status strings.  No GPU work happens here.
//
// Packings follow allhereai.com/news/1346 (packing paragraph: PTQ1_0 compact
// trits, PQ2_0 one trit per 2-bit slot) and wmrh.cn/news/471187 (section
// 关键机制: five trits per byte); the per-128 fp16 scale follows the method
// paragraph of the first page.  The sister formats Q1_0 (1-bit, about 1.125
// bits per weight: opening summary of the second page) and Q2_0_g64 (named
// in its section 后端支持现状) are laid out as this library reads them: a
// sign bit per weight with a scale per 128, and the PQ2_0 stream with a
// scale per 64.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "bgg_internal.h"

namespace bgg {

static thread_local char g_last_error[512] = "";

bgg_status fail(bgg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = 0; }

bgg_status check_desc(const bgg_weights_desc* d) {
  if (!d) return fail(BGG_ERR_NULL, "descriptor is NULL");
  bgg_weights_desc ref;
  if (d->magic != BGG_DESC_MAGIC || d->version != BGG_DESC_VERSION)
    return fail(BGG_ERR_DESC, "descriptor magic/version mismatch");
  if (bgg_describe(d->format, d->N, d->K, &ref) != BGG_OK)
    return fail(BGG_ERR_DESC, "descriptor fields describe no valid matrix");
  if (std::memcmp(&ref, d, sizeof ref) != 0)
    return fail(BGG_ERR_DESC, "descriptor fields were modified after bgg_describe");
  return BGG_OK;
}

}  // namespace bgg

using namespace bgg;

// Base-3 byte of five trits (t + 1 as little-endian digits) and the 2-bit
// code byte of four trits, as the canonical row stream defines them.
static inline uint8_t ptq1_byte(const int8_t* t, int64_t k0, int64_t K) {
  unsigned v = 0, p = 1;
  for (int i = 0; i < 5; ++i, p *= 3) v += (unsigned)((k0 + i < K ? t[k0 + i] : 0) + 1) * p;
  return (uint8_t)v;
}

static inline uint8_t pq2_byte(const int8_t* t, int64_t k0, int64_t K) {
  unsigned v = 0;
  for (int i = 0; i < 4; ++i) v |= (unsigned)((k0 + i < K ? t[k0 + i] : 0) + 1) << (2 * i);
  return (uint8_t)v;
}

// Eight signs (bit i = weight k0+i, 1 for +1); weights past K are -1.
static inline uint8_t q1_byte(const int8_t* t, int64_t k0, int64_t K) {
  unsigned v = 0;
  for (int i = 0; i < 8; ++i)
    if (k0 + i < K && t[k0 + i] == 1) v |= 1u << i;
  return (uint8_t)v;
}

static inline bool f16_finite(uint16_t h) { return ((h >> 10) & 31) != 31; }

static inline bool pq2_stream(int32_t fmt) { return fmt == BGG_FMT_PQ2_0 || fmt == BGG_FMT_Q2_0_G64; }

// The byte of padding rows and columns: zero trits, or all -1 (Q1_0 has no
// zero weight; its padding rows have zero scales).
static inline uint8_t zero_byte(int32_t fmt) {
  return pq2_stream(fmt) ? 0x55 : fmt == BGG_FMT_PTQ1_0 ? 121 : 0x00;
}

extern "C" {

bgg_status bgg_describe(int32_t format, int64_t N, int64_t K, bgg_weights_desc* out) {
  if (!out) return fail(BGG_ERR_NULL, "bgg_describe: out is NULL");
  if (format != BGG_FMT_PQ2_0 && format != BGG_FMT_PTQ1_0 && format != BGG_FMT_Q1_0 &&
      format != BGG_FMT_Q2_0_G64)
    return fail(BGG_ERR_FORMAT, "bgg_describe: unknown format %d", (int)format);
  if (N < 1 || K < BGG_GROUP || K % BGG_GROUP != 0 || N > (int64_t(1) << 31) ||
      K > (int64_t(1) << 28))
    return fail(BGG_ERR_SHAPE, "bgg_describe: need N >= 1 and K a positive multiple of 128 "
                               "(got N=%lld K=%lld)", (long long)N, (long long)K);
  bgg_weights_desc d;
  std::memset(&d, 0, sizeof d);
  d.magic = BGG_DESC_MAGIC;
  d.version = BGG_DESC_VERSION;
  d.format = format;
  d.row_tile = BGG_ROW_TILE;
  d.N = N;
  d.K = K;
  d.groups = K / BGG_GROUP;
  d.row_tiles = (N + BGG_ROW_TILE - 1) / BGG_ROW_TILE;
  d.row_bytes = pq2_stream(format) ? (K + 3) / 4 : format == BGG_FMT_PTQ1_0 ? (K + 4) / 5 : K / 8;
  d.chunks = (d.row_bytes + BGG_CHUNK - 1) / BGG_CHUNK;
  d.trit_bytes = (uint64_t)d.row_tiles * d.chunks * BGG_ROW_TILE * BGG_CHUNK;
  d.scale_offset = (d.trit_bytes + 255) & ~uint64_t(255);
  d.scale_group = format == BGG_FMT_Q2_0_G64 ? 64 : BGG_GROUP;
  d.scales = K / d.scale_group;
  d.scale_bytes = (uint64_t)d.row_tiles * d.scales * BGG_ROW_TILE * 2;
  d.total_bytes = d.scale_offset + d.scale_bytes + BGG_READ_SLACK;
  d.format_bytes = (uint64_t)N * d.row_bytes + (uint64_t)N * d.scales * 2;
  *out = d;
  clear_error();
  return BGG_OK;
}

// Writes row r's canonical byte stream (from `row_stream`) and scales into
// the tiled layout; rows past N are filled with zero trits and zero scales.
// Rows are split over a few host threads (std::thread; the library links no
// OpenMP runtime so it can share a process with any other).
static void place_rows(const bgg_weights_desc* d, uint8_t* dst,
                       void (*row_stream)(const void*, int64_t, uint8_t*), const void* ctx,
                       const uint16_t* scales) {
  const int64_t C = d->chunks, G = d->scales;
  const int64_t padded_row = C * BGG_CHUNK;
  const int64_t rows = d->row_tiles * BGG_ROW_TILE;
  uint16_t* sdst = reinterpret_cast<uint16_t*>(dst + d->scale_offset);
  std::memset(dst + d->trit_bytes, 0, d->scale_offset - d->trit_bytes);
  std::memset(dst + d->scale_offset + d->scale_bytes, 0, BGG_READ_SLACK);
  auto work = [&](int64_t r0, int64_t r1) {
    std::vector<uint8_t> row(padded_row);
    for (int64_t r = r0; r < r1; ++r) {
      std::memset(row.data(), zero_byte(d->format), padded_row);
      if (r < d->N) row_stream(ctx, r, row.data());
      const int64_t t = r / BGG_ROW_TILE, l = r % BGG_ROW_TILE;
      for (int64_t c = 0; c < C; ++c)
        std::memcpy(dst + ((t * C + c) * BGG_ROW_TILE + l) * BGG_CHUNK, row.data() + c * BGG_CHUNK,
                    BGG_CHUNK);
      for (int64_t g = 0; g < G; ++g)
        sdst[(t * G + g) * BGG_ROW_TILE + l] = r < d->N ? scales[r * G + g] : 0;
    }
  };
  const int64_t bytes = rows * (padded_row + 2 * G);
  unsigned nt = bytes < (int64_t(1) << 22) ? 1u : std::min(16u, std::max(1u, std::thread::hardware_concurrency()));
  if (nt == 1) {
    work(0, rows);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (rows + nt - 1) / nt;
  for (unsigned i = 0; i < nt; ++i) {
    const int64_t r0 = i * per, r1 = std::min(rows, r0 + per);
    if (r0 < r1) pool.emplace_back(work, r0, r1);
  }
  for (auto& th : pool) th.join();
}

struct TritCtx {
  const int8_t* trits;
  int64_t K;
  int32_t fmt;
  int64_t row_bytes;
};

static void trit_row_stream(const void* p, int64_t r, uint8_t* out) {
  const TritCtx* c = static_cast<const TritCtx*>(p);
  const int8_t* t = c->trits + r * c->K;
  if (pq2_stream(c->fmt))
    for (int64_t j = 0; j < c->row_bytes; ++j) out[j] = pq2_byte(t, 4 * j, c->K);
  else if (c->fmt == BGG_FMT_PTQ1_0)
    for (int64_t j = 0; j < c->row_bytes; ++j) out[j] = ptq1_byte(t, 5 * j, c->K);
  else
    for (int64_t j = 0; j < c->row_bytes; ++j) out[j] = q1_byte(t, 8 * j, c->K);
}

struct CanonCtx {
  const uint8_t* bytes;
  int64_t row_bytes;
};

static void canonical_row_stream(const void* p, int64_t r, uint8_t* out) {
  const CanonCtx* c = static_cast<const CanonCtx*>(p);
  std::memcpy(out, c->bytes + r * c->row_bytes, c->row_bytes);
}

bgg_status bgg_pack_weights(const bgg_weights_desc* d, const int8_t* trits,
                            const uint16_t* scales, void* packed) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!trits || !scales || !packed) return fail(BGG_ERR_NULL, "bgg_pack_weights: NULL buffer");
  const int64_t NK = d->N * d->K, NG = d->N * d->scales;
  const int lo = -1, hi = 1;
  const bool signs = d->format == BGG_FMT_Q1_0;  // {-1, +1} only
  for (int64_t i = 0; i < NK; ++i)
    if (trits[i] < lo || trits[i] > hi || (signs && trits[i] == 0))
      return fail(BGG_ERR_TRIT, "bgg_pack_weights: weight %d at row %lld col %lld", (int)trits[i],
                  (long long)(i / d->K), (long long)(i % d->K));
  for (int64_t i = 0; i < NG; ++i)
    if (!f16_finite(scales[i]))
      return fail(BGG_ERR_SCALE, "bgg_pack_weights: scale %lld is not finite", (long long)i);
  TritCtx ctx{trits, d->K, d->format, d->row_bytes};
  place_rows(d, static_cast<uint8_t*>(packed), trit_row_stream, &ctx, scales);
  clear_error();
  return BGG_OK;
}

static bool canonical_byte_ok(int32_t fmt, uint8_t b) {
  if (fmt == BGG_FMT_PTQ1_0) return b < 243;
  if (fmt == BGG_FMT_Q1_0) return true;
  for (int i = 0; i < 4; ++i)
    if (((b >> (2 * i)) & 3) == 3) return false;
  return true;
}

bgg_status bgg_repack_canonical(const bgg_weights_desc* d, const uint8_t* canonical,
                                const uint16_t* scales, void* packed) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!canonical || !scales || !packed)
    return fail(BGG_ERR_NULL, "bgg_repack_canonical: NULL buffer");
  const int64_t nb = d->N * d->row_bytes, NG = d->N * d->scales;
  for (int64_t i = 0; i < nb; ++i)
    if (!canonical_byte_ok(d->format, canonical[i]))
      return fail(BGG_ERR_PACKED_BYTE, "bgg_repack_canonical: invalid byte 0x%02x at row %lld",
                  canonical[i], (long long)(i / d->row_bytes));
  for (int64_t i = 0; i < NG; ++i)
    if (!f16_finite(scales[i]))
      return fail(BGG_ERR_SCALE, "bgg_repack_canonical: scale %lld is not finite", (long long)i);
  CanonCtx ctx{canonical, d->row_bytes};
  place_rows(d, static_cast<uint8_t*>(packed), canonical_row_stream, &ctx, scales);
  clear_error();
  return BGG_OK;
}

bgg_status bgg_validate_packed(const bgg_weights_desc* d, const void* packed) {
  bgg_status st = check_desc(d);
  if (st) return st;
  if (!packed) return fail(BGG_ERR_NULL, "bgg_validate_packed: NULL buffer");
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  const int64_t C = d->chunks, G = d->scales, rows = d->row_tiles * BGG_ROW_TILE;
  const uint8_t zb = zero_byte(d->format);
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t t = r / BGG_ROW_TILE, l = r % BGG_ROW_TILE;
    for (int64_t j = 0; j < C * BGG_CHUNK; ++j) {
      uint8_t b = p[((t * C + j / BGG_CHUNK) * BGG_ROW_TILE + l) * BGG_CHUNK + j % BGG_CHUNK];
      if (!canonical_byte_ok(d->format, b))
        return fail(BGG_ERR_PACKED_BYTE, "bgg_validate_packed: invalid byte 0x%02x, row %lld "
                                         "byte %lld", b, (long long)r, (long long)j);
      if ((r >= d->N || j >= d->row_bytes) && b != zb)
        return fail(BGG_ERR_PACKED_BYTE, "bgg_validate_packed: padding byte 0x%02x at row %lld "
                                         "byte %lld is not zero trits", b, (long long)r,
                    (long long)j);
    }
  }
  const uint16_t* s = reinterpret_cast<const uint16_t*>(p + d->scale_offset);
  for (int64_t i = 0; i < d->row_tiles * G * BGG_ROW_TILE; ++i) {
    if (!f16_finite(s[i])) return fail(BGG_ERR_SCALE, "bgg_validate_packed: scale not finite");
    const int64_t r = (i / (G * BGG_ROW_TILE)) * BGG_ROW_TILE + i % BGG_ROW_TILE;
    if (r >= d->N && s[i] != 0) return fail(BGG_ERR_SCALE, "bgg_validate_packed: padding scale");
  }
  for (uint64_t i = d->scale_offset + d->scale_bytes; i < d->total_bytes; ++i)
    if (p[i] != 0) return fail(BGG_ERR_BUFFER, "bgg_validate_packed: slack byte is not zero");
  clear_error();
  return BGG_OK;
}

const char* bgg_status_string(int32_t s) {
  switch (s) {
    case BGG_OK: return "ok";
    case BGG_ERR_NULL: return "null pointer";
    case BGG_ERR_FORMAT: return "unknown or unsupported format";
    case BGG_ERR_SHAPE: return "bad shape";
    case BGG_ERR_TRIT: return "trit outside {-1,0,1}";
    case BGG_ERR_PACKED_BYTE: return "invalid packed byte";
    case BGG_ERR_BUFFER: return "buffer too small or misaligned";
    case BGG_ERR_DESC: return "bad descriptor";
    case BGG_ERR_HIP: return "HIP runtime error";
    case BGG_ERR_SCALE: return "scale is not a finite fp16";
    default: return "unknown status";
  }
}

const char* bgg_last_error(void) { return g_last_error; }

uint32_t bgg_abi_version(void) { return BGG_DESC_VERSION; }

}  // extern "C"
