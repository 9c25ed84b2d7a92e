/*
 * CPU ORACLE for the ternary Hadamard-rotated linear layer -- TEST
 * INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the GPU
 * library: no headers, tables, helpers or generators.
 *
 * Plain, slow and written to be checked by eye against the source pages:
 *   [A] allhereai.com/news/1346, "27B 模型压到 5.95GB，推理能力还保住 98%"
 *       - method paragraph: weights are -1/0/+1, one FP16 scale is shared by
 *         every 128 weights, and the matrix is stored after a block Hadamard
 *         rotation;
 *       - runtime paragraph: the runtime must apply the Hadamard transform
 *         to the activations;
 *       - packing paragraph: PTQ1_0 stores trits compactly, PQ2_0 puts each
 *         trit in a 2-bit slot.
 *   [B] 10100.com/article/156675786, "Bonsai 2，把27B压进6个G", section
 *       "它怎么做到的": the weights are rotated by a Hadamard transform
 *       before ternary rounding, so the input must get the matching
 *       transform at inference or the output is silently wrong.
 *   [C] wmrh.cn/news/471187, section "关键机制": five trits fit in eight
 *       bits (about 1.6 bits per trit); trits carry an FP16 group-wise scale.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - block = scale group = 128 consecutive weights along K, aligned at 0;
 *   - Sylvester (natural) order, no random signs, normalised by 1/sqrt(128);
 *     the matrix is symmetric and orthogonal, so the "inverse" transform of
 *     [B] and the "same" transform of [A] coincide;
 *   - PQ2_0: code = t + 1 in {0,1,2} (3 invalid), trit 4j+i of a row in bits
 *     2i..2i+1 of row byte j;
 *   - PTQ1_0: row byte j = sum_i (t_{5j+i} + 1) * 3^i, a continuous stream of
 *     ceil(K/5) bytes per row, trits past K padded with t = 0; bytes 243..255
 *     are invalid.
 *   - the sister formats the third page names by their effective bits per
 *     weight only ([C] opening summary: 1-bit weights {-1, +1} with an FP16
 *     group scale at about 1.125 bits per weight; section 后端支持现状: a
 *     ternary "Q2_0_g64" file form).  Read here as Q1_0: bit i of row byte j
 *     is weight 8j+i, 1 for +1 and 0 for -1, one FP16 scale per 128 weights
 *     (1 + 16/128 = 1.125 bits); Q2_0_g64: the PQ2_0 row stream with one
 *     FP16 scale per 64 weights (2 + 16/64 = 2.25 bits).  The activation
 *     transform keeps its 128-blocks for every format.
 *
 * All floating point is fp64; fp16 inputs are decoded exactly and fp16
 * outputs (the front end's scales) are rounded once, to nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_PQ2_0 1
#define ORACLE_PTQ1_0 2
#define ORACLE_Q1_0 3
#define ORACLE_Q2_0_G64 4
#define BLOCK 128

/* IEEE 754 binary16 -> double: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is subnormal (no implicit 1), 31 is inf/nan. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* Sylvester Hadamard matrix of order n (a power of two) by its recursion
 * H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]; row-major doubles. */
int oracle_sylvester(int n, double* H) {
  if (n < 1 || (n & (n - 1))) return -1;
  H[0] = 1.0;
  for (int m = 1; m < n; m *= 2) {
    for (int i = 0; i < m; ++i)
      for (int j = 0; j < m; ++j) {
        double h = H[i * n + j];
        H[i * n + (j + m)] = h;
        H[(i + m) * n + j] = h;
        H[(i + m) * n + (j + m)] = -h;
      }
  }
  return 0;
}

/* x'[m] = blockdiag(H_128 / sqrt(128)) x[m] for every row m: an explicit
 * dense 128x128 matrix times each 128-block of the row. [A], [B] */
int oracle_rotate(const uint16_t* x, int64_t M, int64_t K, double* xr) {
  if (K % BLOCK) return -1;
  double* H = (double*)malloc(sizeof(double) * BLOCK * BLOCK);
  if (!H) return -2;
  oracle_sylvester(BLOCK, H);
  const double norm = 1.0 / sqrt((double)BLOCK);
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m) {
    double blk[BLOCK];
    for (int64_t b = 0; b < K / BLOCK; ++b) {
      for (int i = 0; i < BLOCK; ++i) blk[i] = oracle_f16_to_f64(x[m * K + b * BLOCK + i]);
      for (int r = 0; r < BLOCK; ++r) {
        double acc = 0.0;
        for (int i = 0; i < BLOCK; ++i) acc += H[r * BLOCK + i] * blk[i];
        xr[m * K + b * BLOCK + r] = acc * norm;
      }
    }
  }
  free(H);
  return 0;
}

/* Bytes of one packed row (canonical layout). [A] packing, [C] */
int64_t oracle_row_bytes(int fmt, int64_t K) {
  if (fmt == ORACLE_PQ2_0 || fmt == ORACLE_Q2_0_G64) return (K + 3) / 4;
  if (fmt == ORACLE_PTQ1_0) return (K + 4) / 5;
  if (fmt == ORACLE_Q1_0) return (K + 7) / 8;
  return -1;
}

/* Weights that share one fp16 scale: 128 [A method], 64 for Q2_0_g64. */
int64_t oracle_scale_group(int fmt) {
  if (fmt == ORACLE_PQ2_0 || fmt == ORACLE_PTQ1_0 || fmt == ORACLE_Q1_0) return BLOCK;
  if (fmt == ORACLE_Q2_0_G64) return 64;
  return -1;
}

/* Bytes of a whole N x K matrix: packed weights plus one fp16 per scale
 * group. [A] */
int64_t oracle_format_bytes(int fmt, int64_t N, int64_t K) {
  int64_t rb = oracle_row_bytes(fmt, K), group = oracle_scale_group(fmt);
  if (rb < 0 || group < 0 || K % BLOCK) return -1;
  return N * rb + N * (K / group) * 2;
}

/* Canonical packing of trits T[N][K] into out[N][row_bytes]. Returns 0, or
 * -1 for a bad format, -3 for a value outside {-1,0,1} (outside {-1,1} for
 * Q1_0). */
int oracle_pack(int fmt, const int8_t* T, int64_t N, int64_t K, uint8_t* out) {
  int64_t rb = oracle_row_bytes(fmt, K);
  if (rb < 0) return -1;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t j = 0; j < rb; ++j) {
      unsigned byte = 0;
      if (fmt == ORACLE_PQ2_0 || fmt == ORACLE_Q2_0_G64) {
        for (int i = 0; i < 4; ++i) {
          int64_t k = 4 * j + i;
          int t = k < K ? T[n * K + k] : 0;
          if (t < -1 || t > 1) return -3;
          byte |= (unsigned)(t + 1) << (2 * i);
        }
      } else if (fmt == ORACLE_Q1_0) {
        for (int i = 0; i < 8; ++i) {
          int64_t k = 8 * j + i;
          int t = k < K ? T[n * K + k] : -1;
          if (t != -1 && t != 1) return -3;
          if (t == 1) byte |= 1u << i;
        }
      } else {
        unsigned pow3 = 1;
        for (int i = 0; i < 5; ++i) {
          int64_t k = 5 * j + i;
          int t = k < K ? T[n * K + k] : 0;
          if (t < -1 || t > 1) return -3;
          byte += (unsigned)(t + 1) * pow3;
          pow3 *= 3;
        }
      }
      out[n * rb + j] = (uint8_t)byte;
    }
  }
  return 0;
}

/* Inverse of oracle_pack. Returns 0, or -4 for an invalid byte (a PQ2_0 code
 * of 3, a PTQ1_0 byte of 243 or more). */
int oracle_unpack(int fmt, const uint8_t* packed, int64_t N, int64_t K, int8_t* T) {
  int64_t rb = oracle_row_bytes(fmt, K);
  if (rb < 0) return -1;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t j = 0; j < rb; ++j) {
      unsigned byte = packed[n * rb + j];
      if (fmt == ORACLE_Q1_0) {
        for (int i = 0; i < 8; ++i) {
          int64_t k = 8 * j + i;
          if (k < K) T[n * K + k] = (int8_t)(((byte >> i) & 1u) ? 1 : -1);
        }
      } else if (fmt == ORACLE_PQ2_0 || fmt == ORACLE_Q2_0_G64) {
        for (int i = 0; i < 4; ++i) {
          unsigned code = (byte >> (2 * i)) & 3u;
          if (code == 3) return -4;
          int64_t k = 4 * j + i;
          if (k < K) T[n * K + k] = (int8_t)((int)code - 1);
        }
      } else {
        if (byte >= 243) return -4;
        for (int i = 0; i < 5; ++i) {
          unsigned digit = byte % 3;
          byte /= 3;
          int64_t k = 5 * j + i;
          if (k < K) T[n * K + k] = (int8_t)((int)digit - 1);
        }
      }
    }
  }
  return 0;
}

/* y[m][n] = sum_k S[n][k/group] * T[n][k] * xr[m][k] in fp64; S is fp16
 * with K/group scales per row.  xr holds activations already in rotated
 * coordinates. [A] */
int oracle_matvec_group(const int8_t* T, const uint16_t* S, const double* xr, int64_t M,
                        int64_t N, int64_t K, int64_t group, double* y) {
  if (group < 1 || K % group) return -1;
  const int64_t G = K / group;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += oracle_f16_to_f64(S[n * G + k / group]) * (double)T[n * K + k] * xr[m * K + k];
      y[m * N + n] = acc;
    }
  }
  return 0;
}

/* The same with one scale per 128 weights [A method paragraph]. */
int oracle_matvec(const int8_t* T, const uint16_t* S, const double* xr, int64_t M, int64_t N,
                  int64_t K, double* y) {
  if (K % BLOCK) return -1;
  return oracle_matvec_group(T, S, xr, M, N, K, BLOCK, y);
}

/* The whole layer from the stored form: unpack the canonical bytes, rotate
 * the fp16 activations (unless rotate == 0, when x is already rotated), and
 * take the fp64 products. [A], [B] */
int oracle_linear(int fmt, const uint8_t* packed, const uint16_t* S, const uint16_t* x, int64_t M,
                  int64_t N, int64_t K, int rotate, double* y) {
  if (K % BLOCK) return -1;
  int8_t* T = (int8_t*)malloc((size_t)(N * K > 0 ? N * K : 1));
  double* xr = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
  int rc = (T && xr) ? 0 : -2;
  if (!rc) rc = oracle_unpack(fmt, packed, N, K, T);
  if (!rc) {
    if (rotate)
      rc = oracle_rotate(x, M, K, xr);
    else
      for (int64_t i = 0; i < M * K; ++i) xr[i] = oracle_f16_to_f64(x[i]);
  }
  if (!rc) rc = oracle_matvec_group(T, S, xr, M, N, K, oracle_scale_group(fmt), y);
  free(T);
  free(xr);
  return rc;
}

/* double -> IEEE 754 binary16 bits, rounded to nearest with ties to even:
 * the value is written as m * 2^q with the integer m of the target's 11
 * significant bits (fewer for subnormals, whose exponent is pinned at -24),
 * the remainder decides the rounding, and a carry out of the significand
 * moves to the next binade; magnitudes that round past 65504 become inf. */
uint16_t oracle_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (isinf(v)) return (uint16_t)(sign | 0x7C00);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
  int q = e - 11;               /* 2^q = weight of the last kept bit */
  if (q < -24) q = -24;         /* subnormal range: fixed step 2^-24 */
  double scaled = ldexp(a, -q); /* exact: a power-of-two scaling */
  double m = floor(scaled);
  double rem = scaled - m;      /* exact: the fraction of a double */
  if (rem > 0.5 || (rem == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;
  if (m >= 2048.0) {            /* carried into the next binade */
    m /= 2.0;
    q += 1;
  }
  if (m < 1024.0)               /* subnormal (q == -24): exponent field 0 */
    return (uint16_t)(sign | (uint16_t)m);
  int ef = q + 25;              /* value = m * 2^q = (1 + f/1024) 2^(ef - 15) */
  if (ef >= 31) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | (uint16_t)(ef << 10) | (uint16_t)((int)m - 1024));
}

/* Offline front end: float weights W [N][K] -> trits T [N][K] and fp16
 * scales S [N][K/128] in the coordinates the layer stores.
 *   1. rotate: every 128-block of a row becomes H_128/sqrt(128) times that
 *      block (the weight side of the rotation: y = W x = (W Hn)(Hn x) with
 *      Hn symmetric and orthogonal, so the stored rows are W Hn) [A method
 *      paragraph, B "它怎么做到的"];
 *   2. scale of each 128-group: the mean magnitude of its rotated weights,
 *      rounded to fp16 (a reading: the pages give no scale rule);
 *   3. ternary rounding: each rotated weight goes to the nearest of -s, 0,
 *      +s, i.e. t = sign(w') when |w'| > s/2 and 0 otherwise (a tie at s/2
 *      goes to 0, the even neighbour of rint) [B "它怎么做到的"].
 * Returns 0, -1 for K not a multiple of 128, -2 when out of memory. */
int oracle_ternarize(const float* W, int64_t N, int64_t K, int8_t* T, uint16_t* S) {
  if (K % BLOCK || N < 0) return -1;
  double* H = (double*)malloc(sizeof(double) * BLOCK * BLOCK);
  if (!H) return -2;
  oracle_sylvester(BLOCK, H);
  const double norm = 1.0 / sqrt((double)BLOCK);
  const int64_t G = K / BLOCK;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double blk[BLOCK], wr[BLOCK];
    for (int64_t b = 0; b < G; ++b) {
      for (int i = 0; i < BLOCK; ++i) blk[i] = (double)W[n * K + b * BLOCK + i];
      double mag = 0.0;
      for (int r = 0; r < BLOCK; ++r) {
        double acc = 0.0;
        for (int i = 0; i < BLOCK; ++i) acc += H[r * BLOCK + i] * blk[i];
        wr[r] = acc * norm;
        mag += fabs(wr[r]);
      }
      const uint16_t sh = oracle_f64_to_f16(mag / BLOCK);
      const double s = oracle_f16_to_f64(sh);
      S[n * G + b] = sh;
      for (int r = 0; r < BLOCK; ++r) {
        int8_t t = 0;
        if (fabs(wr[r]) > 0.5 * s) t = wr[r] > 0.0 ? 1 : -1;
        T[n * K + b * BLOCK + r] = t;
      }
    }
  }
  free(H);
  return 0;
}

/* Threads the OpenMP loops above run on (for reporting only). */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Run the OpenMP loops on n threads from now on (n >= 1; timing only). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
