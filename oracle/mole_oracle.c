/*
 * mole_oracle.c -- plain, slow CPU oracle for the Mixture-of-Lookup-Experts
 * (MoLE) inference hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant generator with the HIP library; the two meet only in the seeded
 * synthetic inputs.
 *
 * Everything is computed in fp64 from the stored input values (fp32 or bf16
 * bit patterns, upcast exactly), with plain loops in the order the
 * definitions are written.  The only exception is the NF3 encoder, whose
 * integer decisions are taken in fp32 exactly as the encoding is specified
 * (absmax in fp32, fp16 round-to-nearest-even scale, one fp32 multiply per
 * threshold, strict compare).
 *
 * Sources (web pages on MoLE; their formulas were lost in extraction, so the
 * definitions below are the plainest reading the surrounding text supports):
 *  - "ICML 2025 Spotlight | MoLE" article, section "推理阶段" (inference):
 *    the embedding weight matrix is fed to every routed expert, giving the
 *    complete token-id -> expert-output table; at inference the outputs are
 *    fetched by token id.                      -> oracle_build_lut_rows,
 *                                                 oracle_lookup_combine
 *  - same article, section "训练阶段" (training): all routed experts are
 *    active; the router sees the previous layer's output.
 *                                              -> oracle_router_gates
 *  - same article, section "实验结果" (results): the table still works when
 *    compressed to 3 bits, e.g. NF3.           -> oracle_pack_nf3 and friends
 *
 * Layouts (row-major, element counts):
 *   emb    [V][D]        w_up  [N][F][D]   (expert e: u = W_up[e] . x)
 *   w_down [N][D][F]     w_r   [N][D]      (router logits z = W_r . h)
 *   lut    [V][N][D]     h     [T][D]      ids [T] (int64)   y [T][D]
 *   codes  [V][N][3D/8] (LSB-first 3-bit stream per row)
 *   scales [V][N][D/64] (fp16 bit patterns)
 *
 * Parity pins: every function here is pinned by tests that do not call this
 * file's own arithmetic (numpy/scipy library routines, closed forms,
 * brute force on tiny inputs, hand-worked bit patterns).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_OK = 0, OR_ERR_ARG = -1, OR_ERR_ID = -2, OR_ERR_MEM = -3 };

/* Exact upcast of one stored element to double. */
static double load_elem(const void* p, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int dtype_ok(int dtype) { return dtype == OR_F32 || dtype == OR_BF16; }

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* GELU in its exact form: u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)). */
double oracle_gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }

/*
 * LUT reparameterisation (inference section: every routed expert is run on
 * the embedding weight matrix).  For each listed vocabulary row v and expert
 * e:  u[f] = sum_d Emb[v][d] * W_up[e][f][d];  g[f] = GELU(u[f]);
 *     out[r][e][d] = sum_f g[f] * W_down[e][d][f].
 * out is [nrows][N][D] fp64.
 */
int oracle_build_lut_rows(const void* emb, const void* w_up, const void* w_down,
                          int dtype, int64_t V, int64_t D, int64_t F, int64_t N,
                          const int64_t* rows, int64_t nrows, double* out,
                          int nthreads) {
  if (!dtype_ok(dtype) || V < 0 || D <= 0 || F <= 0 || N <= 0 || nrows < 0)
    return OR_ERR_ARG;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= V) return OR_ERR_ID;
  set_threads(nthreads);
  int failed = 0;
#pragma omp parallel
  {
    double* g = (double*)malloc((size_t)F * sizeof(double));
    if (!g) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for collapse(2) schedule(dynamic)
    for (int64_t r = 0; r < nrows; ++r) {
      for (int64_t e = 0; e < N; ++e) {
        if (!g) continue;
        const int64_t v = rows[r];
        for (int64_t f = 0; f < F; ++f) {
          double u = 0.0;
          for (int64_t d = 0; d < D; ++d)
            u += load_elem(emb, dtype, v * D + d) *
                 load_elem(w_up, dtype, (e * F + f) * D + d);
          g[f] = oracle_gelu(u);
        }
        for (int64_t d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int64_t f = 0; f < F; ++f)
            acc += g[f] * load_elem(w_down, dtype, (e * D + d) * F + f);
          out[(r * N + e) * D + d] = acc;
        }
      }
    }
    free(g);
  }
  return failed ? OR_ERR_MEM : OR_OK;
}

/*
 * Router gates (training section: router on the contextual hidden state,
 * every routed expert active, so a dense softmax over all N, no top-k):
 *   z[e] = sum_d h[t][d] * W_r[e][d];  g = softmax(z) (max-subtracted).
 * gates is [T][N] fp64.
 */
int oracle_router_gates(const void* h, const void* w_r, int dtype, int64_t T,
                        int64_t D, int64_t N, double* gates, int nthreads) {
  if (!dtype_ok(dtype) || T < 0 || D <= 0 || N <= 0) return OR_ERR_ARG;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* g = gates + t * N;
    double zmax = -INFINITY;
    for (int64_t e = 0; e < N; ++e) {
      double z = 0.0;
      for (int64_t d = 0; d < D; ++d)
        z += load_elem(h, dtype, t * D + d) * load_elem(w_r, dtype, e * D + d);
      g[e] = z;
      if (z > zmax) zmax = z;
    }
    double sum = 0.0;
    for (int64_t e = 0; e < N; ++e) {
      g[e] = exp(g[e] - zmax);
      sum += g[e];
    }
    for (int64_t e = 0; e < N; ++e) g[e] /= sum;
  }
  return OR_OK;
}

/*
 * Lookup-combine (inference section: fetch each token's expert outputs by
 * token id, weight them with the router):
 *   y[t][d] = sum_e g[t][e] * LUT[id_t][e][d].
 * lut_dtype may differ from the dtype of h and W_r.  y is [T][D] fp64.
 */
int oracle_lookup_combine(const int64_t* ids, const void* h, const void* w_r,
                          int dtype_hw, const void* lut, int dtype_lut,
                          int64_t T, int64_t V, int64_t D, int64_t N, double* y,
                          int nthreads) {
  if (!dtype_ok(dtype_hw) || !dtype_ok(dtype_lut) || T < 0 || V <= 0 ||
      D <= 0 || N <= 0)
    return OR_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return OR_ERR_ID;
  double* gates = (double*)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
  if (!gates) return OR_ERR_MEM;
  int rc = oracle_router_gates(h, w_r, dtype_hw, T, D, N, gates, nthreads);
  if (rc == OR_OK) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const int64_t v = ids[t];
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t e = 0; e < N; ++e)
          acc += gates[t * N + e] * load_elem(lut, dtype_lut, (v * N + e) * D + d);
        y[t * D + d] = acc;
      }
    }
  }
  free(gates);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* NF3: 3-bit NormalFloat codes, blocks of 64 along D, one fp16 absmax scale. */
/* ------------------------------------------------------------------------ */

/* Standard normal CDF from the C library's complementary error function. */
static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Inverse standard normal CDF by plain bisection (p in (0,1)); 200 halvings
 * of [-40, 40] reach the resolution of double. */
double oracle_normal_ppf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/*
 * The NormalFloat construction (Dettmers et al., QLoRA, 2023) at k = 3 bits:
 * with delta = 1/2 (1/(2*7) + 1/(2*8)) and p* = 1 - delta, take
 * Phi^-1 at 2^(k-1)+1 = 5 evenly spaced probabilities from p* down to 1/2
 * (dropping 1/2) for the 4 positive levels, -Phi^-1 at 2^(k-1) = 4 evenly
 * spaced probabilities from p* to 1/2 (dropping 1/2) for the 3 negative
 * levels, add one exact zero, normalise by the largest value, sort, and round
 * each level to fp32.
 */
void oracle_nf3_levels(float out[8]) {
  const double pstar = 1.0 - 0.5 * (1.0 / 14.0 + 1.0 / 16.0);
  double v[8];
  int n = 0;
  for (int i = 0; i < 4; ++i)            /* linspace(p*, 0.5, 5)[0..3] */
    v[n++] = oracle_normal_ppf(pstar + (0.5 - pstar) * (double)i / 4.0);
  for (int i = 0; i < 3; ++i)            /* linspace(p*, 0.5, 4)[0..2] */
    v[n++] = -oracle_normal_ppf(pstar + (0.5 - pstar) * (double)i / 3.0);
  v[n++] = 0.0;
  double vmax = 0.0;
  for (int i = 0; i < 8; ++i) if (v[i] > vmax) vmax = v[i];
  for (int i = 0; i < 8; ++i) v[i] /= vmax;
  for (int i = 1; i < 8; ++i)            /* insertion sort, ascending */
    for (int j = i; j > 0 && v[j - 1] > v[j]; --j) {
      double tmp = v[j]; v[j] = v[j - 1]; v[j - 1] = tmp;
    }
  for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}

/* Decision thresholds: fp32 round-to-nearest-even of the exact midpoint of
 * two neighbouring fp32 levels (the sum of two floats is exact in double). */
void oracle_nf3_midpoints(float out[7]) {
  float lv[8];
  oracle_nf3_levels(lv);
  for (int j = 0; j < 7; ++j) out[j] = (float)(((double)lv[j] + (double)lv[j + 1]) / 2.0);
}

/* IEEE binary32 -> binary16, round to nearest, ties to even, by bit
 * manipulation (finite, non-negative inputs are all the encoder needs, but
 * the sign is carried for completeness; overflow gives infinity). */
uint16_t oracle_f32_to_f16_rne(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  const uint32_t sign = (b >> 16) & 0x8000u;
  const uint32_t ex = (b >> 23) & 0xFFu;
  uint32_t man = b & 0x7FFFFFu;
  if (ex == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
  int e = (int)ex - 127;             /* unbiased exponent */
  if (ex == 0) return (uint16_t)sign; /* f32 subnormals are far below f16's range */
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  uint32_t full = man | 0x800000u;    /* 24-bit significand, value = full * 2^(e-23) */
  int shift;                          /* bits to drop from the 24-bit significand */
  uint32_t hexp;
  if (e >= -14) { shift = 13; hexp = (uint32_t)(e + 15); }
  else {                              /* f16 subnormal: value = m * 2^-24 */
    shift = 13 + (-14 - e);
    hexp = 0;
    if (shift > 25) return (uint16_t)sign; /* below half of the smallest subnormal */
  }
  uint32_t keep = full >> shift;
  uint32_t rem = full & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (keep & 1u))) keep += 1u;
  uint32_t result;
  if (hexp == 0) {
    result = keep;                    /* may carry into the smallest normal: still right */
  } else {
    result = (hexp << 10) + (keep - 0x400u); /* keep holds the implicit bit */
    if (keep == 0x800u) result = ((hexp + 1u) << 10);
  }
  if (result >= 0x7C00u) result = 0x7C00u;
  return (uint16_t)(sign | result);
}

float oracle_f16_to_f32(uint16_t hbits) {
  const double sign = (hbits & 0x8000u) ? -1.0 : 1.0;
  const int ex = (hbits >> 10) & 0x1F;
  const int man = hbits & 0x3FF;
  double v;
  if (ex == 0) v = ldexp((double)man, -24);
  else if (ex == 31) v = man ? NAN : INFINITY;
  else v = ldexp((double)(man + 1024), ex - 25);
  return (float)(sign * v);
}

/* Bit i of a little-endian byte stream. */
static void put_bit(uint8_t* row, int64_t bit, int value) {
  if (value) row[bit >> 3] = (uint8_t)(row[bit >> 3] | (1u << (bit & 7)));
}
static int get_bit(const uint8_t* row, int64_t bit) {
  return (row[bit >> 3] >> (bit & 7)) & 1;
}

/*
 * Encode a [rows][D] table (rows = V*N) into NF3:
 *  1. a  = max |x| over a block of 64 consecutive elements of one row (fp32);
 *  2. s  = fp16_rne(min(a, 65504)); scales[row][b] = s;
 *  3. code = number of j in 0..6 with x > fp32(mid[j] * float(s)), strict,
 *     so an exact tie goes to the lower code; when s == 0 every code is 3
 *     (the zero level);
 *  4. code i of the row occupies bits [3i, 3i+3) of the row's little-endian
 *     bit stream (LSB first); a row is 3D/8 bytes.
 * n_saturated (may be NULL) receives the number of blocks whose absmax
 * exceeded 65504.  D must be a positive multiple of 64.
 */
int oracle_pack_nf3(const void* lut, int dtype, int64_t rows, int64_t D,
                    uint8_t* codes, uint16_t* scales, int64_t* n_saturated,
                    int nthreads) {
  if (!dtype_ok(dtype) || rows < 0 || D <= 0 || D % 64 != 0) return OR_ERR_ARG;
  float mid[7];
  oracle_nf3_midpoints(mid);
  const int64_t row_bytes = 3 * D / 8, nblk = D / 64;
  int64_t nsat = 0;
  set_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(+ : nsat)
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* crow = codes + r * row_bytes;
    memset(crow, 0, (size_t)row_bytes);
    for (int64_t b = 0; b < nblk; ++b) {
      float a = 0.0f;
      for (int64_t i = 0; i < 64; ++i) {
        float x = (float)load_elem(lut, dtype, r * D + b * 64 + i);
        float ax = fabsf(x);
        if (ax > a) a = ax;
      }
      if (a > 65504.0f) { a = 65504.0f; nsat += 1; }
      const uint16_t sbits = oracle_f32_to_f16_rne(a);
      scales[r * nblk + b] = sbits;
      const float s = oracle_f16_to_f32(sbits);
      float thr[7];
      for (int j = 0; j < 7; ++j) thr[j] = mid[j] * s; /* one fp32 multiply */
      for (int64_t i = 0; i < 64; ++i) {
        float x = (float)load_elem(lut, dtype, r * D + b * 64 + i);
        int code = 0;
        if (s == 0.0f) code = 3;
        else for (int j = 0; j < 7; ++j) if (x > thr[j]) code += 1;
        const int64_t pos = 3 * (b * 64 + i);
        put_bit(crow, pos + 0, code & 1);
        put_bit(crow, pos + 1, (code >> 1) & 1);
        put_bit(crow, pos + 2, (code >> 2) & 1);
      }
    }
  }
  if (n_saturated) *n_saturated = nsat;
  return OR_OK;
}

/* Read back the 3-bit codes of a packed [rows][3D/8] stream into [rows][D]. */
int oracle_unpack_nf3(const uint8_t* codes, int64_t rows, int64_t D, uint8_t* out) {
  if (rows < 0 || D <= 0 || D % 64 != 0) return OR_ERR_ARG;
  const int64_t row_bytes = 3 * D / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < D; ++i) {
      const uint8_t* crow = codes + r * row_bytes;
      out[r * D + i] = (uint8_t)(get_bit(crow, 3 * i) | (get_bit(crow, 3 * i + 1) << 1) |
                                 (get_bit(crow, 3 * i + 2) << 2));
    }
  return OR_OK;
}

/* Dequantise: xhat[r][i] = level[code] * s(block), as an exact product in
 * double (an fp32 level times an fp16 scale fits a double exactly). */
int oracle_dequant_nf3(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                       int64_t D, double* out) {
  if (rows < 0 || D <= 0 || D % 64 != 0) return OR_ERR_ARG;
  float lv[8];
  oracle_nf3_levels(lv);
  const int64_t row_bytes = 3 * D / 8, nblk = D / 64;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < D; ++i) {
      const uint8_t* crow = codes + r * row_bytes;
      int c = get_bit(crow, 3 * i) | (get_bit(crow, 3 * i + 1) << 1) |
              (get_bit(crow, 3 * i + 2) << 2);
      out[r * D + i] = (double)lv[c] * (double)oracle_f16_to_f32(scales[r * nblk + i / 64]);
    }
  return OR_OK;
}

/*
 * Lookup-combine over the NF3 table:
 *   y[t][d] = sum_e g[t][e] * level[code(id_t, e, d)] * s(id_t, e, d/64).
 * codes [V][N][3D/8], scales [V][N][D/64].  y is [T][D] fp64.
 */
int oracle_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r,
                              int dtype_hw, const uint8_t* codes,
                              const uint16_t* scales, int64_t T, int64_t V,
                              int64_t D, int64_t N, double* y, int nthreads) {
  if (!dtype_ok(dtype_hw) || T < 0 || V <= 0 || D <= 0 || D % 64 != 0 || N <= 0)
    return OR_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return OR_ERR_ID;
  float lv[8];
  oracle_nf3_levels(lv);
  double* gates = (double*)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
  if (!gates) return OR_ERR_MEM;
  int rc = oracle_router_gates(h, w_r, dtype_hw, T, D, N, gates, nthreads);
  const int64_t row_bytes = 3 * D / 8, nblk = D / 64;
  if (rc == OR_OK) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const int64_t v = ids[t];
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t e = 0; e < N; ++e) {
          const int64_t row = v * N + e;
          const uint8_t* crow = codes + row * row_bytes;
          int c = get_bit(crow, 3 * d) | (get_bit(crow, 3 * d + 1) << 1) |
                  (get_bit(crow, 3 * d + 2) << 2);
          double s = (double)oracle_f16_to_f32(scales[row * nblk + d / 64]);
          acc += gates[t * N + e] * ((double)lv[c] * s);
        }
        y[t * D + d] = acc;
      }
    }
  }
  free(gates);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Shared expert (training section: shared experts, like the router, keep   */
/* reading the previous layer's output; complexity analysis: at inference   */
/* the shared experts are the only experts still computed).                 */
/* ------------------------------------------------------------------------ */

/*
 * One shared-expert FFN with the routed experts' form (D -> F -> D, GELU in
 * its exact form, no biases), applied to every token's hidden state:
 *   u[f] = sum_d h[t][d] * W_s_up[f][d];   g[f] = GELU(u[f]);
 *   out[t][d] = sum_f g[f] * W_s_down[d][f].
 * w_s_up [F][D], w_s_down [D][F], h [T][D], all of `dtype`; out [T][D] fp64.
 */
int oracle_shared_ffn(const void* h, const void* w_s_up, const void* w_s_down,
                      int dtype, int64_t T, int64_t D, int64_t F, double* out,
                      int nthreads) {
  if (!dtype_ok(dtype) || T < 0 || D <= 0 || F <= 0) return OR_ERR_ARG;
  set_threads(nthreads);
  int failed = 0;
#pragma omp parallel
  {
    double* g = (double*)malloc((size_t)F * sizeof(double));
    if (!g) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic)
    for (int64_t t = 0; t < T; ++t) {
      if (!g) continue;
      for (int64_t f = 0; f < F; ++f) {
        double u = 0.0;
        for (int64_t d = 0; d < D; ++d)
          u += load_elem(h, dtype, t * D + d) * load_elem(w_s_up, dtype, f * D + d);
        g[f] = oracle_gelu(u);
      }
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t f = 0; f < F; ++f)
          acc += g[f] * load_elem(w_s_down, dtype, d * F + f);
        out[t * D + d] = acc;
      }
    }
    free(g);
  }
  return failed ? OR_ERR_MEM : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Other table formats (results section: the table still carries redundancy */
/* at 3 bits).  NF4: the NormalFloat construction at k = 4, same blocks and  */
/* scales as NF3.  int8: one fp32 absmax scale per (v, e) row.               */
/* ------------------------------------------------------------------------ */

/* NormalFloat levels at k = 4 bits (the same construction as at 3 bits:
 * p* = 1 - (1/(2*15) + 1/(2*16))/2; Phi^-1 at 9 evenly spaced probabilities
 * from p* down to 1/2 (1/2 dropped) for the 8 positive levels, -Phi^-1 at 8
 * evenly spaced probabilities for the 7 negative ones, one exact zero,
 * normalised by the maximum, sorted, rounded to fp32).  Zero is code 7. */
void oracle_nf4_levels(float out[16]) {
  const double pstar = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
  double v[16];
  int n = 0;
  for (int i = 0; i < 8; ++i)            /* linspace(p*, 0.5, 9)[0..7] */
    v[n++] = oracle_normal_ppf(pstar + (0.5 - pstar) * (double)i / 8.0);
  for (int i = 0; i < 7; ++i)            /* linspace(p*, 0.5, 8)[0..6] */
    v[n++] = -oracle_normal_ppf(pstar + (0.5 - pstar) * (double)i / 7.0);
  v[n++] = 0.0;
  double vmax = 0.0;
  for (int i = 0; i < 16; ++i) if (v[i] > vmax) vmax = v[i];
  for (int i = 0; i < 16; ++i) v[i] /= vmax;
  for (int i = 1; i < 16; ++i)
    for (int j = i; j > 0 && v[j - 1] > v[j]; --j) {
      double tmp = v[j]; v[j] = v[j - 1]; v[j - 1] = tmp;
    }
  for (int i = 0; i < 16; ++i) out[i] = (float)v[i];
}

void oracle_nf4_midpoints(float out[15]) {
  float lv[16];
  oracle_nf4_levels(lv);
  for (int j = 0; j < 15; ++j) out[j] = (float)(((double)lv[j] + (double)lv[j + 1]) / 2.0);
}

/*
 * Encode a [rows][D] table into NF4: per block of 64 elements the fp16
 * absmax scale exactly as for NF3; code = #{ j : x > fp32(mid[j] * s) }
 * (strict), code 7 (zero) if s == 0; code i of a row in bits [4i, 4i+4) of
 * the row's little-endian stream (low nibble first), D/2 bytes per row.
 */
int oracle_pack_nf4(const void* lut, int dtype, int64_t rows, int64_t D,
                    uint8_t* codes, uint16_t* scales, int64_t* n_saturated,
                    int nthreads) {
  if (!dtype_ok(dtype) || rows < 0 || D <= 0 || D % 64 != 0) return OR_ERR_ARG;
  float mid[15];
  oracle_nf4_midpoints(mid);
  const int64_t row_bytes = D / 2, nblk = D / 64;
  int64_t nsat = 0;
  set_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(+ : nsat)
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* crow = codes + r * row_bytes;
    memset(crow, 0, (size_t)row_bytes);
    for (int64_t b = 0; b < nblk; ++b) {
      float a = 0.0f;
      for (int64_t i = 0; i < 64; ++i) {
        float ax = fabsf((float)load_elem(lut, dtype, r * D + b * 64 + i));
        if (ax > a) a = ax;
      }
      if (a > 65504.0f) { a = 65504.0f; nsat += 1; }
      const uint16_t sbits = oracle_f32_to_f16_rne(a);
      scales[r * nblk + b] = sbits;
      const float s = oracle_f16_to_f32(sbits);
      float thr[15];
      for (int j = 0; j < 15; ++j) thr[j] = mid[j] * s;
      for (int64_t i = 0; i < 64; ++i) {
        float x = (float)load_elem(lut, dtype, r * D + b * 64 + i);
        int code = 0;
        if (s == 0.0f) code = 7;
        else for (int j = 0; j < 15; ++j) if (x > thr[j]) code += 1;
        const int64_t pos = 4 * (b * 64 + i);
        for (int k = 0; k < 4; ++k) put_bit(crow, pos + k, (code >> k) & 1);
      }
    }
  }
  if (n_saturated) *n_saturated = nsat;
  return OR_OK;
}

int oracle_unpack_nf4(const uint8_t* codes, int64_t rows, int64_t D, uint8_t* out) {
  if (rows < 0 || D <= 0 || D % 64 != 0) return OR_ERR_ARG;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < D; ++i) {
      const uint8_t* crow = codes + r * (D / 2);
      int c = 0;
      for (int k = 0; k < 4; ++k) c |= get_bit(crow, 4 * i + k) << k;
      out[r * D + i] = (uint8_t)c;
    }
  return OR_OK;
}

int oracle_dequant_nf4(const uint8_t* codes, const uint16_t* scales, int64_t rows,
                       int64_t D, double* out) {
  if (rows < 0 || D <= 0 || D % 64 != 0) return OR_ERR_ARG;
  float lv[16];
  oracle_nf4_levels(lv);
  const int64_t nblk = D / 64;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < D; ++i) {
      const uint8_t* crow = codes + r * (D / 2);
      int c = 0;
      for (int k = 0; k < 4; ++k) c |= get_bit(crow, 4 * i + k) << k;
      out[r * D + i] = (double)lv[c] * (double)oracle_f16_to_f32(scales[r * nblk + i / 64]);
    }
  return OR_OK;
}

/*
 * Encode a [rows][D] table into int8 with one scale per row:
 *   a = max |x| over the row (fp32);  s = fp32(a / 127) (one IEEE division);
 *   q = rint(fp32(x / s)) (IEEE division, ties to even), clamped to
 *   [-127, 127];  q = 0 for every element if s == 0.
 * codes [rows][D] int8, scales [rows] fp32.
 */
int oracle_pack_int8(const void* lut, int dtype, int64_t rows, int64_t D, int8_t* codes,
                     float* scales, int nthreads) {
  if (!dtype_ok(dtype) || rows < 0 || D <= 0) return OR_ERR_ARG;
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float a = 0.0f;
    for (int64_t i = 0; i < D; ++i) {
      float ax = fabsf((float)load_elem(lut, dtype, r * D + i));
      if (ax > a) a = ax;
    }
    const float s = a / 127.0f;
    scales[r] = s;
    for (int64_t i = 0; i < D; ++i) {
      int q = 0;
      if (s != 0.0f) {
        const float x = (float)load_elem(lut, dtype, r * D + i);
        const float qf = rintf(x / s);
        q = qf > 127.0f ? 127 : (qf < -127.0f ? -127 : (int)qf);
      }
      codes[r * D + i] = (int8_t)q;
    }
  }
  return OR_OK;
}

int oracle_dequant_int8(const int8_t* codes, const float* scales, int64_t rows, int64_t D,
                        double* out) {
  if (rows < 0 || D <= 0) return OR_ERR_ARG;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < D; ++i) out[r * D + i] = (double)codes[r * D + i] * (double)scales[r];
  return OR_OK;
}

/*
 * Lookup-combine over an NF4 or int8 table, from the dequantised values:
 *   y[t][d] = sum_e g[t][e] * xhat(id_t, e, d).
 * fmt 4: codes [V][N][D/2], scales fp16 [V][N][D/64];
 * fmt 8: codes int8 [V][N][D], scales fp32 [V][N].
 */
int oracle_lookup_combine_q(int fmt, const int64_t* ids, const void* h, const void* w_r,
                            int dtype_hw, const void* codes, const void* scales, int64_t T,
                            int64_t V, int64_t D, int64_t N, double* y, int nthreads) {
  if ((fmt != 4 && fmt != 8) || !dtype_ok(dtype_hw) || T < 0 || V <= 0 || D <= 0 ||
      D % 64 != 0 || N <= 0)
    return OR_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return OR_ERR_ID;
  double* gates = (double*)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
  double* row = (double*)malloc((size_t)D * sizeof(double));
  if (!gates || !row) { free(gates); free(row); return OR_ERR_MEM; }
  int rc = oracle_router_gates(h, w_r, dtype_hw, T, D, N, gates, nthreads);
  if (rc == OR_OK) {
    for (int64_t t = 0; t < T; ++t) {
      const int64_t v = ids[t];
      for (int64_t d = 0; d < D; ++d) y[t * D + d] = 0.0;
      for (int64_t e = 0; e < N; ++e) {
        const int64_t r = v * N + e;
        if (fmt == 4)
          oracle_dequant_nf4((const uint8_t*)codes + r * (D / 2), (const uint16_t*)scales + r * (D / 64),
                             1, D, row);
        else
          oracle_dequant_int8((const int8_t*)codes + r * D, (const float*)scales + r, 1, D, row);
        for (int64_t d = 0; d < D; ++d) y[t * D + d] += gates[t * N + e] * row[d];
      }
    }
  }
  free(gates);
  free(row);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Training mode (training section: every routed expert reads the shallow  */
/* embedding of the token, all experts are active, the router reads the    */
/* contextual hidden state; inference section: the table is this forward   */
/* pass evaluated for every vocabulary row).                                */
/* ------------------------------------------------------------------------ */

/*
 * Forward: y[t][:] = sum_e g[t][e] * W_down[e] . GELU(W_up[e] . Emb[ids[t]]),
 * g = softmax(W_r . h[t]) over all N.  y is [T][D] fp64.
 */
int oracle_train_forward(const int64_t* ids, const void* emb, const void* w_up, const void* w_down,
                         const void* h, const void* w_r, int dtype, int64_t T, int64_t V, int64_t D,
                         int64_t F, int64_t N, double* y, int nthreads) {
  if (!dtype_ok(dtype) || T < 0 || V <= 0 || D <= 0 || F <= 0 || N <= 0) return OR_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return OR_ERR_ID;
  double* gates = (double*)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
  if (!gates) return OR_ERR_MEM;
  int rc = oracle_router_gates(h, w_r, dtype, T, D, N, gates, nthreads);
  int failed = 0;
  if (rc == OR_OK) {
#pragma omp parallel
    {
      double* g = (double*)malloc((size_t)F * sizeof(double));
      if (!g) {
#pragma omp atomic write
        failed = 1;
      }
#pragma omp for schedule(dynamic)
      for (int64_t t = 0; t < T; ++t) {
        if (!g) continue;
        const int64_t v = ids[t];
        for (int64_t d = 0; d < D; ++d) y[t * D + d] = 0.0;
        for (int64_t e = 0; e < N; ++e) {
          for (int64_t f = 0; f < F; ++f) {
            double u = 0.0;
            for (int64_t d = 0; d < D; ++d)
              u += load_elem(emb, dtype, v * D + d) * load_elem(w_up, dtype, (e * F + f) * D + d);
            g[f] = oracle_gelu(u);
          }
          for (int64_t d = 0; d < D; ++d) {
            double o = 0.0;
            for (int64_t f = 0; f < F; ++f) o += g[f] * load_elem(w_down, dtype, (e * D + d) * F + f);
            y[t * D + d] += gates[t * N + e] * o;
          }
        }
      }
      free(g);
    }
  }
  free(gates);
  if (rc != OR_OK) return rc;
  return failed ? OR_ERR_MEM : OR_OK;
}

/* d GELU / du = Phi(u) + u * phi(u). */
static double gelu_grad(double u) {
  const double phi = exp(-0.5 * u * u) / sqrt(2.0 * 3.14159265358979323846);
  return 0.5 * (1.0 + erf(u / sqrt(2.0))) + u * phi;
}

/*
 * Backward of oracle_train_forward for an upstream gradient dy [T][D]
 * (fp64), by the chain rule written out per token and expert:
 *   o_e = W_down[e] . G_e,  G_e = GELU(u_e),  u_e = W_up[e] . x,  x = Emb[id];
 *   dg_e = dy . o_e;  dz_e = g_e (dg_e - sum_e' g_e' dg_e');
 *   d W_r[e] += dz_e h;  dh += sum_e dz_e W_r[e];
 *   d o_e = g_e dy;  d W_down[e] += d o_e (x) G_e;  d G_e = W_down[e]^T . d o_e;
 *   d u_e = d G_e * GELU'(u_e);  d W_up[e] += d u_e (x) x;  d x += W_up[e]^T . d u_e;
 *   d Emb[id] += d x.
 * Outputs (fp64, overwritten): d_w_up [N][F][D], d_w_down [N][D][F],
 * d_w_r [N][D], d_h [T][D], d_emb [V][D].  Serial over tokens (the weight
 * gradients are sums over the batch).
 */
int oracle_train_backward(const int64_t* ids, const void* emb, const void* w_up, const void* w_down,
                          const void* h, const void* w_r, int dtype, const double* dy, int64_t T,
                          int64_t V, int64_t D, int64_t F, int64_t N, double* d_w_up, double* d_w_down,
                          double* d_w_r, double* d_h, double* d_emb) {
  if (!dtype_ok(dtype) || T < 0 || V <= 0 || D <= 0 || F <= 0 || N <= 0) return OR_ERR_ARG;
  for (int64_t t = 0; t < T; ++t)
    if (ids[t] < 0 || ids[t] >= V) return OR_ERR_ID;
  memset(d_w_up, 0, (size_t)(N * F * D) * sizeof(double));
  memset(d_w_down, 0, (size_t)(N * D * F) * sizeof(double));
  memset(d_w_r, 0, (size_t)(N * D) * sizeof(double));
  memset(d_h, 0, (size_t)(T * D) * sizeof(double));
  memset(d_emb, 0, (size_t)(V * D) * sizeof(double));
  double* gates = (double*)malloc((size_t)(T > 0 ? T : 1) * N * sizeof(double));
  double* u = (double*)malloc((size_t)(N * F) * sizeof(double));
  double* G = (double*)malloc((size_t)(N * F) * sizeof(double));
  double* o = (double*)malloc((size_t)(N * D) * sizeof(double));
  double* dg = (double*)malloc((size_t)N * sizeof(double));
  double* dG = (double*)malloc((size_t)F * sizeof(double));
  if (!gates || !u || !G || !o || !dg || !dG) {
    free(gates); free(u); free(G); free(o); free(dg); free(dG);
    return OR_ERR_MEM;
  }
  int rc = oracle_router_gates(h, w_r, dtype, T, D, N, gates, 1);
  for (int64_t t = 0; rc == OR_OK && t < T; ++t) {
    const int64_t v = ids[t];
    const double* g = gates + t * N;
    for (int64_t e = 0; e < N; ++e) {
      for (int64_t f = 0; f < F; ++f) {
        double s = 0.0;
        for (int64_t d = 0; d < D; ++d)
          s += load_elem(emb, dtype, v * D + d) * load_elem(w_up, dtype, (e * F + f) * D + d);
        u[e * F + f] = s;
        G[e * F + f] = oracle_gelu(s);
      }
      for (int64_t d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t f = 0; f < F; ++f) s += G[e * F + f] * load_elem(w_down, dtype, (e * D + d) * F + f);
        o[e * D + d] = s;
      }
      double s = 0.0;
      for (int64_t d = 0; d < D; ++d) s += dy[t * D + d] * o[e * D + d];
      dg[e] = s;
    }
    double gdg = 0.0;
    for (int64_t e = 0; e < N; ++e) gdg += g[e] * dg[e];
    for (int64_t e = 0; e < N; ++e) {
      const double dz = g[e] * (dg[e] - gdg);
      for (int64_t d = 0; d < D; ++d) {
        d_w_r[e * D + d] += dz * load_elem(h, dtype, t * D + d);
        d_h[t * D + d] += dz * load_elem(w_r, dtype, e * D + d);
      }
    }
    for (int64_t e = 0; e < N; ++e) {
      for (int64_t f = 0; f < F; ++f) dG[f] = 0.0;
      for (int64_t d = 0; d < D; ++d) {
        const double dod = g[e] * dy[t * D + d];
        for (int64_t f = 0; f < F; ++f) {
          d_w_down[(e * D + d) * F + f] += dod * G[e * F + f];
          dG[f] += load_elem(w_down, dtype, (e * D + d) * F + f) * dod;
        }
      }
      for (int64_t f = 0; f < F; ++f) {
        const double du = dG[f] * gelu_grad(u[e * F + f]);
        for (int64_t d = 0; d < D; ++d) {
          d_w_up[(e * F + f) * D + d] += du * load_elem(emb, dtype, v * D + d);
          d_emb[v * D + d] += du * load_elem(w_up, dtype, (e * F + f) * D + d);
        }
      }
    }
  }
  free(gates); free(u); free(G); free(o); free(dg); free(dG);
  return rc;
}
