/*
 * das_oracle.c -- fp64 CPU oracle for single-query (decode) softmax attention
 * and the log-sum-exp merge of attention states.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it includes nothing but libc,
 * libm and OpenMP.
 *
 * Sources (cited by page title and section):
 *   [FD++]  "FlashDecoding++: 시퀀스 차원 KV 분할 병렬화와 GPU 언더유틸라이제이션
 *           극복을 통한 LLM 서빙 극대화" (TechKnowGenie post).  §1 describes the
 *           decode step (one query token against N cached K/V rows); §3
 *           describes phase 1 (per-chunk logits, chunk max, exponentials,
 *           chunk sum, unnormalised chunk output) and phase 2 (global max,
 *           per-chunk correction factors, global sum, final division); §5
 *           computes the unsplit ground truth as matmul -> softmax -> matmul.
 *   [SGL-PAR] "병렬 처리 개요 (Parallelism Overview)", SGLang Diffusion docs
 *           (data-sketchers wiki).  "What happens to the shapes" and
 *           "Constraints": ring attention and the tail/replicated-part path
 *           join partial attention results through an online-softmax merge
 *           that needs each part's softmax log-sum-exp.
 *
 * Readings taken where the pages are silent (the plainest one the rest of the
 * pages supports):
 *   - lse is the natural log of the sum of exp(scaled logit);
 *   - no epsilon is added to the softmax denominator (the emulator in §5 adds
 *     one, but the pages call the result exact, and the denominator is >= 1);
 *   - GQA: query head h reads kv-head h / (Hq / Hkv);
 *   - seq_lens[b] is clamped to [0, Smax]; an empty row set gives out = 0,
 *     lse = -inf (the identity of the merge);
 *   - scale multiplies the finished dot product q.k.
 *
 * Arithmetic: every bf16 input is widened exactly to double; dot products,
 * exponentials, sums and divisions run in double with libm exp/log, in the
 * plain order the definition states.  Build with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int clamp_len(int32_t L, int32_t smax) {
  if (L < 0) return 0;
  if (L > smax) return smax;
  return L;
}

int das_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void das_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Logit of row j for query row qrow: scale * sum_d q[d] * k[j][d]. */
static double logit(const uint16_t* qrow, const uint16_t* krow, int D, double scale) {
  double dot = 0.0;
  for (int d = 0; d < D; ++d) dot += widen_bf16(qrow[d]) * widen_bf16(krow[d]);
  return scale * dot;
}

/*
 * The value of a V element in the weighted sum: the element itself, or, for
 * the magnitude form (absv != 0), its absolute value.
 */
static double vterm(double x, int absv) { return absv ? fabs(x) : x; }

/*
 * Unsplit attention, the plain definition ([FD++] §1 decode step, §5 ground
 * truth):  s_j = scale * q.k_j,  M = max_j s_j,  w_j = exp(s_j - M),
 * Z = sum_j w_j,  out = sum_j w_j v_j / Z,  lse = M + ln Z.
 * With absv != 0, out = sum_j w_j |v_j| / Z instead (elementwise absolute
 * values): the magnitude of the terms the output averages, which bounds how
 * far rounding can move an output that cancels to near zero.
 *
 * q: [B][Hq][D] bf16 bits; k, v: [B][Hkv][Smax][D] bf16 bits;
 * out: [B][Hq][D] double; lse: [B][Hq] double.
 */
static void attention_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t Smax, int32_t D, double scale, double* out, double* lse,
                           int absv) {
  const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const int L = clamp_len(seq_lens[b], Smax);
      const uint16_t* qrow = q + ((size_t)b * Hq + h) * D;
      const uint16_t* kbase = k + ((size_t)b * Hkv + g) * (size_t)Smax * D;
      const uint16_t* vbase = v + ((size_t)b * Hkv + g) * (size_t)Smax * D;
      double* o = out + ((size_t)b * Hq + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (L == 0) {
        lse[(size_t)b * Hq + h] = -INFINITY;
        continue;
      }
      double* w = (double*)malloc(sizeof(double) * (size_t)L);
      double M = -INFINITY;
      for (int j = 0; j < L; ++j) {
        w[j] = logit(qrow, kbase + (size_t)j * D, D, scale);
        if (w[j] > M) M = w[j];
      }
      double Z = 0.0;
      for (int j = 0; j < L; ++j) {
        w[j] = exp(w[j] - M);
        Z += w[j];
      }
      for (int j = 0; j < L; ++j) {
        const uint16_t* vrow = vbase + (size_t)j * D;
        for (int d = 0; d < D; ++d) o[d] += w[j] * vterm(widen_bf16(vrow[d]), absv);
      }
      for (int d = 0; d < D; ++d) o[d] /= Z;
      lse[(size_t)b * Hq + h] = M + log(Z);
      free(w);
    }
  }
}

void das_oracle_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t Smax, int32_t D, double scale, double* out, double* lse) {
  attention_bf16(q, k, v, seq_lens, B, Hq, Hkv, Smax, D, scale, out, lse, 0);
}

/* out = sum_j w_j |v_j| / Z: the magnitude form of das_oracle_attention. */
void das_oracle_abs_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t Smax, int32_t D, double scale, double* out, double* lse) {
  attention_bf16(q, k, v, seq_lens, B, Hq, Hkv, Smax, D, scale, out, lse, 1);
}

/*
 * Two-phase split form, in the order [FD++] §3 gives it.  The row range
 * [0, Smax) is cut into consecutive chunks of `chunk` rows (the last one
 * ragged); rows at or past seq_lens[b] belong to no chunk, so trailing chunks
 * can be empty.
 *   Phase 1, per chunk c: logits over the chunk, chunk max m_c, exponentials
 *     p_j = exp(s_j - m_c), chunk sum l_c = sum p_j, unnormalised output
 *     o_c = sum p_j v_j.  An empty chunk has m_c = -inf, l_c = 0, o_c = 0.
 *   Phase 2: global max M = max_c m_c, factor f_c = exp(m_c - M) (0 for an
 *     empty chunk), global sum Lsum = sum_c f_c l_c, output
 *     out = (sum_c f_c o_c) / Lsum, and lse = M + ln Lsum.
 * Used to pin that splitting is exact; the GPU path is never compared to it.
 */
void das_oracle_split_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                int32_t Smax, int32_t D, double scale, int32_t chunk,
                                double* out, double* lse) {
  const int G = Hq / Hkv;
  const int nchunks = chunk > 0 ? (Smax + chunk - 1) / chunk : 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const int L = clamp_len(seq_lens[b], Smax);
      const uint16_t* qrow = q + ((size_t)b * Hq + h) * D;
      const uint16_t* kbase = k + ((size_t)b * Hkv + g) * (size_t)Smax * D;
      const uint16_t* vbase = v + ((size_t)b * Hkv + g) * (size_t)Smax * D;
      double* o = out + ((size_t)b * Hq + h) * D;
      double* m_c = (double*)malloc(sizeof(double) * (size_t)(nchunks > 0 ? nchunks : 1));
      double* l_c = (double*)malloc(sizeof(double) * (size_t)(nchunks > 0 ? nchunks : 1));
      double* o_c = (double*)calloc((size_t)(nchunks > 0 ? nchunks : 1) * D, sizeof(double));
      double* p = (double*)malloc(sizeof(double) * (size_t)(chunk > 0 ? chunk : 1));
      /* phase 1 */
      for (int c = 0; c < nchunks; ++c) {
        const int j0 = c * chunk;
        const int j1 = (j0 + chunk < L) ? j0 + chunk : L;
        m_c[c] = -INFINITY;
        l_c[c] = 0.0;
        if (j1 <= j0) continue;
        for (int j = j0; j < j1; ++j) {
          p[j - j0] = logit(qrow, kbase + (size_t)j * D, D, scale);
          if (p[j - j0] > m_c[c]) m_c[c] = p[j - j0];
        }
        for (int j = j0; j < j1; ++j) {
          p[j - j0] = exp(p[j - j0] - m_c[c]);
          l_c[c] += p[j - j0];
        }
        for (int j = j0; j < j1; ++j) {
          const uint16_t* vrow = vbase + (size_t)j * D;
          for (int d = 0; d < D; ++d) o_c[(size_t)c * D + d] += p[j - j0] * widen_bf16(vrow[d]);
        }
      }
      /* phase 2 */
      double M = -INFINITY;
      for (int c = 0; c < nchunks; ++c)
        if (m_c[c] > M) M = m_c[c];
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (M == -INFINITY) {
        lse[(size_t)b * Hq + h] = -INFINITY;
      } else {
        double Lsum = 0.0;
        for (int c = 0; c < nchunks; ++c) {
          const double f = (m_c[c] == -INFINITY) ? 0.0 : exp(m_c[c] - M);
          Lsum += f * l_c[c];
          for (int d = 0; d < D; ++d) o[d] += f * o_c[(size_t)c * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= Lsum;
        lse[(size_t)b * Hq + h] = M + log(Lsum);
      }
      free(m_c);
      free(l_c);
      free(o_c);
      free(p);
    }
  }
}

/*
 * Merge of two normalised attention states over disjoint row sets
 * ([SGL-PAR] "What happens to the shapes", "Constraints": online-softmax
 * merge driven by each part's LSE):
 *   mx = max(a, b); if mx = -inf the result is (0, -inf);
 *   lse = mx + ln(exp(a - mx) + exp(b - mx));
 *   o = exp(a - lse) o_a + exp(b - lse) o_b.
 * The formula is symmetric in its two arguments.
 */
void das_oracle_merge(const double* o_a, const double* lse_a, const double* o_b,
                      const double* lse_b, int64_t rows, int32_t D, double* o_out,
                      double* lse_out) {
  for (int64_t r = 0; r < rows; ++r) {
    const double a = lse_a[r], b = lse_b[r];
    const double mx = a > b ? a : b;
    double* o = o_out + (size_t)r * D;
    if (mx == -INFINITY) {
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      lse_out[r] = -INFINITY;
      continue;
    }
    const double lse = mx + log(exp(a - mx) + exp(b - mx));
    const double wa = exp(a - lse), wb = exp(b - lse);
    for (int d = 0; d < D; ++d) o[d] = wa * o_a[(size_t)r * D + d] + wb * o_b[(size_t)r * D + d];
    lse_out[r] = lse;
  }
}

/*
 * 8-bit floating point K/V cache ([FD++] §4: quantised K and V are read from
 * memory and turned back into wider floats before the products).  The pages
 * name FP8 but not its encoding or scaling; the readings taken here are
 * OCP E4M3 codes and one fp32 scale per kv-head for K and one for V, so that
 * the cached value of element d of row j of kv-head g is
 * k_scale[g] * e4m3(code).
 *
 * E4M3 (OCP 8-bit floating point, "E4M3" encoding): sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits.  Exponent field 0 holds the subnormals
 * m * 2^-9; exponent 1..15 the normals (1 + m/8) * 2^(e - 7), except that
 * exponent 15 with mantissa 7 is NaN.  There are no infinities.
 */
static double e4m3_value(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

void das_oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
}

/*
 * Unsplit attention over an E4M3 K/V cache: the same definition as
 * das_oracle_attention with k = k_scale[g] * e4m3(code), v likewise (the
 * product is exact in double: 4 + 24 significant bits).
 * k, v: [B][Hkv][Smax][D] codes; k_scale, v_scale: [Hkv] fp32.
 */
static void attention_e4m3(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                           const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                           int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                           double scale, double* out, double* lse, int absv) {
  const int G = Hq / Hkv;
  double e4m3[256];  /* the value of every code, from e4m3_value */
  for (int c = 0; c < 256; ++c) e4m3[c] = e4m3_value((uint8_t)c);
#pragma omp parallel for collapse(2) schedule(dynamic, 1) firstprivate(e4m3)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const int L = clamp_len(seq_lens[b], Smax);
      const uint16_t* qrow = q + ((size_t)b * Hq + h) * D;
      const uint8_t* kbase = k + ((size_t)b * Hkv + g) * (size_t)Smax * D;
      const uint8_t* vbase = v + ((size_t)b * Hkv + g) * (size_t)Smax * D;
      const double ks = (double)k_scale[g], vs = (double)v_scale[g];
      double* o = out + ((size_t)b * Hq + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (L == 0) {
        lse[(size_t)b * Hq + h] = -INFINITY;
        continue;
      }
      double* w = (double*)malloc(sizeof(double) * (size_t)L);
      double M = -INFINITY;
      for (int j = 0; j < L; ++j) {
        const uint8_t* krow = kbase + (size_t)j * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += widen_bf16(qrow[d]) * (ks * e4m3[krow[d]]);
        w[j] = scale * dot;
        if (w[j] > M) M = w[j];
      }
      double Z = 0.0;
      for (int j = 0; j < L; ++j) {
        w[j] = exp(w[j] - M);
        Z += w[j];
      }
      for (int j = 0; j < L; ++j) {
        const uint8_t* vrow = vbase + (size_t)j * D;
        for (int d = 0; d < D; ++d) o[d] += w[j] * vterm(vs * e4m3[vrow[d]], absv);
      }
      for (int d = 0; d < D; ++d) o[d] /= Z;
      lse[(size_t)b * Hq + h] = M + log(Z);
      free(w);
    }
  }
}

void das_oracle_attention_fp8(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                              const float* k_scale, const float* v_scale,
                              const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t Smax, int32_t D, double scale, double* out, double* lse) {
  attention_e4m3(q, k, v, k_scale, v_scale, seq_lens, B, Hq, Hkv, Smax, D, scale, out, lse, 0);
}

/* out = sum_j w_j |v_j| / Z over the E4M3 cache: the magnitude form. */
void das_oracle_abs_attention_fp8(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t Smax, int32_t D, double scale, double* out,
                                  double* lse) {
  attention_e4m3(q, k, v, k_scale, v_scale, seq_lens, B, Hq, Hkv, Smax, D, scale, out, lse, 1);
}

/*
 * 4-bit integer K/V cache ([FD++] §4 names INT4 beside FP8: quantised K and V
 * are turned back into wider floats on chip, a quarter of the bf16 bytes).
 * The pages give neither the code nor the scaling; the readings taken here:
 * two's-complement 4-bit integers (-8..7), two per byte, element 2i in the
 * low nibble and element 2i+1 in the high nibble; one fp32 scale per cached
 * row (batch row, kv-head, token) for K and one for V.  Element d of row j of
 * kv-head g of batch row b is k_scale[b][g][j] * int4(element d).
 */
static int int4_value(uint8_t byte, int high) {
  const int n = high ? (byte >> 4) : (byte & 15);
  return n >= 8 ? n - 16 : n;
}

/* Element i of a packed INT4 array (n elements, n/2 bytes). */
void das_oracle_int4_decode(const uint8_t* packed, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (double)int4_value(packed[i / 2], (int)(i & 1));
}

/*
 * Unsplit attention over an INT4 K/V cache: the same definition as
 * das_oracle_attention with k = k_scale[b][g][j] * int4(code), v likewise
 * (exact in double).  k, v: [B][Hkv][Smax][D/2] bytes; k_scale, v_scale:
 * [B][Hkv][Smax] fp32.
 */
static void attention_i4(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                         const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                         int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                         double scale, double* out, double* lse, int absv) {
  const int G = Hq / Hkv;
  const int row_bytes = D / 2;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const int L = clamp_len(seq_lens[b], Smax);
      const uint16_t* qrow = q + ((size_t)b * Hq + h) * D;
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)Smax;
      double* o = out + ((size_t)b * Hq + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      if (L == 0) {
        lse[(size_t)b * Hq + h] = -INFINITY;
        continue;
      }
      double* w = (double*)malloc(sizeof(double) * (size_t)L);
      double M = -INFINITY;
      for (int j = 0; j < L; ++j) {
        const uint8_t* krow = k + (slab + j) * row_bytes;
        const double ks = (double)k_scale[slab + j];
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += widen_bf16(qrow[d]) * (ks * (double)int4_value(krow[d / 2], d & 1));
        w[j] = scale * dot;
        if (w[j] > M) M = w[j];
      }
      double Z = 0.0;
      for (int j = 0; j < L; ++j) {
        w[j] = exp(w[j] - M);
        Z += w[j];
      }
      for (int j = 0; j < L; ++j) {
        const uint8_t* vrow = v + (slab + j) * row_bytes;
        const double vs = (double)v_scale[slab + j];
        for (int d = 0; d < D; ++d)
          o[d] += w[j] * vterm(vs * (double)int4_value(vrow[d / 2], d & 1), absv);
      }
      for (int d = 0; d < D; ++d) o[d] /= Z;
      lse[(size_t)b * Hq + h] = M + log(Z);
      free(w);
    }
  }
}

void das_oracle_attention_int4(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                               const float* k_scale, const float* v_scale,
                               const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                               int32_t Smax, int32_t D, double scale, double* out, double* lse) {
  attention_i4(q, k, v, k_scale, v_scale, seq_lens, B, Hq, Hkv, Smax, D, scale, out, lse, 0);
}

/* out = sum_j w_j |v_j| / Z over the INT4 cache: the magnitude form. */
void das_oracle_abs_attention_int4(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                   int32_t Smax, int32_t D, double scale, double* out,
                                   double* lse) {
  attention_i4(q, k, v, k_scale, v_scale, seq_lens, B, Hq, Hkv, Smax, D, scale, out, lse, 1);
}
