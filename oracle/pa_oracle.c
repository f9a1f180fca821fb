/*
 * pa_oracle.c -- fp64 CPU reference for paged-KV grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY (see pa_oracle.h).  Plain C99 + OpenMP; every
 * output row is evaluated independently, straight from the definition, with a
 * two-pass softmax in double precision.  No blocking, no online rescaling, no
 * reordering beyond "for each visible key in increasing logical order".
 */
#include "pa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bfloat16 is the upper half of an IEEE binary32: widen and convert. */
double pao_bf16_to_double(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/*
 * OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
 * there are no infinities and S.1111.111 is NaN, so the largest finite
 * magnitude is 1.75 * 2^8 = 448.  (Reading of the unnamed "fp8" KV format on
 * the pages: the amax/448 per-tensor descale fixes the E4M3FN range.)
 */
double pao_fp8_e4m3_to_double(uint8_t byte) {
  const int sign = byte >> 7;
  const int e = (byte >> 3) & 0xF;
  const int m = byte & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, 1 - 7);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Element d of the K or V row of (physical page, slot, kv head). */
static double kv_elem(const pao_problem* pr, const void* pool, int64_t page,
                      int64_t slot, int64_t g, int64_t d, double descale) {
  const int64_t D = pr->head_dim, H = pr->num_kv_heads;
  const int64_t page_stride =
      pr->kv_page_stride ? pr->kv_page_stride : (int64_t)pr->page_size * H * D;
  const int64_t idx = page * page_stride + (slot * H + g) * D + d;
  if (pr->kv_dtype == PAO_KV_BF16)
    return pao_bf16_to_double(((const uint16_t*)pool)[idx]);
  return pao_fp8_e4m3_to_double(((const uint8_t*)pool)[idx]) * descale;
}

static int check_problem(const pao_problem* pr) {
  if (!pr) return PAO_ERR_ARG;
  if (pr->num_seqs < 0 || pr->num_q_heads <= 0 || pr->num_kv_heads <= 0 ||
      pr->head_dim <= 0 || pr->page_size <= 0 || pr->num_pages < 0 ||
      pr->pt_cols < 0 || pr->pt_row_stride < pr->pt_cols)
    return PAO_ERR_ARG;
  if (pr->num_q_heads % pr->num_kv_heads) return PAO_ERR_ARG;
  if (pr->kv_dtype != PAO_KV_BF16 && pr->kv_dtype != PAO_KV_FP8_E4M3)
    return PAO_ERR_ARG;
  if (!(pr->softcap >= 0.0) || isinf(pr->softcap)) return PAO_ERR_ARG;
  if (pr->q_dtype != PAO_Q_BF16 && pr->q_dtype != PAO_Q_FP8_E4M3) return PAO_ERR_ARG;
  if (pr->head_dim > 1024) return PAO_ERR_ARG;
  return PAO_OK;
}

/* Validate the per-sequence metadata once, before any row is evaluated. */
static int check_metadata(const pao_problem* pr, const int32_t* page_table,
                          const int32_t* cu_q_lens, const int32_t* seq_lens) {
  if (cu_q_lens[0] != 0) return PAO_ERR_DATA;
  for (int32_t b = 0; b < pr->num_seqs; ++b) {
    const int64_t q_len = (int64_t)cu_q_lens[b + 1] - cu_q_lens[b];
    const int64_t L = seq_lens[b];
    if (q_len < 0 || L < 0 || q_len > L) return PAO_ERR_DATA;
    if (L > (int64_t)pr->pt_cols * pr->page_size) return PAO_ERR_DATA;
    const int64_t used = (L + pr->page_size - 1) / pr->page_size;
    for (int64_t p = 0; p < used; ++p) {
      const int32_t phys = page_table[(int64_t)b * pr->pt_row_stride + p];
      if (phys < 0 || phys >= pr->num_pages) return PAO_ERR_DATA;
    }
  }
  return PAO_OK;
}

/* One output row (t, h): gather keys through the page table, two-pass softmax. */
static void one_row(const pao_problem* pr, const void* q,
                    const void* k_pool, const void* v_pool,
                    const int32_t* page_table, const int32_t* cu_q_lens,
                    const int32_t* seq_lens, int32_t key_begin, int32_t key_end,
                    int64_t t, int64_t h, double* s /* scratch [L] */,
                    double* o_row, double* lse_out) {
  const int64_t D = pr->head_dim;
  const int64_t G = pr->num_q_heads / pr->num_kv_heads;
  const int64_t q_stride = pr->q_stride_t ? pr->q_stride_t : pr->num_q_heads * D;

  /* the sequence that owns token t */
  int64_t b = 0;
  while (b + 1 < pr->num_seqs && cu_q_lens[b + 1] <= t) ++b;
  const int64_t i = t - cu_q_lens[b];
  const int64_t q_len = (int64_t)cu_q_lens[b + 1] - cu_q_lens[b];
  const int64_t L = seq_lens[b];
  /* Bottom-right causal alignment: the new tokens are the last q_len of the
   * sequence, so token i sits at absolute position L - q_len + i.  This is the
   * one reading under which a single-token decode sees every live key and a
   * chunked prefill on cached tokens sees its whole prefix. */
  const int64_t pos = L - q_len + i;
  /* Contiguous GQA groups: query heads g*G .. g*G+G-1 share KV head g. */
  const int64_t g = h / G;

  int64_t lo = key_begin > 0 ? key_begin : 0;
  int64_t hi = L;
  if (key_end >= 0 && key_end < hi) hi = key_end;
  if (pr->causal && pos + 1 < hi) hi = pos + 1;

  for (int64_t d = 0; d < D; ++d) o_row[d] = 0.0;
  if (hi <= lo) {
    *lse_out = -INFINITY;
    return;
  }

  /* The query row, decoded: bf16 exactly, or (fp8 queries, the fp8-in path
   * of vLLM PR #48156, fp8/descale discussion: fp8 inputs, bf16 output)
   * e4m3(byte) * q_descale. */
  double qrow[1024];
  for (int64_t d = 0; d < D; ++d)
    qrow[d] = pr->q_dtype == PAO_Q_FP8_E4M3
                  ? pao_fp8_e4m3_to_double(((const uint8_t*)q)[t * q_stride + h * D + d]) * pr->q_descale
                  : pao_bf16_to_double(((const uint16_t*)q)[t * q_stride + h * D + d]);
  double m = -INFINITY;
  for (int64_t j = lo; j < hi; ++j) {
    const int64_t phys = page_table[b * pr->pt_row_stride + j / pr->page_size];
    const int64_t slot = j % pr->page_size;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d)
      dot += qrow[d] * kv_elem(pr, k_pool, phys, slot, g, d, pr->k_descale);
    s[j - lo] = pr->scale * dot;
    /* Logit soft-capping: the unified kernel of vLLM PR #16828 (review thread
     * on the masked-score line) caps the scaled scores before the mask; the
     * page names the step without its formula, read here as the usual
     * c * tanh(s / c). */
    if (pr->softcap > 0.0) s[j - lo] = pr->softcap * tanh(s[j - lo] / pr->softcap);
    if (s[j - lo] > m) m = s[j - lo];
  }
  double l = 0.0;
  for (int64_t j = lo; j < hi; ++j) l += exp(s[j - lo] - m);
  const double lse = m + log(l);
  for (int64_t j = lo; j < hi; ++j) {
    const int64_t phys = page_table[b * pr->pt_row_stride + j / pr->page_size];
    const int64_t slot = j % pr->page_size;
    const double p = exp(s[j - lo] - lse);
    for (int64_t d = 0; d < D; ++d)
      o_row[d] += p * kv_elem(pr, v_pool, phys, slot, g, d, pr->v_descale);
  }
  *lse_out = lse;
}

int pao_attention(const pao_problem* pr, const void* q, const void* k_pool,
                  const void* v_pool, const int32_t* page_table,
                  const int32_t* cu_q_lens, const int32_t* seq_lens,
                  int32_t key_begin, int32_t key_end, const int64_t* rows,
                  int64_t num_rows, double* out, double* lse, int threads) {
  int rc = check_problem(pr);
  if (rc != PAO_OK) return rc;
  if (!q || !k_pool || !v_pool || !page_table || !cu_q_lens || !seq_lens || !out)
    return PAO_ERR_ARG;
  rc = check_metadata(pr, page_table, cu_q_lens, seq_lens);
  if (rc != PAO_OK) return rc;

  const int64_t Hq = pr->num_q_heads, D = pr->head_dim;
  const int64_t T = cu_q_lens[pr->num_seqs];
  const int64_t n = rows ? num_rows : T * Hq;
  if (rows)
    for (int64_t r = 0; r < n; ++r)
      if (rows[r] < 0 || rows[r] >= T * Hq) return PAO_ERR_DATA;
  int64_t max_L = 0;
  for (int32_t b = 0; b < pr->num_seqs; ++b)
    if (seq_lens[b] > max_L) max_L = seq_lens[b];

#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#else
  (void)threads;
#endif
  int failed = 0;
#pragma omp parallel num_threads(threads)
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_L > 0 ? max_L : 1));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        double lse_r;
        one_row(pr, q, k_pool, v_pool, page_table, cu_q_lens, seq_lens, key_begin,
                key_end, flat / Hq, flat % Hq, s, out + r * D, &lse_r);
        if (lse) lse[r] = lse_r;
      }
      free(s);
    }
  }
  return failed ? PAO_ERR_ARG : PAO_OK;
}

int pao_merge(int32_t num_parts, int64_t n, int32_t head_dim,
              const double* o_parts, const double* lse_parts, double* o,
              double* lse) {
  if (num_parts <= 0 || n < 0 || head_dim <= 0 || !o_parts || !lse_parts || !o)
    return PAO_ERR_ARG;
  for (int64_t r = 0; r < n; ++r) {
    double m = -INFINITY;
    for (int32_t s = 0; s < num_parts; ++s)
      if (lse_parts[s * n + r] > m) m = lse_parts[s * n + r];
    for (int32_t d = 0; d < head_dim; ++d) o[r * head_dim + d] = 0.0;
    if (m == -INFINITY) {
      if (lse) lse[r] = -INFINITY;
      continue;
    }
    double sum = 0.0;
    for (int32_t s = 0; s < num_parts; ++s)
      if (lse_parts[s * n + r] != -INFINITY) sum += exp(lse_parts[s * n + r] - m);
    const double total = m + log(sum);
    for (int32_t s = 0; s < num_parts; ++s) {
      const double ls = lse_parts[s * n + r];
      if (ls == -INFINITY) continue;
      const double w = exp(ls - total);
      for (int32_t d = 0; d < head_dim; ++d)
        o[r * head_dim + d] += w * o_parts[((int64_t)s * n + r) * head_dim + d];
    }
    if (lse) lse[r] = total;
  }
  return PAO_OK;
}

/*
 * Nearest finite OCP FP8 E4M3 code to x, ties to the code with an even
 * mantissa, magnitudes beyond the largest finite value (448) saturating to it;
 * NaN gives the NaN pattern (all exponent and mantissa bits set) with x's sign.
 * Written as a search over the 127 finite non-negative codes so that it rests
 * on the decoder above and nothing else.
 */
uint8_t pao_fp8_e4m3_encode(double x) {
  const int neg = signbit(x) != 0;
  if (isnan(x)) return (uint8_t)(0x7F | (neg ? 0x80 : 0));   /* E4M3's only NaN pattern */
  const double a = fabs(x);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c < 0x7F; ++c) {            /* 0x7F is NaN */
    const double err = fabs(pao_fp8_e4m3_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (neg ? 0x80 : 0));
}

/*
 * KV-cache append.  The new tokens of sequence b are rows cu_new[b] ..
 * cu_new[b+1]-1 of k_new / v_new; they are the LAST n_b tokens of the
 * sequence whose length (after the append) is seq_lens[b], so new token i
 * goes to position L - n_b + i: physical page page_table[b][pos / page],
 * slot pos % page, head g.  bf16 pools receive the bits unchanged; fp8 pools
 * receive the E4M3 code nearest to the binary32 quotient value / descale
 * (the stored code times the descale reproduces the value, as for reads).
 * Nothing else in the pools is written.  (The fused preprocessing of
 * TensorRT-LLM PR #17399, section "Planning, preprocessing, and workspace
 * ownership", appends the step's K/V to the paged cache before attention.)
 */
int pao_append(const pao_problem* pr, const uint16_t* k_new, const uint16_t* v_new,
               int64_t new_stride_t, const int32_t* page_table, const int32_t* cu_new,
               const int32_t* seq_lens, void* k_pool, void* v_pool) {
  int rc = check_problem(pr);
  if (rc != PAO_OK) return rc;
  if (!k_new || !v_new || !page_table || !cu_new || !seq_lens || !k_pool || !v_pool)
    return PAO_ERR_ARG;
  rc = check_metadata(pr, page_table, cu_new, seq_lens);
  if (rc != PAO_OK) return rc;
  const int64_t D = pr->head_dim, H = pr->num_kv_heads;
  const int64_t stride = new_stride_t ? new_stride_t : H * D;
  const int64_t page_stride =
      pr->kv_page_stride ? pr->kv_page_stride : (int64_t)pr->page_size * H * D;
  const float kd = (float)pr->k_descale, vd = (float)pr->v_descale;
  for (int32_t b = 0; b < pr->num_seqs; ++b) {
    const int64_t n = (int64_t)cu_new[b + 1] - cu_new[b];
    const int64_t L = seq_lens[b];
    for (int64_t i = 0; i < n; ++i) {
      const int64_t t = cu_new[b] + i;
      const int64_t pos = L - n + i;
      const int64_t page = page_table[(int64_t)b * pr->pt_row_stride + pos / pr->page_size];
      const int64_t slot = pos % pr->page_size;
      for (int64_t g = 0; g < H; ++g)
        for (int64_t d = 0; d < D; ++d) {
          const int64_t src = t * stride + g * D + d;
          const int64_t dst = page * page_stride + (slot * H + g) * D + d;
          if (pr->kv_dtype == PAO_KV_BF16) {
            ((uint16_t*)k_pool)[dst] = k_new[src];
            ((uint16_t*)v_pool)[dst] = v_new[src];
          } else {
            const float kq = (float)pao_bf16_to_double(k_new[src]) / kd;
            const float vq = (float)pao_bf16_to_double(v_new[src]) / vd;
            ((uint8_t*)k_pool)[dst] = pao_fp8_e4m3_encode((double)kq);
            ((uint8_t*)v_pool)[dst] = pao_fp8_e4m3_encode((double)vq);
          }
        }
    }
  }
  return PAO_OK;
}

/* ------------------------------------------------------------------------ */
/* MLA decode                                                                */
/* ------------------------------------------------------------------------ */

static void mla_row(const pao_mla_problem* pr, const uint16_t* q, const uint16_t* kv,
                    const int32_t* page_table, const int32_t* seq_lens, int64_t row,
                    double* s, double* o_row, double* lse_out) {
  const int64_t Dk = (int64_t)pr->d_latent + pr->d_rope;
  const int64_t Dv = pr->d_latent;
  const int64_t page_stride = pr->kv_page_stride ? pr->kv_page_stride : (int64_t)pr->page_size * Dk;
  const int64_t q_stride = pr->q_stride_t ? pr->q_stride_t : (int64_t)pr->num_q_heads * Dk;
  const int64_t b = row / pr->num_q_heads;
  const int64_t h = row % pr->num_q_heads;
  const int64_t L = seq_lens[b];
  for (int64_t d = 0; d < Dv; ++d) o_row[d] = 0.0;
  if (L <= 0) {
    *lse_out = -INFINITY;
    return;
  }
  const uint16_t* qrow = q + b * q_stride + h * Dk;
  double m = -INFINITY;
  for (int64_t j = 0; j < L; ++j) {
    const uint16_t* c = kv + (int64_t)page_table[b * pr->pt_row_stride + j / pr->page_size] * page_stride +
                        (j % pr->page_size) * Dk;
    double dot = 0.0;
    for (int64_t d = 0; d < Dk; ++d) dot += pao_bf16_to_double(qrow[d]) * pao_bf16_to_double(c[d]);
    s[j] = pr->scale * dot;
    if (pr->softcap > 0.0) s[j] = pr->softcap * tanh(s[j] / pr->softcap);
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < L; ++j) l += exp(s[j] - m);
  const double lse = m + log(l);
  for (int64_t j = 0; j < L; ++j) {
    const uint16_t* c = kv + (int64_t)page_table[b * pr->pt_row_stride + j / pr->page_size] * page_stride +
                        (j % pr->page_size) * Dk;
    const double p = exp(s[j] - lse);
    for (int64_t d = 0; d < Dv; ++d) o_row[d] += p * pao_bf16_to_double(c[d]);
  }
  *lse_out = lse;
}

int pao_mla_decode(const pao_mla_problem* pr, const uint16_t* q, const uint16_t* kv,
                   const int32_t* page_table, const int32_t* seq_lens,
                   const int64_t* rows, int64_t num_rows, double* out, double* lse,
                   int threads) {
  if (!pr || !q || !kv || !page_table || !seq_lens || !out) return PAO_ERR_ARG;
  if (pr->num_seqs < 0 || pr->num_q_heads <= 0 || pr->d_latent <= 0 || pr->d_rope < 0 ||
      pr->page_size <= 0 || pr->num_pages < 0 || pr->pt_cols < 0 ||
      pr->pt_row_stride < pr->pt_cols || !(pr->softcap >= 0.0) || isinf(pr->softcap))
    return PAO_ERR_ARG;
  int64_t max_L = 0;
  for (int32_t b = 0; b < pr->num_seqs; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 0 || L > (int64_t)pr->pt_cols * pr->page_size) return PAO_ERR_DATA;
    for (int64_t p = 0; p < (L + pr->page_size - 1) / pr->page_size; ++p) {
      const int32_t phys = page_table[(int64_t)b * pr->pt_row_stride + p];
      if (phys < 0 || phys >= pr->num_pages) return PAO_ERR_DATA;
    }
    if (L > max_L) max_L = L;
  }
  const int64_t total = (int64_t)pr->num_seqs * pr->num_q_heads;
  const int64_t n = rows ? num_rows : total;
  if (rows)
    for (int64_t r = 0; r < n; ++r)
      if (rows[r] < 0 || rows[r] >= total) return PAO_ERR_DATA;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#else
  (void)threads;
#endif
  int failed = 0;
#pragma omp parallel num_threads(threads)
  {
    double* s = (double*)malloc((size_t)(max_L > 0 ? max_L : 1) * sizeof(double));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n; ++r) {
        double l;
        mla_row(pr, q, kv, page_table, seq_lens, rows ? rows[r] : r, s,
                out + r * pr->d_latent, &l);
        if (lse) lse[r] = l;
      }
      free(s);
    }
  }
  return failed ? PAO_ERR_ARG : PAO_OK;
}
