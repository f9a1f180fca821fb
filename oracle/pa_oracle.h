/*
 * pa_oracle.h -- fp64 CPU reference for paged-KV grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the parity oracle for the HIP
 * kernels of the paged_kv_gqa_attention_amd package.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header or table with the HIP
 * library, and it is deliberately plain and slow: every output row is the
 * textbook definition evaluated in double precision, one row at a time.
 *
 * What is computed (one output row per query token t and query head h):
 *
 *   b       : the sequence that owns token t, i.e. cu_q_lens[b] <= t < cu_q_lens[b+1]
 *   i       : t - cu_q_lens[b], the token's index inside the new query chunk
 *   q_len   : cu_q_lens[b+1] - cu_q_lens[b];  L : seq_lens[b]   (q_len <= L)
 *   pos     : L - q_len + i, the token's absolute position in its sequence
 *             (queries are the last q_len tokens of the sequence)
 *   g       : h / (Hq / Hkv), the KV head shared by a contiguous group of
 *             query heads
 *   key j   : for j < L, physical page page_table[b * row_stride + j / page],
 *             slot j % page, row k_pool[page][slot][g][0..D) (same for V)
 *   visible : j < L and (causal == 0 or j <= pos), intersected with an
 *             optional key window [key_begin, key_end) used for split-KV
 *             partials
 *   s_j     : scale * sum_d q[t][h][d] * K_j[d]      (fp64); with a soft cap
 *             c > 0 the score becomes c * tanh(s_j / c) before the softmax
 *   LSE     : max_j s_j + ln sum_j exp(s_j - max)    (natural log)
 *   O       : sum_j exp(s_j - LSE) * V_j             (fp64)
 *   empty visible set: O = 0 and LSE = -inf
 *
 * Sources: the varlen any-query-length attention with a masked-score
 * select of vLLM PR #16828 ("[Kernel] Unified Triton kernel that doesn't
 * distinguish between prefill + decode", description and the review thread on
 * the masked-score line); the page-resolution rule and the live seq_lens of
 * TensorRT-LLM PR #17399 ("integrate PrimTS FMHA kernels", section "Unified
 * page-table metadata"); fp8 KV with descale and a bf16 output from vLLM PR
 * #48156 ("[Perf][FA4] Warm up dense (paged) FA4 attention kernels", summary
 * and the fp8/descale discussion).  Where the pages are silent (causal offset,
 * head map, LSE base, fp8 format) the reading taken is documented next to the
 * code that implements it.
 *
 * Element formats: Q and bf16 K/V are passed as raw bfloat16 bit patterns
 * (uint16); fp8 K/V are raw OCP FP8 E4M3 bytes.  Decoding is exact.
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PAO_OK = 0, PAO_ERR_ARG = -1, PAO_ERR_DATA = -2 };
enum { PAO_KV_BF16 = 0, PAO_KV_FP8_E4M3 = 1 };
enum { PAO_Q_BF16 = 0, PAO_Q_FP8_E4M3 = 1 };

typedef struct {
  int32_t num_seqs;        /* B */
  int32_t num_q_heads;     /* Hq */
  int32_t num_kv_heads;    /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;        /* D */
  int32_t page_size;       /* tokens per page */
  int32_t num_pages;       /* P: physical pages in each pool */
  int32_t pt_cols;         /* C: logical pages per sequence (page-table width) */
  int32_t pt_row_stride;   /* elements between page-table rows (>= C) */
  int64_t kv_page_stride;  /* elements between physical pages; 0 = page*Hkv*D */
  int64_t q_stride_t;      /* elements between query tokens; 0 = Hq*D */
  int32_t kv_dtype;        /* PAO_KV_BF16 or PAO_KV_FP8_E4M3 */
  int32_t causal;          /* 0 or 1 */
  double scale;            /* softmax scale applied to q.k */
  double k_descale;        /* fp8 only: K value = e4m3(byte) * k_descale */
  double v_descale;        /* fp8 only: V value = e4m3(byte) * v_descale */
  double softcap;          /* > 0: scores s -> softcap * tanh(s / softcap); 0: off */
  int32_t q_dtype;         /* PAO_Q_BF16, or PAO_Q_FP8_E4M3: q holds E4M3 codes and
                              the query value is e4m3(byte) * q_descale */
  double q_descale;
} pao_problem;

/* Exact decoders of the element formats. */
double pao_bf16_to_double(uint16_t bits);
double pao_fp8_e4m3_to_double(uint8_t byte);

/*
 * Reference attention.
 *   q          : bf16 bits (or E4M3 bytes, q_dtype), token t / head h / dim d at
 *                q[t*q_stride_t + h*D + d]
 *   k_pool, v_pool : uint16 (bf16) or uint8 (fp8) elements, [P][page][Hkv][D]
 *                with kv_page_stride between pages
 *   page_table : int32 [B][pt_row_stride]; only the first ceil(L_b/page)
 *                columns of row b are read
 *   cu_q_lens  : int32 [B+1], non-decreasing, cu_q_lens[0] == 0
 *   seq_lens   : int32 [B]
 *   key_begin, key_end : key window; key_end < 0 means "no upper limit"
 *   rows       : NULL for every (t, h) in order, else num_rows flat indices
 *                t*Hq + h
 *   out        : fp64 [rows][D];  lse : fp64 [rows] (may be NULL)
 *   threads    : worker threads (<= 0: all available)
 * Returns PAO_OK, PAO_ERR_ARG for bad shapes, PAO_ERR_DATA for metadata
 * that breaks the contract (q_len > L, L > C*page, page id outside [0, P),
 * row index outside [0, T*Hq)).
 */
int pao_attention(const pao_problem* pr,
                  const void* q,
                  const void* k_pool, const void* v_pool,
                  const int32_t* page_table,
                  const int32_t* cu_q_lens, const int32_t* seq_lens,
                  int32_t key_begin, int32_t key_end,
                  const int64_t* rows, int64_t num_rows,
                  double* out, double* lse, int threads);

/*
 * Combine partial results computed over disjoint key windows:
 *   LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) * O_s
 * Partials with LSE_s = -inf contribute nothing (their O_s is not read).
 *   o_parts   : [S][n][D];  lse_parts : [S][n];  o : [n][D];  lse : [n]
 */
int pao_merge(int32_t num_parts, int64_t n, int32_t head_dim,
              const double* o_parts, const double* lse_parts,
              double* o, double* lse);

/*
 * Nearest finite OCP FP8 E4M3 code to x (ties to an even mantissa),
 * saturating to +-448; NaN gives the NaN code with x's sign.
 */
uint8_t pao_fp8_e4m3_encode(double x);

/*
 * KV-cache append: new token i of sequence b (row cu_new[b] + i of k_new and
 * v_new, bf16 bits, new_stride_t elements between tokens, 0 = Hkv*D) is the
 * token at position seq_lens[b] - n_b + i, where n_b = cu_new[b+1] - cu_new[b]
 * and seq_lens holds the lengths after the append.  Its rows are written to
 * k_pool / v_pool at that position's (page, slot) for every KV head: bf16
 * bits unchanged, or for fp8 pools the E4M3 code nearest to the binary32
 * quotient value / descale (pr->k_descale, pr->v_descale taken as binary32).
 * pr->num_q_heads, scale and causal are not used.  Returns PAO_ERR_DATA for
 * metadata that breaks the contract (n_b > L, L > C*page, page id out of range).
 */
int pao_append(const pao_problem* pr, const uint16_t* k_new, const uint16_t* v_new,
               int64_t new_stride_t, const int32_t* page_table, const int32_t* cu_new,
               const int32_t* seq_lens, void* k_pool, void* v_pool);

/*
 * MLA decode (DeepSeek-style multi-head latent attention over a paged latent
 * cache): one logical KV head whose cached row holds the compressed latent
 * (d_latent values) followed by the RoPE key (d_rope values).  For query head h
 * of sequence b (one query token per sequence, row b*Hq + h):
 *   s_j = scale * sum_{d < d_latent + d_rope} q[b][h][d] * C_j[d]   (j < L_b)
 *   LSE = max_j s_j + ln sum_j exp(s_j - max),   O = sum_j exp(s_j - LSE) C_j[0:d_latent)
 * i.e. the latent part of the cached row is both a key and the value.  The
 * query holds the absorbed latent query then its RoPE part.  C_j is the row of
 * page page_table[b][j / page], slot j % page.  Rows of a sequence with no key
 * give O = 0, LSE = -inf.  (BF16 MLA decode with one logical KV head, at most
 * 128 query heads, KV-LoRA rank 512 and RoPE dimension 64: TensorRT-LLM PR
 * #17399, "Integration and supported scope".)
 *   q     : bf16 bits, [B][q_stride_t] with head h at h*(d_latent+d_rope)
 *   kv    : bf16 bits, [P][page][d_latent+d_rope] with kv_page_stride between pages
 *   out   : fp64 [rows][d_latent];  lse : fp64 [rows] (may be NULL)
 */
typedef struct {
  int32_t num_seqs;        /* B */
  int32_t num_q_heads;     /* Hq */
  int32_t d_latent;        /* KV-LoRA rank (value width) */
  int32_t d_rope;          /* RoPE key width */
  int32_t page_size;
  int32_t num_pages;
  int32_t pt_cols;
  int32_t pt_row_stride;
  int64_t kv_page_stride;  /* elements between pages; 0 = page*(d_latent+d_rope) */
  int64_t q_stride_t;      /* elements between sequences' query rows; 0 = Hq*(d_latent+d_rope) */
  double scale;
  double softcap;          /* > 0: s -> softcap * tanh(s / softcap); 0: off */
} pao_mla_problem;

int pao_mla_decode(const pao_mla_problem* pr, const uint16_t* q, const uint16_t* kv,
                   const int32_t* page_table, const int32_t* seq_lens,
                   const int64_t* rows, int64_t num_rows, double* out, double* lse,
                   int threads);

#ifdef __cplusplus
}
#endif
#endif /* PA_ORACLE_H */
