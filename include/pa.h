/*
 * pa.h -- C ABI of libpa.so: paged-KV grouped-query attention on MI355X (gfx950).
 *
 * One operation, three schedules.  Every run computes, for each query token t
 * and query head h,
 *
 *     O[t, h, :] = sum_{j visible} softmax_j(scale * q[t,h] . K_j) * V_j
 *     LSE[t, h]  = ln sum_{j visible} exp(scale * q[t,h] . K_j)
 *
 * over the keys of t's sequence b, gathered through an int32 page table:
 * logical key j < seq_lens[b] lives in physical page page_table[b][j / page],
 * slot j % page, KV head g = h / (Hq / Hkv).  Queries are the last q_len_b
 * tokens of their sequence, so token i of sequence b sits at position
 * seq_lens[b] - q_len_b + i and, when causal, sees keys j <= that position.
 * Sources:
 *   - TensorRT-LLM PR #17399 "integrate PrimTS FMHA kernels", section
 *     "Unified page-table metadata": int32 fixed row-strided page table [B, C]
 *     plus live int32 sequence lengths [B]; logical page p of request b is
 *     block_tables[b, p]; columns past the live page count are never consumed;
 *     K and V keep their own pool displacement.  Section "Planning,
 *     preprocessing, and workspace ownership": one plan per batch shape,
 *     request metadata bound at run time, context needs no scratch, decode
 *     takes a caller-provided aligned workspace, the split-KV counter is the
 *     only state that must be reset.  Section "Integration and supported
 *     scope": page sizes 16/32/64/128, head dims 64/128/256, GQA ratio up to
 *     32, unsupported requests fail closed so a caller can fall back.
 *   - vLLM PR #16828 "Unified Triton kernel that doesn't distinguish between
 *     prefill + decode": one kernel for any query length (varlen, like a
 *     varlen flash-attention call), GQA query heads packed along the query
 *     dimension, masks applied by selecting -inf.
 *   - vLLM PR #48156 "[Perf][FA4] Warm up dense (paged) FA4 attention
 *     kernels": paged prefill/decode specialisations keyed on query-tile
 *     stage and split-KV (num_splits 0 = heuristic), fp8 KV with descale and
 *     a bf16 output.
 *
 * Conventions
 *   Ownership   The caller owns every device buffer, the workspace included.
 *               The library allocates no device memory.  A plan is a host
 *               object owned by the caller (pa_plan_destroy).
 *   Streams     pa_run_* enqueue kernels on the given stream and return; they
 *               never synchronise, allocate, or read device memory on the host,
 *               so they may be captured into a HIP graph.  Metadata (page table,
 *               lengths, cu_q_lens, descales) is read by the kernels when they
 *               run, so a captured graph replays against the current contents.
 *   Concurrency A plan is immutable after pa_plan and may be shared by threads.
 *               Runs that overlap in time need distinct workspaces.
 *   Errors      Host-checkable problems return PA_ERR_INVALID (null or
 *               misaligned pointers, bad strides, missing fp8 descale),
 *               PA_ERR_WORKSPACE (workspace smaller than pa_workspace_bytes),
 *               PA_ERR_UNSUPPORTED (geometry outside the compiled scope: fail
 *               closed) or PA_ERR_HIP (a launch failed).  Nothing is enqueued
 *               when a run returns an error.  Device-side contract violations
 *               (q_len_b > seq_lens[b], seq_lens[b] > C * page, a live page id
 *               outside [0, num_pages), cu_q_lens[B] > max_total_q) are the
 *               caller's responsibility; lengths are clamped so the kernels
 *               stay inside the buffers, page ids are not checked by the runs
 *               (pa_check_metadata checks all of these on the device).
 *   Layouts     All element strides are in elements, not bytes.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,      /* bad argument: null/misaligned pointer, bad stride or size */
  PA_ERR_UNSUPPORTED = -2,  /* geometry outside the compiled scope (fail closed) */
  PA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than pa_workspace_bytes() */
  PA_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  PA_ERR_SCRATCH = -5       /* pa_run_decode_static: the plan needs more scratch than its static array */
} pa_status;

typedef enum {
  PA_KV_BF16 = 0,           /* K/V pools hold bfloat16 */
  PA_KV_FP8_E4M3 = 1        /* K/V pools hold OCP FP8 E4M3 bytes, value = e4m3 * descale */
} pa_kv_dtype;

typedef enum {
  PA_Q_BF16 = 0,            /* queries are bfloat16 */
  PA_Q_FP8_E4M3 = 1         /* queries are OCP FP8 E4M3 bytes, value = e4m3 * q_descale */
} pa_q_dtype;

/*
 * Shape bounds of a plan (host values only).
 *   num_seqs              B: sequences per run (page-table rows, seq_lens entries)
 *   num_q_heads           Hq; num_kv_heads Hkv; Hq % Hkv == 0, G = Hq/Hkv in {1,2,4,8,16,32}
 *   head_dim              D in {64, 128, 256}
 *   page_size             tokens per page, in {16, 32, 64, 128}
 *   num_pages             P: physical pages in each pool (bounds the page ids)
 *   page_table_cols       C: logical pages per sequence; seq_lens[b] <= C * page_size
 *   page_table_row_stride elements between page-table rows, >= C (e.g. 2C for the
 *                         K plane of a [B, 2, C] table)
 *   kv_page_stride        elements between consecutive physical pages of a pool;
 *                         0 means page_size * Hkv * D (dense pool)
 *   max_total_q           upper bound on total query tokens T = cu_q_lens[B]
 *   max_q_len             upper bound on any q_len_b (1 for decode)
 *   max_seq_len           upper bound on any seq_lens[b] (used by the split heuristic;
 *                         0 means C * page_size)
 *   kv_dtype              pa_kv_dtype
 *   num_splits            split-KV factor for decode and mixed runs; 0 = heuristic;
 *                         -1 = balanced decode: pa_run_decode runs one persistent
 *                         workgroup per resident slot, each streaming an equal
 *                         share of all (sequence, KV head) keys, and merges
 *                         items cut between workgroups (a task-scheduled
 *                         decode, as the PrimTS kernels of TensorRT-LLM PR
 *                         #17399 are described in its "Description"); and
 *                         pa_run_mixed runs the task-queue schedule: one
 *                         persistent workgroup per resident slot, drawing
 *                         (q-block, KV head) items from a prefill-type and a
 *                         decode-type queue (each sequence's q-blocks
 *                         most-keys-first) until both are empty, never
 *                         splitting keys.  The heuristic (0) picks balanced
 *                         decode wherever it would split, and the task queues
 *                         for mixed runs wherever it would not.
 *   num_cus               compute units to plan for; 0 = query the current device
 *                         (>0 lets plans be built without a GPU)
 *   q_dtype               PA_Q_BF16, or PA_Q_FP8_E4M3: queries arrive as E4M3
 *                         codes with a per-tensor q_descale (fp8 inputs, bf16
 *                         output: the fp8 path of vLLM PR #48156, fp8/descale
 *                         discussion).  Supported for pa_run_prefill with an
 *                         fp8 cache and head dim 64 or 128, where the score
 *                         product runs on the E4M3 matrix cores; other runs of
 *                         such a plan return PA_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;
  int32_t page_table_cols;
  int32_t page_table_row_stride;
  int64_t kv_page_stride;
  int32_t max_total_q;
  int32_t max_q_len;
  int32_t max_seq_len;
  int32_t kv_dtype;
  int32_t num_splits;
  int32_t num_cus;
  int32_t q_dtype;
} pa_desc;

typedef struct pa_plan_s* pa_plan_t;

/*
 * Per-run arguments (device pointers unless stated).
 *   q             bf16 [T, Hq, D], head_dim contiguous, 16-byte aligned
 *   q_stride_t    elements between consecutive tokens of q (0 = Hq*D); multiple of 8
 *   k_pool,v_pool [P, page_size, Hkv, D] of kv_dtype, 16-byte aligned, with
 *                 kv_page_stride elements between pages
 *   page_table    int32 [B, page_table_row_stride]; row b's first
 *                 ceil(seq_lens[b] / page_size) entries are read, nothing else
 *   cu_q_lens     int32 [B+1], cu_q_lens[0] = 0, non-decreasing.  Optional for
 *                 pa_run_decode (NULL means token b belongs to sequence b).
 *   seq_lens      int32 [B], live key count per sequence (0 allowed)
 *   softmax_scale host float multiplying q.k; must be positive and finite
 *                 (PA_ERR_INVALID otherwise).  For fp8 KV, *k_descale must be
 *                 positive as well (device value, not checked).
 *   causal        host flag: 1 = bottom-right aligned causal mask, 0 = none
 *   k_descale, v_descale  device fp32 scalars; required for PA_KV_FP8_E4M3 and
 *                 ignored for PA_KV_BF16
 *   out           bf16 [T, Hq, D], 16-byte aligned
 *   o_stride_t    elements between consecutive tokens of out (0 = Hq*D); multiple of 8
 *   lse           fp32 [T, Hq] natural-log LSE, or NULL to skip.  Rows with no
 *                 visible key get O = 0 and LSE = -inf.
 *   workspace     device scratch of at least pa_workspace_bytes(plan) bytes,
 *                 256-byte aligned; may be NULL when that size is 0
 *   q_descale     device fp32 scalar, required when the plan's q_dtype is
 *                 PA_Q_FP8_E4M3 (query value = code * q_descale), else ignored;
 *                 fp8 queries also need q 16-byte aligned and q_stride_t a
 *                 multiple of 16
 *   softcap       host float; 0 = off, > 0 = logit soft-capping: each scaled
 *                 score s becomes softcap * tanh(s / softcap) before the mask
 *                 and the softmax (the capped scores of the unified kernel in
 *                 vLLM PR #16828, review thread on the masked-score line).
 *                 Negative, NaN or infinite values give PA_ERR_INVALID.
 */
typedef struct {
  const void* q;
  int64_t q_stride_t;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* cu_q_lens;
  const int32_t* seq_lens;
  float softmax_scale;
  int32_t causal;
  const float* k_descale;
  const float* v_descale;
  void* out;
  int64_t o_stride_t;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  float softcap;
  const float* q_descale;
} pa_args;

/* What a plan chose (for tests and benchmarks). */
typedef struct {
  int32_t num_splits;        /* split-KV factor used by decode and mixed runs */
  int32_t split_keys;        /* keys per split window (multiple of the key tile) */
  int32_t q_block_tokens;    /* query tokens per work item of prefill runs */
  int32_t group;             /* G = Hq / Hkv */
  int32_t num_cus;           /* compute units planned for */
  int32_t mixed_q_block_tokens;  /* query tokens per work item of mixed runs */
  int32_t balanced_workgroups;   /* > 0: balanced decode with this many workgroups */
  size_t workspace_bytes;    /* = pa_workspace_bytes(plan) */
  int32_t queue_workgroups;  /* > 0: mixed runs use the task queues with this many workgroups */
} pa_plan_info;

/* Validate a shape description and build a plan.  Host only; uses the HIP
 * runtime only when desc->num_cus == 0.  Returns PA_ERR_INVALID for malformed
 * descriptions and PA_ERR_UNSUPPORTED for geometry outside the compiled scope
 * (this includes a page of 2^32 bytes or more, kv_page_stride included, and a
 * slot of 2^24 bytes or more, num_kv_heads * head_dim * element size: the
 * kernels address pages with 32-bit products); *out is set only on PA_OK.  One plan per batch shape, metadata bound at run
 * time, unsupported requests refused so the caller can fall back: TensorRT-LLM
 * PR #17399, "Planning, preprocessing, and workspace ownership" and
 * "Integration and supported scope". */
pa_status pa_plan(const pa_desc* desc, pa_plan_t* out);

/* Bytes of workspace a run of this plan needs (0 when no split is used).
 * Prefill runs need none; decode and mixed runs need this much when the plan
 * splits the key range. Returns 0 for a NULL plan.  The caller owns and
 * aligns the workspace, context (prefill) runs need none: TensorRT-LLM PR
 * #17399, "Planning, preprocessing, and workspace ownership". */
size_t pa_workspace_bytes(pa_plan_t plan);

/* Fill *info with the plan's choices. */
pa_status pa_plan_get_info(pa_plan_t plan, pa_plan_info* info);

/* Varlen prefill (any q_len_b <= seq_lens[b], including chunked prefill on
 * cached keys): query heads of one KV head packed into bf16 MFMA tiles, K/V
 * tiles shared through LDS, online softmax.  Never splits the key range and
 * needs no workspace.  The paged prefill specialisation of vLLM PR #48156
 * (summary and kernel micro-benchmark table), with the varlen GQA packing of
 * vLLM PR #16828 (description). */
pa_status pa_run_prefill(pa_plan_t plan, const pa_args* args, hipStream_t stream);

/* Decode: at most one query token per sequence (token b of sequence b when
 * cu_q_lens is NULL).  Split-KV over the plan's num_splits windows (the last
 * window takes every key past the others), then a log-sum-exp merge pass when
 * splits > 1; or, for a balanced plan (num_splits = -1), the balanced
 * persistent schedule and its merge pass.  The paged decode with split-KV of
 * vLLM PR #48156 (split-KV discussion) over the page-table metadata of
 * TensorRT-LLM PR #17399 ("Unified page-table metadata"). */
pa_status pa_run_decode(pa_plan_t plan, const pa_args* args, hipStream_t stream);

/*
 * Decode without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same computation, kernels and arguments as
 * pa_run_decode, except that args->workspace and args->workspace_bytes are
 * ignored: the split partials, balanced-decode records and schedule words live
 * in a static device array of PA_STATIC_SCRATCH_BYTES (32 MiB) inside
 * the library, one copy per device, held until the process ends.  The copy of
 * the current device is used (make the stream's device current); its address
 * is looked up on the first call on each device.  Nothing is allocated and
 * nothing needs to start at zero: every word a run reads is written earlier
 * in the same run.  All calls on one device share the array, so calls that
 * overlap in time on one device (other streams, other threads) race; serialise
 * them.  Returns PA_ERR_SCRATCH, with nothing enqueued, when
 * pa_workspace_bytes(plan) exceeds the array; other errors as pa_run_decode.
 */
#define PA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_run_decode_static(pa_plan_t plan, const pa_args* args, hipStream_t stream);

/* Unified mixed batch: any mix of q_len_b in one main launch.  Short rows
 * (q_len_b * G <= 32) take the decode schedule, longer ones the prefill
 * schedule, both inside the same kernel; split-KV and the merge pass as for
 * decode.  A plan with num_splits = -1 runs the task-queue schedule instead
 * (a one-workgroup setup launch that lays out the queues in the workspace,
 * then the persistent main launch; no merge).  One kernel for any query
 * length: vLLM PR #16828 (description, "Further benchmarking"). */
pa_status pa_run_mixed(pa_plan_t plan, const pa_args* args, hipStream_t stream);

/*
 * KV-cache append (the step before attention): write the K and V rows of a
 * step's new tokens into the paged pools, as the fused preprocessing of
 * TensorRT-LLM PR #17399 does before its kernels run (section "Planning,
 * preprocessing, and workspace ownership": QKV extraction, RoPE, KV-cache
 * append, page metadata).
 *   k_new, v_new  bf16 [T_new, Hkv, D], head_dim contiguous, 16-byte aligned;
 *                 new_stride_t elements between tokens (0 = Hkv*D), multiple of 8
 *   cu_new        int32 [B+1]: sequence b's new tokens are rows
 *                 cu_new[b] .. cu_new[b+1]-1 (cu_new[B] <= the plan's max_total_q)
 *   seq_lens      int32 [B]: lengths AFTER the append; new token i of sequence b
 *                 is position seq_lens[b] - n_b + i (n_b = cu_new[b+1] - cu_new[b]),
 *                 the same "queries are the last tokens" convention as the runs
 *   page_table, k_pool, v_pool  as in pa_args (written, not read, at those
 *                 positions; page ids must be valid for every appended position)
 *   k_descale, v_descale  fp8 pools only: device fp32 scalars; the stored code is
 *                 the E4M3 value nearest to (binary32) value / descale, ties to an
 *                 even mantissa, saturating at +-448 (NaN gives the NaN code, sign kept)
 * Uses the plan's geometry (B, Hkv, D, page size, pool layout, KV dtype); Hq,
 * splits and the workspace play no part.  Nothing else in the pools changes.
 * A token whose position falls outside 0 .. page_table_cols * page - 1, whose
 * page id lies outside [0, num_pages), or whose row is at or past max_total_q,
 * breaks the contract and is skipped (the metadata lives on the device, so no
 * status reports it).  All buffers stay the caller's;
 * the library keeps no pointer past the call.  Asynchronous on `stream`; host-side
 * errors as for the runs (PA_ERR_INVALID for a NULL or misaligned pointer, a
 * stride below Hkv*D or not a multiple of 8, missing fp8 descales).
 */
typedef struct {
  const void* k_new;
  const void* v_new;
  int64_t new_stride_t;
  const int32_t* cu_new;
  const int32_t* seq_lens;
  const int32_t* page_table;
  void* k_pool;
  void* v_pool;
  const float* k_descale;
  const float* v_descale;
} pa_append_args;

pa_status pa_run_append(pa_plan_t plan, const pa_append_args* args, hipStream_t stream);

/*
 * Device-content check of a run's metadata (a debugging aid).  The runs
 * trust what the device arrays hold: a page id outside the pool, a query run
 * longer than its sequence or a sequence longer than its page-table row is
 * undefined behaviour there, as the planning contract of TensorRT-LLM PR
 * #17399 leaves it ("Unified page-table metadata": the page table and live
 * lengths are the caller's).  This call scans the metadata of `args` on
 * `stream` and writes a mask of what it finds into the device int32 *flags
 * (0 = clean); it reads only the metadata (never a page id as an address),
 * allocates nothing and is graph-capturable.  Bits:
 *   PA_CHECK_PAGE_ID    a page-table column that holds live keys names a page
 *                       outside [0, num_pages)
 *   PA_CHECK_Q_LEN      q_len_b > seq_lens[b] > 0 (queries are the last keys)
 *   PA_CHECK_SEQ_LEN    seq_lens[b] < 0 or > page_table_cols * page_size
 *   PA_CHECK_CU_Q_LENS  cu_q_lens decreasing, not starting at 0, or its total
 *                       above the plan's max_total_q
 * Uses page_table, cu_q_lens (NULL: one token per sequence), seq_lens.
 * Returns PA_ERR_INVALID for NULL plan, args or flags, or NULL metadata when
 * num_seqs > 0.
 */
enum {
  PA_CHECK_PAGE_ID = 1,
  PA_CHECK_Q_LEN = 2,
  PA_CHECK_SEQ_LEN = 4,
  PA_CHECK_CU_Q_LENS = 8
};
pa_status pa_check_metadata(pa_plan_t plan, const pa_args* args, int32_t* flags, hipStream_t stream);

/* Release a plan (NULL is ignored).  The plan is the caller's host object,
 * built once per batch shape (TensorRT-LLM PR #17399, "Planning,
 * preprocessing, and workspace ownership"). */
void pa_plan_destroy(pa_plan_t plan);

/*
 * MLA decode (DeepSeek-style multi-head latent attention), the third path of
 * TensorRT-LLM PR #17399 ("Integration and supported scope": BF16 MLA decode,
 * one logical KV head, at most 128 local query heads, KV-LoRA rank 512, RoPE
 * head dimension 64; "Planning, preprocessing, and workspace ownership": MLA
 * sizes only its own scratch).  Each cached token is one 576-wide bf16 row:
 * the 512 compressed latent values, then the 64-wide RoPE key.  For query head
 * h of sequence b (one query token per sequence):
 *   s_j = softmax_scale * q[b][h] . C_j  over all 576 columns, j < seq_lens[b]
 *   (optionally soft-capped), out[b][h] = sum_j softmax_j * C_j[0:512],
 *   lse[b][h] = ln sum_j exp(s_j)
 * i.e. the latent part of the row is both key and value.  Same page-table and
 * seq_lens contract as the other runs.
 *
 * Shape bounds (host only):
 *   num_seqs, num_q_heads (1..128), page_size (16/32/64/128), num_pages,
 *   page_table_cols, page_table_row_stride (>= cols), kv_page_stride
 *   (elements between pages; 0 = page_size * 576), max_seq_len (0 = cols *
 *   page_size), num_splits (0 = heuristic, >= 1 forced, -1 = balanced: one
 *   workgroup per compute unit, each streaming an equal share of all keys,
 *   items cut between workgroups merged afterwards), num_cus (0 = query the
 *   device)
 */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t page_size;
  int32_t num_pages;
  int32_t page_table_cols;
  int32_t page_table_row_stride;
  int64_t kv_page_stride;
  int32_t max_seq_len;
  int32_t num_splits;
  int32_t num_cus;
} pa_mla_desc;

typedef struct pa_mla_plan_s* pa_mla_plan_t;

/*
 * Per-run arguments (device pointers unless stated):
 *   q           bf16 [B, Hq, 576] (absorbed latent query, then RoPE query),
 *               16-byte aligned; q_stride_t elements between sequences
 *               (0 = Hq * 576), multiple of 8
 *   kv_cache    bf16 [P, page_size, 576], 16-byte aligned
 *   page_table  int32 [B, row_stride];  seq_lens int32 [B]
 *   softmax_scale  host float > 0;  softcap host float >= 0 (0 = off)
 *   out         bf16 [B, Hq, 512], 16-byte aligned; o_stride_t elements between
 *               sequences (0 = Hq * 512), multiple of 8
 *   lse         fp32 [B, Hq] natural log, or NULL
 *   workspace   at least pa_mla_workspace_bytes(plan) bytes, 256-byte aligned
 * Errors: PA_ERR_INVALID for NULL/misaligned pointers, bad strides or scales;
 * PA_ERR_WORKSPACE for a missing or short workspace; PA_ERR_HIP for a failed
 * launch.  Asynchronous on `stream`; no allocation, no host synchronisation.
 */
typedef struct {
  const void* q;
  int64_t q_stride_t;
  const void* kv_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float softmax_scale;
  float softcap;
  void* out;
  int64_t o_stride_t;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
} pa_mla_args;

/* Validate an MLA shape description and build its plan (PA_ERR_INVALID,
 * PA_ERR_UNSUPPORTED as for pa_plan). */
pa_status pa_mla_plan(const pa_mla_desc* desc, pa_mla_plan_t* out);
/* Workspace bytes a run of this plan needs (0 when it does not split). */
size_t pa_mla_workspace_bytes(pa_mla_plan_t plan);
/* Split-KV factor the plan chose (-1: the balanced schedule). */
int32_t pa_mla_num_splits(pa_mla_plan_t plan);
/* Run MLA decode: one main launch, plus the log-sum-exp merge when split. */
pa_status pa_run_mla_decode(pa_mla_plan_t plan, const pa_mla_args* args, hipStream_t stream);
/* Release an MLA plan (NULL is ignored). */
void pa_mla_plan_destroy(pa_mla_plan_t plan);

/* Static string naming a status code. */
const char* pa_status_str(pa_status status);

/* ---------------------------------------------------------------------------
 * Measurement (not part of the attention path)
 *
 * The roofline fractions of the prefill lines are taken against the published
 * dense MFMA peaks; these two calls measure the rate this GPU actually
 * sustains when it does nothing but MFMAs on random operands -- bf16
 * (v_mfma_f32_32x32x16_bf16) or, with fp8 = 1, OCP E4M3
 * (v_mfma_scale_f32_32x32x64_f8f6f4 without block scales) -- the practical
 * ceiling of any MFMA-bound kernel here.  The score and PV products they
 * stand for are the dense contractions of the attention definition (vLLM PR
 * #48156, "Residual warmed gap": kernel time attributed by microbenchmark).
 *   operands  device, 16-byte aligned, num_workgroups * 32768 16-bit words
 *             (bf16: 4 waves x 16 operands x 64 lanes x 16 bytes per
 *             workgroup) or num_workgroups * 65536 (fp8: 32-byte operands),
 *             read once; the caller fills them (random values for the ceiling)
 *   sink      device, num_workgroups * 256 floats, written (the accumulators'
 *             sums, so that no product is dead code)
 *   iters     loop trips; each wave issues 64 MFMAs per trip
 *   fp8       0: bf16 operands, 1: E4M3 operands
 * A wave holds about 200 registers: two four-wave workgroups per compute
 * unit are resident at once.
 *   operand_words, sink_floats  the sizes of those two buffers, checked
 *             against what the launch reads and writes
 * Errors: PA_ERR_INVALID for null or misaligned pointers, non-positive sizes,
 * buffers smaller than the launch needs or fp8 outside {0, 1}, PA_ERR_HIP
 * when the launch fails.
 * pa_calibrate_mfma_flops returns the floating-point operations one such
 * launch performs. */
pa_status pa_calibrate_mfma(const uint16_t* operands, int64_t operand_words, float* sink, int64_t sink_floats,
                            int32_t num_workgroups, int32_t iters, int32_t fp8, hipStream_t stream);
double pa_calibrate_mfma_flops(int32_t num_workgroups, int32_t iters, int32_t fp8);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
