// pa_internal.h -- parameters shared by the host side of libpa.so and its HIP kernels.
#ifndef PA_INTERNAL_H
#define PA_INTERNAL_H

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "pa.h"

namespace pa {

// Which work decomposition a launch uses.
//   kDecode : one query token per sequence; grid (B, Hkv, splits); the waves of a
//             workgroup split the key range of one (sequence, KV head, split).
//   kPrefill: grid (q-block bound, Hkv, 1); the waves split the query rows of a
//             q-block and share K/V tiles through LDS.
//   kMixed  : grid (q-block bound, Hkv, splits); each q-block picks the decode
//             schedule when its rows fit one wave (q_len * G <= 32), else the
//             prefill schedule.
enum Mode : int { kDecode = 0, kPrefill = 1, kMixed = 2 };

struct AttnParams {
  const uint16_t* q;            // bf16 bits [T, Hq, D] (E4M3 bytes when q_fp8)
  int64_t q_stride_t;           // elements between tokens
  const uint8_t* k_pool;        // raw element bytes
  const uint8_t* v_pool;
  int64_t kv_page_bytes;        // bytes between physical pages
  const int32_t* page_table;    // [B, pt_row_stride]
  int32_t pt_row_stride;
  int32_t pt_cols;              // C; live keys are clamped to C * page
  const int32_t* cu_q_lens;     // [B+1]; NULL for decode (token b = sequence b)
  const int32_t* seq_lens;      // [B]
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                // G = Hq / Hkv
  int32_t page_shift;           // log2(page size)
  int32_t causal;
  float scale_log2;             // softmax_scale * log2(e)
  float softcap;                // > 0: scaled scores s -> softcap * tanh(s / softcap)
  const float* k_descale;       // fp8 only (device scalar)
  const float* v_descale;
  uint16_t* out;                // bf16 bits [T, Hq, D]
  int64_t o_stride_t;
  float* lse;                   // fp32 [T, Hq] natural log, or NULL
  int32_t num_splits;           // > 1: write partials, merged by merge_kernel
  int32_t split_keys;           // keys per split window (multiple of 64)
  float* part_o;                // [S][max_total_q][Hq][D]
  float* part_lse;              // [S][max_total_q][Hq], log2 units
  int32_t max_total_q;          // rows at or past this token index are not computed
  int32_t q_block_tokens;       // tokens per q-block (prefill / mixed)
  int32_t balanced;             // decode only: persistent balanced schedule (see launch)
  int32_t* sched;               // balanced: [4 + B + 1] ints of workspace (unit offsets)
  int32_t head_groups;          // MLA: groups of up to 64 query heads per item (group = heads per group)
  int32_t q_fp8;                // queries are E4M3 codes (streamed fp8 prefill only)
  const float* q_descale;       // device scalar, fp8 queries
  int32_t queue;                // mixed only: persistent workgroups pull items from
                                // the task queues in sched (queue_sched_ints ints)
};

// Task queues of a mixed launch, in the workspace (int32 words): kQueueCtrs
// draw counters (one per XCD share of the prefill-type list, then the
// decode-type list's, then a spare), kQueueSlots arrival counters (one per
// compute unit id), then the item offsets of each sequence in the
// prefill-type list [B+1] and in the decode-type list [B+1].
constexpr int kQueueShares = 8;                   // XCDs of an MI355X
constexpr int kQueueDecodeCtr = kQueueShares;
constexpr int kQueueCtrs = kQueueShares + 2;
constexpr int kQueueSlots = 1024;
inline int64_t queue_sched_ints(int64_t num_seqs) { return kQueueCtrs + kQueueSlots + 2 * (num_seqs + 1); }

struct QueueSetupParams {
  const int32_t* cu_q_lens;     // [B+1]
  int32_t* sched;               // queue_sched_ints(B) words
  int32_t num_seqs;
  int32_t group;                // G
  int32_t num_kv_heads;
  int32_t q_block_tokens;       // tokens per prefill-type item
};

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  int32_t num_splits;
  int32_t max_total_q;
  int32_t num_q_heads;
  const int32_t* cu_q_lens;     // NULL: total rows = num_seqs (decode)
  int32_t num_seqs;
  uint16_t* out;
  int64_t o_stride_t;
  float* lse;
};

struct AppendParams {
  const uint16_t* k_new;        // bf16 bits [T_new, Hkv, D]
  const uint16_t* v_new;
  int64_t new_stride_t;         // elements between new tokens
  const int32_t* cu_new;        // [B+1]
  const int32_t* seq_lens;      // [B], after the append
  const int32_t* page_table;    // [B, pt_row_stride]
  int32_t pt_row_stride;
  int32_t pt_cols;              // positions at or past C * page are not written
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_shift;
  int32_t max_new;              // token rows at or past this index are not written
  int64_t kv_page_bytes;        // bytes between physical pages
  uint8_t* k_pool;
  uint8_t* v_pool;
  int32_t fp8;
  const float* k_descale;
  const float* v_descale;
  int32_t num_pages;            // page ids outside [0, num_pages) are not written through
};

struct BalancedMergeParams {
  const float* part_o;          // [2 W][G][D], O / l of cut pieces
  const float* part_lse;        // [2 W][G], log2 units
  const int32_t* sched;         // U, total, -, -, S_0 .. S_B (written by the attention kernel)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;         // items per sequence (KV heads, or MLA head groups)
  int32_t rows_per_item;        // query rows of one item (G, or MLA heads per group)
  int32_t max_total_q;
  const int32_t* cu_q_lens;     // NULL: token b = sequence b
  uint16_t* out;
  int64_t o_stride_t;
  float* lse;
};

// Launch the MLA decode kernel (head dim 576 / value dim 512, one KV head) on a
// one-dimensional grid of B * num_splits * head_groups workgroups; partials
// (splits > 1) use the split-KV layout with head dim 512 and are merged by
// launch_merge(512, ...).
hipError_t launch_mla(const AttnParams& p, dim3 grid, hipStream_t stream);
// Launch the merge of balanced decode pieces.
hipError_t launch_merge_balanced(int head_dim, const BalancedMergeParams& p, hipStream_t stream);
hipError_t launch_queue_setup(const QueueSetupParams& p, hipStream_t stream);

struct CheckParams {
  const int32_t* page_table;    // [B, pt_row_stride]
  int32_t pt_row_stride;
  int32_t pt_cols;
  int32_t page_shift;
  int32_t num_pages;
  const int32_t* cu_q_lens;     // [B+1] or NULL (one token per sequence)
  const int32_t* seq_lens;      // [B]
  int32_t num_seqs;
  int32_t max_total_q;
  int32_t* flags;               // device int32 mask
};
hipError_t launch_check(const CheckParams& p, hipStream_t stream);

// Launch the KV-cache append.
hipError_t launch_append(const AppendParams& p, hipStream_t stream);

// The allocation-free decode entry point keeps its scratch in a file-scope
// device array of this many bytes (one copy per device, held until the
// process ends).  static_scratch returns the current device's copy, looked up
// once per device with that device current.
constexpr size_t kStaticScratchBytes = PA_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** ptr);

// Launch the attention kernel instance for (head_dim, kv dtype, mode).
hipError_t launch_attention(int head_dim, bool kv_fp8, Mode mode, const AttnParams& p,
                            dim3 grid, hipStream_t stream);
// Launch the split-KV log-sum-exp merge.
hipError_t launch_merge(int head_dim, const MergeParams& p, hipStream_t stream);
// LDS bytes the attention instance uses (host-side check).
int attention_lds_bytes(int head_dim, bool kv_fp8, Mode mode);
// Workgroups of the attention instance that fit on one compute unit at once
// (by LDS and by waves per SIMD).
int workgroups_per_cu(int head_dim, bool kv_fp8, Mode mode);
// Packed query rows (tokens x GQA heads) per workgroup of a launch mode.
int block_rows(int head_dim, Mode mode, bool q_fp8 = false);

}  // namespace pa

#endif  // PA_INTERNAL_H
