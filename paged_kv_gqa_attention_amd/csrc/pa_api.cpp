// pa_api.cpp -- the C ABI of libpa.so: plan validation, split choice, launches.
//
// The plan/run split, the caller-owned workspace and the fail-closed scope
// follow TensorRT-LLM PR #17399 ("integrate PrimTS FMHA kernels", sections
// "Planning, preprocessing, and workspace ownership" and "Integration and
// supported scope"); num_splits = 0 meaning "choose by heuristic" follows the
// split-KV discussion of vLLM PR #48156 ("[Perf][FA4] Warm up dense (paged)
// FA4 attention kernels").  No function here reads device memory, allocates
// device memory or synchronises a stream.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kSplitAlign = 128;          // split windows: whole 64-key tiles, page aligned
constexpr int kMinSplitKeys = 1024;       // do not split below this many keys per window
constexpr size_t kWsAlign = 256;

int ilog2(int64_t x) { int s = 0; while ((int64_t(1) << s) < x) ++s; return s; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct pa_plan_s {
  pa_desc d;
  int32_t group;
  int32_t page_shift;
  int32_t esz;
  int32_t num_splits;
  int32_t split_keys;
  int32_t q_block_tokens;          // prefill launches
  int32_t mixed_q_block_tokens;    // mixed launches
  int32_t num_cus;
  int32_t rows_cap;          // token rows the partial buffers are laid out for
  int64_t kv_page_bytes;
  int32_t balanced_wgs;      // > 0: decode runs use the balanced persistent schedule
  int32_t queue_wgs;         // > 0: mixed runs use the task queues
  size_t part_o_bytes;       // split-KV layout: partial O, then partial LSE
  size_t bal_part_o_bytes;   // balanced layout: partial O, partial LSE, schedule
  size_t bal_part_lse_bytes;
  size_t ws_bytes;
};

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID: return "PA_ERR_INVALID: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: geometry outside the supported scope";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime or launch failure";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the plan needs more scratch than pa_run_decode_static's static array holds";
  }
  return "unknown pa_status";
}

pa_status pa_plan(const pa_desc* desc, pa_plan_t* out) {
  if (!desc || !out) return PA_ERR_INVALID;
  const pa_desc& d = *desc;
  if (d.num_seqs < 0 || d.num_q_heads <= 0 || d.num_kv_heads <= 0 || d.head_dim <= 0 ||
      d.page_size <= 0 || d.num_pages < 0 || d.page_table_cols < 0 ||
      d.page_table_row_stride < d.page_table_cols || d.kv_page_stride < 0 ||
      d.max_total_q < 0 || d.max_q_len < 0 || d.max_seq_len < 0 || d.num_splits < -1 ||
      d.num_cus < 0)
    return PA_ERR_INVALID;
  if (d.num_q_heads % d.num_kv_heads != 0) return PA_ERR_INVALID;
  if (d.kv_dtype != PA_KV_BF16 && d.kv_dtype != PA_KV_FP8_E4M3) return PA_ERR_INVALID;
  if (d.q_dtype != PA_Q_BF16 && d.q_dtype != PA_Q_FP8_E4M3) return PA_ERR_INVALID;
  const int G = d.num_q_heads / d.num_kv_heads;
  // compiled scope (fail closed)
  if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32)) return PA_ERR_UNSUPPORTED;
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (d.page_size != 16 && d.page_size != 32 && d.page_size != 64 && d.page_size != 128)
    return PA_ERR_UNSUPPORTED;
  // fp8 queries: the streamed prefill of an fp8 cache (head dim <= 128) only
  if (d.q_dtype == PA_Q_FP8_E4M3 && (d.kv_dtype != PA_KV_FP8_E4M3 || d.head_dim > 128))
    return PA_ERR_UNSUPPORTED;
  const int esz = d.kv_dtype == PA_KV_FP8_E4M3 ? 1 : 2;
  const int64_t dense_page = (int64_t)d.page_size * d.num_kv_heads * d.head_dim;
  const int64_t page_elems = d.kv_page_stride ? d.kv_page_stride : dense_page;
  if (page_elems < dense_page || (page_elems * esz) % 16 != 0) return PA_ERR_INVALID;
  // the kernels form a page base as a 32 x 32 -> 64-bit product and the
  // offset of a slot inside its page with a 24-bit multiply
  if (page_elems * esz >= (int64_t(1) << 32)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)d.num_kv_heads * d.head_dim * esz >= (int64_t(1) << 24)) return PA_ERR_UNSUPPORTED;
  const int64_t capacity = (int64_t)d.page_table_cols * d.page_size;
  if (capacity > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  if (d.max_seq_len > capacity) return PA_ERR_INVALID;

  int cus = d.num_cus;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return PA_ERR_HIP;
    if (cus <= 0) return PA_ERR_HIP;
  }

  pa_plan_s* p = new (std::nothrow) pa_plan_s;
  if (!p) return PA_ERR_INVALID;
  p->d = d;
  p->group = G;
  p->page_shift = ilog2(d.page_size);
  p->esz = esz;
  p->num_cus = cus;
  p->q_block_tokens = std::max(1, pa::block_rows(d.head_dim, pa::kPrefill, d.q_dtype == PA_Q_FP8_E4M3) / G);
  p->mixed_q_block_tokens = std::max(1, pa::block_rows(d.head_dim, pa::kMixed) / G);
  p->kv_page_bytes = page_elems * esz;
  p->rows_cap = std::max(d.max_total_q, d.num_seqs);

  // Split-KV factor.  Work items of a decode/mixed launch: one per (q-block,
  // KV head).  Split until every compute unit has about two rounds of the
  // workgroups it holds at once (each split adds a workgroup prologue and
  // partial-result traffic; fewer leave the tail unbalanced), but never into
  // windows shorter than kMinSplitKeys keys.
  const int64_t max_len = d.max_seq_len ? d.max_seq_len : capacity;
  int splits = d.num_splits;
  if (splits <= 0) {
    const int64_t qblocks = std::max<int64_t>(1, ceil_div(d.max_total_q, p->mixed_q_block_tokens));
    const int64_t items = std::max<int64_t>(1, std::max<int64_t>(d.num_seqs, qblocks)) * d.num_kv_heads;
    const int64_t resident = pa::workgroups_per_cu(d.head_dim, d.kv_dtype == PA_KV_FP8_E4M3, pa::kDecode);
    const int64_t want = ceil_div(2 * resident * (int64_t)cus, items);
    const int64_t by_len = std::max<int64_t>(1, max_len / kMinSplitKeys);
    splits = (int)std::max<int64_t>(1, std::min(want, by_len));
  }
  // windows laid over the longest live sequence the plan expects; the last
  // window takes every key past the others (longer sequences stay correct)
  int64_t split_keys = max_len > 0 ? ceil_div(max_len, splits) : kSplitAlign;
  split_keys = std::max<int64_t>(kSplitAlign, ceil_div(split_keys, kSplitAlign) * kSplitAlign);
  splits = (int)std::max<int64_t>(1, max_len > 0 ? ceil_div(max_len, split_keys) : 1);
  p->num_splits = splits;
  p->split_keys = (int32_t)split_keys;
  if (splits > 1) {
    const size_t rows = (size_t)splits * (size_t)p->rows_cap * (size_t)d.num_q_heads;
    p->part_o_bytes = align_up(rows * (size_t)d.head_dim * sizeof(float), kWsAlign);
    p->ws_bytes = p->part_o_bytes + align_up(rows * sizeof(float), kWsAlign);
  } else {
    p->part_o_bytes = 0;
    p->ws_bytes = 0;
  }
  // Balanced decode: requested (-1), or chosen by the heuristic wherever it
  // splits, i.e. where (sequence, KV head) items are too few to fill the
  // device in balanced rounds.  One persistent workgroup per resident slot;
  // its workspace layout is used by decode runs only, the split layout by
  // mixed runs, so the workspace is the larger of the two.
  p->balanced_wgs = 0;
  p->bal_part_o_bytes = 0;
  p->bal_part_lse_bytes = 0;
  if (d.num_splits == -1 || (d.num_splits == 0 && splits > 1)) {
    const int resident = pa::workgroups_per_cu(d.head_dim, d.kv_dtype == PA_KV_FP8_E4M3, pa::kDecode);
    const int64_t W = (int64_t)resident * cus;
    const size_t recs = (size_t)(2 * W) * (size_t)G;
    p->balanced_wgs = (int32_t)W;
    p->bal_part_o_bytes = align_up(recs * (size_t)d.head_dim * sizeof(float), kWsAlign);
    p->bal_part_lse_bytes = align_up(recs * sizeof(float), kWsAlign);
    const size_t bal = p->bal_part_o_bytes + p->bal_part_lse_bytes +
                       align_up((size_t)(4 + d.num_seqs + 1) * sizeof(int32_t), kWsAlign);
    p->ws_bytes = std::max(p->ws_bytes, bal);
  }
  // Task-queue mixed runs: requested (-1), or chosen by the heuristic wherever
  // it does not split (enough items to fill the device; measured 3-9 % faster
  // than one workgroup per item on the 1000-token serving mix).  One
  // persistent workgroup per resident slot of the mixed kernel; the queues
  // live in the workspace.
  p->queue_wgs = 0;
  if (d.num_splits == -1 || (d.num_splits == 0 && splits == 1)) {
    p->queue_wgs = pa::workgroups_per_cu(d.head_dim, d.kv_dtype == PA_KV_FP8_E4M3, pa::kMixed) * cus;
    p->ws_bytes = std::max(p->ws_bytes, align_up((size_t)pa::queue_sched_ints(d.num_seqs) * sizeof(int32_t), kWsAlign));
  }
  *out = p;
  return PA_OK;
}

size_t pa_workspace_bytes(pa_plan_t plan) { return plan ? plan->ws_bytes : 0; }

pa_status pa_plan_get_info(pa_plan_t plan, pa_plan_info* info) {
  if (!plan || !info) return PA_ERR_INVALID;
  std::memset(info, 0, sizeof(*info));
  info->num_splits = plan->num_splits;
  info->split_keys = plan->split_keys;
  info->q_block_tokens = plan->q_block_tokens;
  info->mixed_q_block_tokens = plan->mixed_q_block_tokens;
  info->group = plan->group;
  info->num_cus = plan->num_cus;
  info->balanced_workgroups = plan->balanced_wgs;
  info->queue_workgroups = plan->queue_wgs;
  info->workspace_bytes = plan->ws_bytes;
  return PA_OK;
}

pa_status pa_check_metadata(pa_plan_t plan, const pa_args* a, int32_t* flags, hipStream_t stream) {
  if (!plan || !a || !flags) return PA_ERR_INVALID;
  const pa_desc& d = plan->d;
  if (d.num_seqs > 0 && (!a->page_table || !a->seq_lens)) return PA_ERR_INVALID;
  pa::CheckParams q;
  q.page_table = a->page_table;
  q.pt_row_stride = d.page_table_row_stride;
  q.pt_cols = d.page_table_cols;
  q.page_shift = plan->page_shift;
  q.num_pages = d.num_pages;
  q.cu_q_lens = a->cu_q_lens;
  q.seq_lens = a->seq_lens;
  q.num_seqs = d.num_seqs;
  q.max_total_q = plan->rows_cap;
  q.flags = flags;
  return pa::launch_check(q, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_run_append(pa_plan_t plan, const pa_append_args* a, hipStream_t stream) {
  if (!plan || !a) return PA_ERR_INVALID;
  const pa_desc& d = plan->d;
  if (d.num_seqs == 0) return PA_OK;
  const bool fp8 = d.kv_dtype == PA_KV_FP8_E4M3;
  const int64_t row = (int64_t)d.num_kv_heads * d.head_dim;
  const int64_t stride = a->new_stride_t ? a->new_stride_t : row;
  if (!a->k_new || !a->v_new || !a->cu_new || !a->seq_lens || !a->page_table || !a->k_pool || !a->v_pool)
    return PA_ERR_INVALID;
  if (!aligned16(a->k_new) || !aligned16(a->v_new) || !aligned16(a->k_pool) ||
      !aligned16(a->v_pool))
    return PA_ERR_INVALID;
  if (stride < row || stride % 8) return PA_ERR_INVALID;
  if (fp8 && (!a->k_descale || !a->v_descale)) return PA_ERR_INVALID;
  pa::AppendParams p;
  std::memset(&p, 0, sizeof(p));
  p.k_new = static_cast<const uint16_t*>(a->k_new);
  p.v_new = static_cast<const uint16_t*>(a->v_new);
  p.new_stride_t = stride;
  p.cu_new = a->cu_new;
  p.seq_lens = a->seq_lens;
  p.page_table = a->page_table;
  p.pt_row_stride = d.page_table_row_stride;
  p.pt_cols = d.page_table_cols;
  p.num_seqs = d.num_seqs;
  p.num_kv_heads = d.num_kv_heads;
  p.head_dim = d.head_dim;
  p.page_shift = plan->page_shift;
  p.max_new = plan->rows_cap;
  p.kv_page_bytes = plan->kv_page_bytes;
  p.k_pool = static_cast<uint8_t*>(a->k_pool);
  p.v_pool = static_cast<uint8_t*>(a->v_pool);
  p.fp8 = fp8 ? 1 : 0;
  p.k_descale = fp8 ? a->k_descale : nullptr;
  p.v_descale = fp8 ? a->v_descale : nullptr;
  p.num_pages = d.num_pages;
  return pa::launch_append(p, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

void pa_plan_destroy(pa_plan_t plan) { delete plan; }

}  // extern "C"

namespace {

// Host-side checks shared by the three runs; fills the kernel parameters.
pa_status prepare(pa_plan_t plan, const pa_args* a, pa::Mode mode, bool use_splits,
                  pa::AttnParams* kp) {
  if (!plan || !a) return PA_ERR_INVALID;
  const pa_desc& d = plan->d;
  const bool fp8 = d.kv_dtype == PA_KV_FP8_E4M3;
  const bool q_fp8 = d.q_dtype == PA_Q_FP8_E4M3;
  if (q_fp8 && mode != pa::kPrefill) return PA_ERR_UNSUPPORTED;
  const int64_t row = (int64_t)d.num_q_heads * d.head_dim;
  const int64_t q_stride = a->q_stride_t ? a->q_stride_t : row;
  const int64_t o_stride = a->o_stride_t ? a->o_stride_t : row;
  if (d.num_seqs > 0) {
    if (!a->q || !a->k_pool || !a->v_pool || !a->page_table || !a->seq_lens || !a->out)
      return PA_ERR_INVALID;
    if (mode != pa::kDecode && !a->cu_q_lens) return PA_ERR_INVALID;
    if (!aligned16(a->q) || !aligned16(a->k_pool) || !aligned16(a->v_pool) || !aligned16(a->out))
      return PA_ERR_INVALID;
    if (fp8 && (!a->k_descale || !a->v_descale)) return PA_ERR_INVALID;
    if (q_fp8 && !a->q_descale) return PA_ERR_INVALID;
  }
  if (q_stride < row || o_stride < row || q_stride % 8 || o_stride % 8) return PA_ERR_INVALID;
  if (q_fp8 && q_stride % 16) return PA_ERR_INVALID;      // 16-byte query rows
  // the kernels fold the scale into exp2 arguments and need it positive and finite
  if (!(a->softmax_scale > 0.f) || !(a->softmax_scale < 3.0e38f)) return PA_ERR_INVALID;
  if (!(a->softcap >= 0.f) || !(a->softcap < 3.0e38f)) return PA_ERR_INVALID;
  const bool balanced = mode == pa::kDecode && plan->balanced_wgs > 0;
  const bool queue = mode == pa::kMixed && plan->queue_wgs > 0;
  const bool split = use_splits && !queue && plan->num_splits > 1;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  int32_t* sched = nullptr;
  if (queue && d.num_seqs > 0) {
    if (!a->workspace || a->workspace_bytes < plan->ws_bytes) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->workspace) & (kWsAlign - 1)) != 0) return PA_ERR_INVALID;
    sched = static_cast<int32_t*>(a->workspace);
  } else if (balanced && d.num_seqs > 0) {
    if (!a->workspace || a->workspace_bytes < plan->ws_bytes) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->workspace) & (kWsAlign - 1)) != 0) return PA_ERR_INVALID;
    char* ws = static_cast<char*>(a->workspace);
    part_o = reinterpret_cast<float*>(ws);
    part_lse = reinterpret_cast<float*>(ws + plan->bal_part_o_bytes);
    sched = reinterpret_cast<int32_t*>(ws + plan->bal_part_o_bytes + plan->bal_part_lse_bytes);
  } else if (split) {
    if (!a->workspace || a->workspace_bytes < plan->ws_bytes) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->workspace) & (kWsAlign - 1)) != 0) return PA_ERR_INVALID;
    part_o = static_cast<float*>(a->workspace);
    part_lse = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + plan->part_o_bytes);
  }
  pa::AttnParams& p = *kp;
  std::memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_stride_t = q_stride;
  p.k_pool = static_cast<const uint8_t*>(a->k_pool);
  p.v_pool = static_cast<const uint8_t*>(a->v_pool);
  p.kv_page_bytes = plan->kv_page_bytes;
  p.page_table = a->page_table;
  p.pt_row_stride = d.page_table_row_stride;
  p.pt_cols = d.page_table_cols;
  p.cu_q_lens = a->cu_q_lens;
  p.seq_lens = a->seq_lens;
  p.num_seqs = d.num_seqs;
  p.num_q_heads = d.num_q_heads;
  p.num_kv_heads = d.num_kv_heads;
  p.group = plan->group;
  p.page_shift = plan->page_shift;
  p.causal = a->causal ? 1 : 0;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.softcap = a->softcap;
  p.k_descale = fp8 ? a->k_descale : nullptr;
  p.v_descale = fp8 ? a->v_descale : nullptr;
  p.out = static_cast<uint16_t*>(a->out);
  p.o_stride_t = o_stride;
  p.lse = a->lse;
  p.num_splits = split ? plan->num_splits : 1;
  p.split_keys = split ? plan->split_keys : INT32_MAX / 2;
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.max_total_q = plan->rows_cap;
  p.q_block_tokens = mode == pa::kPrefill ? plan->q_block_tokens : plan->mixed_q_block_tokens;
  p.balanced = balanced ? 1 : 0;
  p.queue = queue ? 1 : 0;
  p.sched = sched;
  p.q_fp8 = q_fp8 ? 1 : 0;
  p.q_descale = q_fp8 ? a->q_descale : nullptr;
  return PA_OK;
}

pa_status launch(pa_plan_t plan, const pa::AttnParams& p, pa::Mode mode, hipStream_t stream) {
  const pa_desc& d = plan->d;
  if (d.num_seqs == 0) return PA_OK;
  const bool fp8 = d.kv_dtype == PA_KV_FP8_E4M3;
  if (p.balanced) {
    const dim3 grid((unsigned)plan->balanced_wgs, 1, 1);
    if (pa::launch_attention(d.head_dim, fp8, mode, p, grid, stream) != hipSuccess) return PA_ERR_HIP;
    pa::BalancedMergeParams m;
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.sched = p.sched;
    m.num_seqs = d.num_seqs;
    m.num_q_heads = d.num_q_heads;
    m.num_kv_heads = d.num_kv_heads;
    m.rows_per_item = plan->group;
    m.max_total_q = p.max_total_q;
    m.cu_q_lens = p.cu_q_lens;
    m.out = p.out;
    m.o_stride_t = p.o_stride_t;
    m.lse = p.lse;
    return pa::launch_merge_balanced(d.head_dim, m, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  if (p.queue) {
    pa::QueueSetupParams q;
    q.cu_q_lens = p.cu_q_lens;
    q.sched = p.sched;
    q.num_seqs = d.num_seqs;
    q.group = plan->group;
    q.num_kv_heads = d.num_kv_heads;
    q.q_block_tokens = p.q_block_tokens;
    if (pa::launch_queue_setup(q, stream) != hipSuccess) return PA_ERR_HIP;
    const dim3 grid((unsigned)plan->queue_wgs, 1, 1);
    return pa::launch_attention(d.head_dim, fp8, mode, p, grid, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  dim3 grid;
  if (mode == pa::kDecode) {
    grid = dim3((unsigned)d.num_seqs, (unsigned)d.num_kv_heads, (unsigned)p.num_splits);
  } else {
    const int64_t blocks = (int64_t)plan->rows_cap / p.q_block_tokens + d.num_seqs;
    grid = dim3((unsigned)blocks, (unsigned)d.num_kv_heads, (unsigned)p.num_splits);
  }
  if (pa::launch_attention(d.head_dim, fp8, mode, p, grid, stream) != hipSuccess) return PA_ERR_HIP;
  if (p.num_splits > 1) {
    pa::MergeParams m;
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.num_splits = p.num_splits;
    m.max_total_q = p.max_total_q;
    m.num_q_heads = d.num_q_heads;
    m.cu_q_lens = p.cu_q_lens;
    m.num_seqs = d.num_seqs;
    m.out = p.out;
    m.o_stride_t = p.o_stride_t;
    m.lse = p.lse;
    if (pa::launch_merge(d.head_dim, m, stream) != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

pa_status run(pa_plan_t plan, const pa_args* args, hipStream_t stream, pa::Mode mode) {
  pa::AttnParams p;
  const pa_status st = prepare(plan, args, mode, mode != pa::kPrefill, &p);
  if (st != PA_OK) return st;
  return launch(plan, p, mode, stream);
}

}  // namespace

extern "C" {

pa_status pa_run_prefill(pa_plan_t plan, const pa_args* args, hipStream_t stream) {
  return run(plan, args, stream, pa::kPrefill);
}

pa_status pa_run_decode(pa_plan_t plan, const pa_args* args, hipStream_t stream) {
  if (plan && plan->d.max_q_len > 1) return PA_ERR_INVALID;
  return run(plan, args, stream, pa::kDecode);
}

pa_status pa_run_mixed(pa_plan_t plan, const pa_args* args, hipStream_t stream) {
  return run(plan, args, stream, pa::kMixed);
}

pa_status pa_run_decode_static(pa_plan_t plan, const pa_args* args, hipStream_t stream) {
  if (!plan || !args) return PA_ERR_INVALID;
  if (plan->d.max_q_len > 1) return PA_ERR_INVALID;
  if (plan->ws_bytes > pa::kStaticScratchBytes) return PA_ERR_SCRATCH;
  void* scratch = nullptr;
  if (pa::static_scratch(&scratch) != hipSuccess) return PA_ERR_HIP;
  pa_args a = *args;
  a.workspace = scratch;
  a.workspace_bytes = pa::kStaticScratchBytes;
  return run(plan, &a, stream, pa::kDecode);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// MLA decode
// ---------------------------------------------------------------------------

namespace {
constexpr int kMlaDk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaMinSplitKeys = 256;     // a window of at least 8 key tiles
}  // namespace

struct pa_mla_plan_s {
  pa_mla_desc d;
  int32_t page_shift;
  int32_t num_splits;
  int32_t split_keys;
  int32_t head_groups;
  int32_t group;              // query heads per head group
  int32_t balanced_wgs;       // > 0: balanced schedule with this many workgroups
  int64_t kv_page_bytes;
  size_t part_o_bytes;
  size_t part_lse_bytes;      // balanced layout only
  size_t ws_bytes;
};

extern "C" {

pa_status pa_mla_plan(const pa_mla_desc* desc, pa_mla_plan_t* out) {
  if (!desc || !out) return PA_ERR_INVALID;
  const pa_mla_desc& d = *desc;
  if (d.num_seqs < 0 || d.num_q_heads <= 0 || d.page_size <= 0 || d.num_pages < 0 ||
      d.page_table_cols < 0 || d.page_table_row_stride < d.page_table_cols || d.kv_page_stride < 0 ||
      d.max_seq_len < 0 || d.num_splits < -1 || d.num_cus < 0)
    return PA_ERR_INVALID;
  if (d.num_q_heads > 128) return PA_ERR_UNSUPPORTED;
  if (d.page_size != 16 && d.page_size != 32 && d.page_size != 64 && d.page_size != 128)
    return PA_ERR_UNSUPPORTED;
  const int64_t dense_page = (int64_t)d.page_size * kMlaDk;
  const int64_t page_elems = d.kv_page_stride ? d.kv_page_stride : dense_page;
  if (page_elems < dense_page || (page_elems * 2) % 16 != 0) return PA_ERR_INVALID;
  if (page_elems * 2 >= (int64_t(1) << 32)) return PA_ERR_UNSUPPORTED;   // 32-bit page bytes
  const int64_t capacity = (int64_t)d.page_table_cols * d.page_size;
  if (capacity > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  if (d.max_seq_len > capacity) return PA_ERR_INVALID;
  int cus = d.num_cus;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return PA_ERR_HIP;
    if (cus <= 0) return PA_ERR_HIP;
  }
  pa_mla_plan_s* p = new (std::nothrow) pa_mla_plan_s;
  if (!p) return PA_ERR_INVALID;
  p->d = d;
  p->page_shift = ilog2(d.page_size);
  p->kv_page_bytes = page_elems * 2;
  p->head_groups = d.num_q_heads <= 64 ? 1 : (int32_t)ceil_div(d.num_q_heads, 64);
  p->group = d.num_q_heads <= 64 ? d.num_q_heads : 64;
  p->balanced_wgs = 0;
  p->part_lse_bytes = 0;
  if (d.num_splits == -1) {
    // Balanced schedule: one workgroup per compute unit, equal key shares
    // over all (sequence, head group) items; two partial records of `group`
    // rows per workgroup, then the unit offsets.
    p->balanced_wgs = cus;
    p->num_splits = 1;
    p->split_keys = (int32_t)std::max<int64_t>(capacity, kSplitAlign);
    const size_t recs = (size_t)2 * cus * (size_t)p->group;
    p->part_o_bytes = align_up(recs * kMlaDv * sizeof(float), kWsAlign);
    p->part_lse_bytes = align_up(recs * sizeof(float), kWsAlign);
    p->ws_bytes = p->part_o_bytes + p->part_lse_bytes +
                  align_up((size_t)(4 + d.num_seqs + 1) * sizeof(int32_t), kWsAlign);
    *out = p;
    return PA_OK;
  }
  // Split so that the items (sequence, window, head group) fill the device in
  // one round (one workgroup fits on a compute unit; a partial second round
  // measured slower than fewer, longer windows), in windows of at least
  // kMlaMinSplitKeys keys.
  const int64_t max_len = d.max_seq_len ? d.max_seq_len : capacity;
  int splits = d.num_splits;
  if (splits == 0) {
    const int64_t items = std::max<int64_t>(1, (int64_t)d.num_seqs * p->head_groups);
    const int64_t want = std::max<int64_t>(1, (int64_t)cus / items);
    const int64_t by_len = std::max<int64_t>(1, max_len / kMlaMinSplitKeys);
    splits = (int)std::max<int64_t>(1, std::min(want, by_len));
  }
  const int64_t span = std::max<int64_t>(max_len, 1);
  int64_t split_keys = ceil_div(span, splits);
  split_keys = std::max<int64_t>(kSplitAlign, ceil_div(split_keys, kSplitAlign) * kSplitAlign);
  splits = (int)std::max<int64_t>(1, ceil_div(span, split_keys));
  p->num_splits = splits;
  p->split_keys = (int32_t)(splits > 1 ? split_keys : std::max<int64_t>(capacity, kSplitAlign));
  if (splits > 1) {
    const size_t rows = (size_t)splits * (size_t)d.num_seqs * (size_t)d.num_q_heads;
    p->part_o_bytes = align_up(rows * kMlaDv * sizeof(float), kWsAlign);
    p->ws_bytes = p->part_o_bytes + align_up(rows * sizeof(float), kWsAlign);
  } else {
    p->part_o_bytes = 0;
    p->ws_bytes = 0;
  }
  *out = p;
  return PA_OK;
}

size_t pa_mla_workspace_bytes(pa_mla_plan_t plan) { return plan ? plan->ws_bytes : 0; }

int32_t pa_mla_num_splits(pa_mla_plan_t plan) {
  if (!plan) return 0;
  return plan->balanced_wgs > 0 ? -1 : plan->num_splits;
}

pa_status pa_run_mla_decode(pa_mla_plan_t plan, const pa_mla_args* a, hipStream_t stream) {
  if (!plan || !a) return PA_ERR_INVALID;
  const pa_mla_desc& d = plan->d;
  const int64_t qrow = (int64_t)d.num_q_heads * kMlaDk;
  const int64_t orow = (int64_t)d.num_q_heads * kMlaDv;
  const int64_t q_stride = a->q_stride_t ? a->q_stride_t : qrow;
  const int64_t o_stride = a->o_stride_t ? a->o_stride_t : orow;
  if (q_stride < qrow || o_stride < orow || q_stride % 8 || o_stride % 8) return PA_ERR_INVALID;
  if (!(a->softmax_scale > 0.f) || !(a->softmax_scale < 3.0e38f)) return PA_ERR_INVALID;
  if (!(a->softcap >= 0.f) || !(a->softcap < 3.0e38f)) return PA_ERR_INVALID;
  if (d.num_seqs == 0) return PA_OK;
  if (!a->q || !a->kv_cache || !a->page_table || !a->seq_lens || !a->out) return PA_ERR_INVALID;
  if (!aligned16(a->q) || !aligned16(a->kv_cache) || !aligned16(a->out)) return PA_ERR_INVALID;
  const bool balanced = plan->balanced_wgs > 0;
  const bool split = plan->num_splits > 1;
  if (split || balanced) {
    if (!a->workspace || a->workspace_bytes < plan->ws_bytes) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(a->workspace) & (kWsAlign - 1)) != 0) return PA_ERR_INVALID;
  }
  pa::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = static_cast<const uint16_t*>(a->q);
  p.q_stride_t = q_stride;
  p.k_pool = static_cast<const uint8_t*>(a->kv_cache);
  p.v_pool = p.k_pool;
  p.kv_page_bytes = plan->kv_page_bytes;
  p.page_table = a->page_table;
  p.pt_row_stride = d.page_table_row_stride;
  p.pt_cols = d.page_table_cols;
  p.seq_lens = a->seq_lens;
  p.num_seqs = d.num_seqs;
  p.num_q_heads = d.num_q_heads;
  p.num_kv_heads = 1;
  p.group = d.num_q_heads;
  p.page_shift = plan->page_shift;
  p.causal = 1;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.softcap = a->softcap;
  p.out = static_cast<uint16_t*>(a->out);
  p.o_stride_t = o_stride;
  p.lse = a->lse;
  p.num_splits = plan->num_splits;
  p.split_keys = plan->split_keys;
  p.max_total_q = d.num_seqs;
  p.head_groups = plan->head_groups;
  p.group = plan->group;
  if (split || balanced) {
    char* ws = static_cast<char*>(a->workspace);
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_lse = reinterpret_cast<float*>(ws + plan->part_o_bytes);
  }
  if (balanced) {
    p.balanced = 1;
    p.sched = reinterpret_cast<int32_t*>(static_cast<char*>(a->workspace) + plan->part_o_bytes +
                                         plan->part_lse_bytes);
    if (pa::launch_mla(p, dim3((unsigned)plan->balanced_wgs, 1, 1), stream) != hipSuccess) return PA_ERR_HIP;
    pa::BalancedMergeParams m;
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.sched = p.sched;
    m.num_seqs = d.num_seqs;
    m.num_q_heads = d.num_q_heads;
    m.num_kv_heads = plan->head_groups;
    m.rows_per_item = plan->group;
    m.max_total_q = d.num_seqs;
    m.cu_q_lens = nullptr;
    m.out = p.out;
    m.o_stride_t = p.o_stride_t;
    m.lse = p.lse;
    return pa::launch_merge_balanced(kMlaDv, m, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  const int64_t blocks = (int64_t)d.num_seqs * plan->num_splits * plan->head_groups;
  if (blocks > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (pa::launch_mla(p, dim3((unsigned)blocks, 1, 1), stream) != hipSuccess) return PA_ERR_HIP;
  if (split) {
    pa::MergeParams m;
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.num_splits = p.num_splits;
    m.max_total_q = p.max_total_q;
    m.num_q_heads = d.num_q_heads;
    m.cu_q_lens = nullptr;
    m.num_seqs = d.num_seqs;
    m.out = p.out;
    m.o_stride_t = p.o_stride_t;
    m.lse = p.lse;
    if (pa::launch_merge(kMlaDv, m, stream) != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

void pa_mla_plan_destroy(pa_mla_plan_t plan) { delete plan; }

}  // extern "C"
