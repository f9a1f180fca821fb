// pa_kernels.hip -- paged-KV grouped-query attention kernels for gfx950 (MI355X).
//
// One kernel template covers prefill, decode and mixed batches.  The math per
// (query row, key) pair is the varlen masked-softmax attention of vLLM PR
// #16828 ("Unified Triton kernel that doesn't distinguish between prefill +
// decode": any query length in one kernel, GQA heads packed along the query
// dimension, masked scores selected to -inf), over a KV cache resolved through
// the int32 page table and live seq_lens of TensorRT-LLM PR #17399
// ("integrate PrimTS FMHA kernels", section "Unified page-table metadata").
// The split-KV decode with a log-sum-exp reduction follows the split-KV
// specialisation discussed in vLLM PR #48156 ("[Perf][FA4] Warm up dense
// (paged) FA4 attention kernels"); fp8 KV is dequantised with a descale and
// written out in bf16 as that page describes.
//
// gfx950 design
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K rows are the A operand (32 keys), the packed query rows (up to 32 =
//     tokens x GQA heads) are the B operand.  The 32x32 accumulator then holds,
//     in each lane, 16 keys of ONE query row, so the row max and row sum are a
//     per-lane reduction plus one exchange with lane^32, the running rescale
//     factor is a per-lane scalar, and the probabilities P^T are already in the
//     B-operand layout of the second product O^T += V^T P^T (no shuffle of P).
//   * V stays row-major in LDS; the PV A-operand (8 consecutive keys of one
//     head-dim column per lane) comes from the LDS unit's transposing reads
//     (ds_read_b64_tr_b16 / _tr_b8).  K rows are permuted inside a 32-key
//     score tile so that each lane's probabilities for one PV k-step are
//     exactly those 8 consecutive keys.
//   * fp8 e4m3 K/V stay fp8 in LDS and are widened to bf16 in registers right
//     before each MFMA with v_cvt_scalef32_pk_bf16_fp8 (exact: e4m3 is a subset
//     of bf16); k_descale is folded into the score scale, v_descale into the
//     epilogue.
//   * Decode schedule: the waves of a workgroup take interleaved 32-key
//     sub-tiles of one (sequence, KV head, split), each wave staging its own
//     sub-tile through a private LDS region with register prefetch of the next
//     one, and the per-wave softmax states are merged through LDS at the end.
//   * Streamed prefill schedule (head dim <= 128): 12 waves (head dim 128) or
//     8 (head dim 64) each own 32 packed query rows; 64-key K/V tiles stream through a ring of four LDS buffers
//     filled by direct global->LDS loads two tiles ahead; each wave issues the
//     score product of its next 32 keys before the softmax and PV product of
//     the current ones.
//   * Row-split schedule (mixed-batch q-blocks, head dim 256 prefill): 4 waves
//     each own 32 rows; 64-key tiles double-buffered with register prefetch.
//   * Causal sub-tiles above a wave's diagonal are skipped, and only
//     diagonal/tail sub-tiles are masked.
//   * Keys past seq_lens[b] are never loaded (loads clamp to the last live
//     key), page-table columns past the live page count are never read, and
//     masked scores are selected to -inf, so poisoned cache contents cannot
//     leak into outputs.
#include <atomic>

#include "pa_internal.h"

// Scratch of pa_run_decode_static (split partials, balanced-decode records
// and their schedule words): a file-scope device array, one copy per device.
// In host code this name is only a stand-in for the symbol; kernels receive
// the device address that static_scratch looks up.
static __device__ __align__(256) unsigned char scratch[pa::kStaticScratchBytes];

namespace pa {

// Device address of `scratch` on the current device, resolved with
// hipGetSymbolAddress the first time each device asks and kept afterwards
// (every device holds its own copy at its own address).
hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kDecWaves = 4;              // waves per workgroup, decode and mixed launches
// waves per workgroup of the streamed prefill: three per SIMD at head dim 128
// (168 VGPRs; measured 6-9 % faster than two per SIMD, the third wave hiding
// LDS and MFMA dependency latency), two at head dim 64 (whose fp8 tile has
// fewer direct loads than twelve waves)
// (with fp8 queries, whose E4M3 PV product keeps more state per wave, two
// per SIMD at head dim 128 as well)
constexpr int stream_waves(int D, bool qf8) { return D == 128 && !qf8 ? 12 : 8; }

// Workgroup shape of a launch.  Decode and mixed workgroups have 4 waves so
// that two of them share a compute unit and one's prologue/epilogue overlaps
// the other's streaming.  Prefill at head dim <= 128 runs the streamed
// schedule: 12 or 8 waves, one workgroup per compute unit, all of LDS a ring
// of K/V tiles.  Head dim 256 keeps a 128-row fp32 accumulator per wave, so
// its workgroups run one wave per SIMD with the accumulator in AGPRs.
template <int MODE, int D, bool QF8 = false>
struct Block {
  static constexpr bool stream = MODE == kPrefill && D <= 128;
  static constexpr int waves = stream ? stream_waves(D, QF8) : kDecWaves;
  static constexpr int threads = waves * kWave;
  // prefill schedule: 32-row MFMA column tiles per wave (a second tile would
  // share every K/V operand read, but its accumulator costs the occupancy that
  // hides LDS and exp latency -- measured slower)
  static constexpr int nct = 1;
  static constexpr int waves_per_eu = D == 256 ? 1 : (stream ? waves / 4 : 2);
};

// Decode of an fp8 cache at head dim 256 runs the ring schedule (ring_item):
// each of the four waves streams its own 32-key steps through a private LDS
// ring filled by direct global->LDS loads.
template <int D, bool FP8, int MODE>
struct RingDec { static constexpr bool value = MODE == kDecode && D == 256 && FP8; };

// The ring decode runs eight waves, two per SIMD (its query rows sit in LDS,
// so that the 128-register accumulator fits the 256 registers of two waves);
// every other instance has the shape of Block.
constexpr int kRingWaves = 8;
template <int D, bool FP8, int MODE, bool QF8 = false>
struct Shape {
  static constexpr bool ring = RingDec<D, FP8, MODE>::value;
  static constexpr int waves = ring ? kRingWaves : Block<MODE, D, QF8>::waves;
  static constexpr int threads = waves * kWave;
  static constexpr int waves_per_eu = ring ? kRingWaves / 4 : Block<MODE, D, QF8>::waves_per_eu;
};
constexpr int kSub = 32;                  // keys per score tile (MFMA M of S^T)
constexpr int kCols = 32;                 // packed query rows per wave (MFMA N)
constexpr int kTile = 64;                 // keys per shared LDS tile (prefill schedule)
constexpr int kLdsMax = 160 * 1024;
constexpr int kPcacheEntries = 1024;      // page ids cached in LDS per chunk of keys
constexpr int kXcds = 8;                  // accelerator complex dies of an MI355X
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

template <int A, int B>
struct CMax { static constexpr int value = A > B ? A : B; };

// Byte geometry of one (head_dim, kv dtype) instance.
template <int D, bool FP8>
struct Geo {
  static constexpr int esz = FP8 ? 1 : 2;              // bytes per K/V element
  static constexpr int row_bytes = D * esz;            // one token's row of one KV head
  static constexpr int chunks = row_bytes / 16;        // 16-byte chunks per row
  static constexpr int elems_per_chunk = 16 / esz;
  static constexpr int k_pitch = row_bytes + 16;       // LDS bytes per staged K row
  static constexpr int q_pitch = D * 2 + 16;           // LDS bytes per staged Q row
  // V rows are staged row-major like K and read transposed by the LDS unit
  // (ds_read_b64_tr_b16 / _tr_b8); the extra pad staggers the rows one
  // transposed read touches across banks.
  static constexpr int v_pitch = row_bytes + 32;
  // decode schedule: each wave step stages dec_step keys (K rows, then V rows,
  // in one region): one 32-key tile per step at every geometry (two tiles at
  // fp8 head dim 256 held 32 KB per wave in registers and spilled in the
  // mixed kernels; pure decode of that geometry runs the ring schedule).
  static constexpr int dec_tiles = 1;
  static constexpr int dec_step = kSub * dec_tiles;
  static constexpr int dec_keys_per_lane = (dec_step * chunks) / kWave;   // >= 1
  static constexpr int stage_bytes = CMax<dec_step * k_pitch, dec_step * v_pitch>::value;
  static constexpr int q_bytes = kCols * q_pitch;
  // waves of a decode-schedule item that stage K/V (for an NWB-wave workgroup)
  template <int NWB>
  struct DecWaves { static constexpr int value = (NWB * stage_bytes + q_bytes <= kLdsMax - 8192) ? NWB : NWB / 2; };
  static constexpr bool dec_prefetch = chunks <= 16;   // keep staging registers <= 64 VGPRs
  // prefill schedules: 64-key tile, K rows then V rows at their pitches
  static constexpr int tile_k_bytes = kTile * k_pitch;
  static constexpr int tile_bytes = tile_k_bytes + kTile * v_pitch;
  // streamed prefill: a ring of tile buffers filled by direct global->LDS
  // loads of 1 KB (64 lanes x 16 bytes) each; the pitches are whole 16-byte
  // slots, so a tile is exactly k_slots + v_slots such loads
  static constexpr int k_slots = k_pitch / 16;
  static constexpr int v_slots = v_pitch / 16;
  static constexpr int ring_loads = k_slots + v_slots;
  static constexpr int ring_avail = kLdsMax - 64 - kPcacheEntries * 4;
  static constexpr int ring_bufs = ring_avail / tile_bytes >= 4 ? 4 : ring_avail / tile_bytes;
  // per-wave softmax state exchanged at the end of the decode schedule
  static constexpr int red_floats = D / 2 + 4;         // acc registers + (l, m) record, per lane
  static constexpr int red_bytes = red_floats * kWave * 4;
};

// Byte geometry of the ring decode.  A half-step is the K rows (or the V rows)
// of 32 keys, unpadded; bank conflicts are avoided by storing 16-byte chunk c
// of row r at chunk position c ^ (r mod 16).  Each wave owns two half-step
// buffers (K and V of one step), filled by direct global->LDS loads of 1 KB;
// the block's 32 bf16 query rows follow the rings (padded rows, so that the
// eight lanes of a 16-byte read hit distinct banks).
template <int D, bool FP8>
struct RingGeo {
  static constexpr int esz = FP8 ? 1 : 2;
  static constexpr int row_bytes = D * esz;
  static constexpr int chunks = row_bytes / 16;
  static constexpr int half_bytes = kSub * row_bytes;       // K (or V) rows of one step
  static constexpr int half_loads = half_bytes / 1024;      // direct loads per half-step
  static constexpr int wave_bytes = 2 * half_bytes;         // K, V
  static constexpr int ring_bytes = kRingWaves * wave_bytes;
  static constexpr int q_pitch = D * 2 + 16;
  static constexpr int q_off = ring_bytes;
  static constexpr int bytes = q_off + kCols * q_pitch;
  static_assert(chunks == 16, "one row is exactly the 16 swizzled chunks");
  static_assert(bytes + 64 + kPcacheEntries * 4 <= kLdsMax, "LDS budget of the ring");
};

template <int D, bool FP8, bool RING>
struct RingBytes { static constexpr int bytes = 0; };
template <int D, bool FP8>
struct RingBytes<D, FP8, true> { static constexpr int bytes = RingGeo<D, FP8>::bytes; };

template <int D, bool FP8, int MODE>
struct Lds {
  using G = Geo<D, FP8>;
  static constexpr int dec = RingDec<D, FP8, MODE>::value
                                 ? RingBytes<D, FP8, RingDec<D, FP8, MODE>::value>::bytes
                                 : G::q_bytes + G::template DecWaves<Block<MODE, D>::waves>::value * G::stage_bytes;
  // streamed prefill of an fp8 cache: the ring, then room for the E4M3 query
  // rows of every wave when the queries are fp8 (q8_pitch bytes per row)
  static constexpr int q8_pitch = D + 16;
  static constexpr int q8_off = (Block<MODE, D>::stream ? G::ring_bufs : 2) * G::tile_bytes;
  static constexpr int pre = q8_off + (Block<MODE, D>::stream && FP8 ? Block<MODE, D, true>::waves * kCols * q8_pitch : 0);
  static constexpr int base = MODE == kDecode ? dec : (MODE == kPrefill ? pre : CMax<dec, pre>::value);
  static constexpr int meta = 64;                      // work-item metadata words
  static constexpr int pcache_entries = kPcacheEntries;
  static constexpr int pcache_off = base + meta;
  static constexpr int bytes = pcache_off + pcache_entries * 4;
  static_assert(bytes <= kLdsMax, "LDS budget exceeded");
};

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x64 product of OCP E4M3 operands (format 0 for both, no block
// scales): lane l holds row l % 32 and k = 32 (l / 32) .. +31 of its operand
// (32 bytes); the accumulator layout is that of the bf16 product above.
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// s_waitcnt vmcnt(0): every vector-memory load of this wave has returned
// (expcnt and lgkmcnt fields left at their "no wait" maxima).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 8 fp8 e4m3 bytes (two dwords) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

// Value of lane l^32.  v_permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second; with both operands x, lanes < 32
// find their partner in the second result and lanes >= 32 in the first.
// threadIdx.x through an opaque move.  The schedules of one work item call
// this instead of reading threadIdx.x: in the task-queue kernel, which runs
// many items per workgroup, the per-lane addresses derived from it are then
// recomputed for each item instead of being hoisted to the kernel prologue
// and kept live (spilled) across the whole item loop.
__device__ __forceinline__ int item_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

__device__ __forceinline__ float xor32(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// Value of lane l^16 (v_permlane16_swap exchanges the odd 16-lane rows of its
// first operand with the even rows of its second; with both operands x, lanes
// in even rows find their partner in the second result, the others in the
// first).
__device__ __forceinline__ float xor16(float x) {
  const int xi = __builtin_bit_cast(int, x);
  const auto r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

// ---------------------------------------------------------------------------
// K / V staging: a "unit" is NK consecutive keys x one 16-byte chunk of their rows
// ---------------------------------------------------------------------------

// Where a sequence's K/V rows live.  Page ids of the keys being processed are
// cached in LDS (pcache[i] = page_table[row][first_page + i]) so that every
// K/V load can be issued without waiting on a page-table load.
struct PageWalk {
  const int32_t* pt_row;   // page-table row of the sequence
  const int32_t* pcache;   // LDS copy of page ids from first_page on
  int32_t first_page;
  int64_t page_bytes;      // bytes between physical pages
  int64_t head_off;        // g * row_bytes
  int32_t row_stride_b;    // Hkv * row_bytes (bytes between slots of a page)
  int32_t shift;           // log2(page)
  int32_t klimit;          // live keys (clamped to C * page)
  int32_t kend;            // loads clamp to keys below this: min(chunk end, klimit)
};

// Copy the page ids of keys [k_begin, k_end) (clamped to live keys) into the
// LDS cache.  Only columns below ceil(klimit / page) are ever read.
__device__ __forceinline__ void fill_pcache(PageWalk& w, int32_t* pcache, int k_begin, int k_end) {
  const int last_key = min(k_end, w.klimit) - 1;
  w.kend = last_key + 1;
  w.first_page = k_begin >> w.shift;
  w.pcache = pcache;
  const int n = last_key >= k_begin ? (last_key >> w.shift) - w.first_page + 1 : 0;
  for (int i = item_tid(); i < n; i += blockDim.x) pcache[i] = w.pt_row[w.first_page + i];
}

// NK consecutive keys from key0 (a multiple of NK), one 16-byte chunk each,
// from the K pool and the V pool (same offsets).  NK divides 16 and every page
// holds a multiple of 16 keys, so an aligned group never crosses a page: one
// page-id lookup and one 64-bit page base serve the whole group.  Keys at or
// past the end of the cached window (never past the live length) are clamped
// to its last key: they load finite data that the score mask gives
// probability 0.
template <int NK>
__device__ __forceinline__ void load_kv_unit(const uint8_t* __restrict__ kpool,
                                             const uint8_t* __restrict__ vpool, const PageWalk& w,
                                             int key0, int chunk, u32x4 (&kr)[NK], u32x4 (&vr)[NK]) {
  static_assert(NK <= 16 && 16 % NK == 0, "a key group must not cross a page");
  const int kc0 = min(key0, w.kend - 1);
  const int64_t page_off = (int64_t)w.pcache[(kc0 >> w.shift) - w.first_page] * w.page_bytes +
                           w.head_off + chunk * 16;
  const uint8_t* kb = kpool + page_off;
  const uint8_t* vb = vpool + page_off;
  const int slot_mask = (1 << w.shift) - 1;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int slot = min(key0 + i, w.kend - 1) & slot_mask;
    const uint32_t off = (uint32_t)slot * (uint32_t)w.row_stride_b;
    kr[i] = *reinterpret_cast<const u32x4*>(kb + off);
    vr[i] = *reinterpret_cast<const u32x4*>(vb + off);
  }
}

// Same for one pool only.
template <int NK>
__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ pool, const PageWalk& w,
                                          int key0, int chunk, u32x4 (&r)[NK]) {
  static_assert(NK <= 16 && 16 % NK == 0, "a key group must not cross a page");
  const int kc0 = min(key0, w.kend - 1);
  const uint8_t* base = pool + (int64_t)w.pcache[(kc0 >> w.shift) - w.first_page] * w.page_bytes +
                        w.head_off + chunk * 16;
  const int slot_mask = (1 << w.shift) - 1;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int slot = min(key0 + i, w.kend - 1) & slot_mask;
    r[i] = *reinterpret_cast<const u32x4*>(base + (uint32_t)slot * (uint32_t)w.row_stride_b);
  }
}

// K or V rows: key (krow0 + i) at the row pitch, chunk offset.
template <int NK, int PITCH>
__device__ __forceinline__ void store_k(uint8_t* kl, int krow0, int chunk, const u32x4 (&r)[NK]) {
#pragma unroll
  for (int i = 0; i < NK; ++i)
    *reinterpret_cast<u32x4*>(kl + (krow0 + i) * PITCH + chunk * 16) = r[i];
}

// ---------------------------------------------------------------------------
// one 32-key score tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T
// ---------------------------------------------------------------------------

template <int D>
struct SoftmaxState {
  f32x16 o[D / 32];   // O^T tiles: reg i of tile t <-> d = 32t + (i/4)*8 + (lane/32)*4 + i%4
  float m;            // running max of scaled scores (log2 units), per query row
  float l;            // running sum of exp2(score - m), this lane's 16 keys of each tile
};

template <int D>
__device__ __forceinline__ void state_init(SoftmaxState<D>& st) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[t][i] = 0.f;
  st.m = neg_inf();
  st.l = 0.f;
}

// Key order inside a 32-key score tile.  MFMA row m of S^T = K Q^T holds key
// kperm(m) (bits 2 and 3 of m swapped).  With that order, accumulator element
// i of lane l holds key (i & 7) + 8*(l/32) + 16*(i/8): each lane's probabilities
// for one PV k-step are 8 CONSECUTIVE keys, which is what the transposing LDS
// reads below deliver for the V operand.
__device__ __forceinline__ int kperm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
__device__ __forceinline__ int acc_key(int i, int lane) { return (i & 7) + 8 * (lane >> 5) + 16 * (i >> 3); }

// K operand for k-step j: K[key = kb + kperm(lane%32)][d = 16j + (lane/32)*8 .. +8]
template <int D, bool FP8, int KPITCH>
__device__ __forceinline__ bf16x8 k_operand(const uint8_t* kl, int kb, int j, int lane) {
  const uint8_t* src = kl + (kb + kperm(lane & 31)) * KPITCH + (16 * j + (lane >> 5) * 8) * (FP8 ? 1 : 2);
  if constexpr (FP8) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(src);
    return fp8x8_to_bf16(w[0], w[1]);
  } else {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(src));
  }
}

// fp8 K operand for the 64-wide k-step j of the E4M3 score product: the 32
// bytes K[key = kb + kperm(lane%32)][64 j + 32 (lane/32) .. +32], left in fp8.
template <int KPITCH>
__device__ __forceinline__ i32x8 k_operand_f8(const uint8_t* kl, int kb, int j, int lane) {
  const uint8_t* src = kl + (kb + kperm(lane & 31)) * KPITCH + 64 * j + 32 * (lane >> 5);
  const u32x4 a = *reinterpret_cast<const u32x4*>(src);
  const u32x4 b = *reinterpret_cast<const u32x4*>(src + 16);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// E4M3 query operand of the 64-wide k-step j from this lane's query row in
// LDS (qrow already offset by 32 bytes for lanes >= 32): 32 bytes.
__device__ __forceinline__ i32x8 q8_operand(const uint8_t* qrow, int j) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(qrow + 64 * j);
  const u32x4 b = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// V^T operand for d-tile t and k-step s of the tile whose keys start at row kb
// of a row-major V stage: lane l needs V[kb + 16s + 8*(l/32) + kk][32t + l%32]
// for kk = 0..7.  Within each 16-lane group the transposing read hands output
// lane L element L%4 (tr_b16) / byte L%8 (tr_b8) of the 8-byte segments read by
// a fixed set of source lanes; each source lane below reads the segment that
// makes output lane L receive consecutive keys of column 32t + (l%32).
template <bool FP8, int VPITCH>
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* vl, int kb, int t, int s, int lane) {
  const int L = lane & 15;
  const int d0 = 32 * t + 16 * ((lane >> 4) & 1);
  const int k0 = kb + 16 * s + 8 * (lane >> 5);
  if constexpr (FP8) {
    // source lane L: key k0 + L/2, columns d0 + 8*(L%2) .. +7
    const uint8_t* src = vl + (k0 + (L >> 1)) * VPITCH + d0 + 8 * (L & 1);
    const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(src));
    return fp8x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
  } else {
    // source lane L: key k0 + L/4 (+4 for the second read), columns d0 + 4*(L%4) .. +3
    const uint8_t* src = vl + (k0 + (L >> 2)) * VPITCH + 2 * (d0 + 4 * (L & 3));
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + 4 * VPITCH));
    return as_bf16x8(u32x4{__builtin_bit_cast(u32x2, a)[0], __builtin_bit_cast(u32x2, a)[1],
                           __builtin_bit_cast(u32x2, b)[0], __builtin_bit_cast(u32x2, b)[1]});
  }
}

// Scores of NS consecutive 32-key tiles (key rows kb, kb+32, ...): raw q.k in
// fp32.  The NS accumulation chains are interleaved so that consecutive MFMAs
// never wait on each other's results.
template <int D, bool FP8, int KPITCH, bool QLDS, int NS>
__device__ __forceinline__ void score_tiles(f32x16 (&s)[NS], const uint8_t* kl, int kb,
                                            const bf16x8* qreg, const uint8_t* ql, int qpitch,
                                            int lane) {
#pragma unroll
  for (int n = 0; n < NS; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[n][i] = 0.f;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    bf16x8 bq;
    if constexpr (QLDS)
      bq = as_bf16x8(*reinterpret_cast<const u32x4*>(ql + (lane & 31) * qpitch + (16 * j + (lane >> 5) * 8) * 2));
    else
      bq = qreg[j];
#pragma unroll
    for (int n = 0; n < NS; ++n) s[n] = mfma32(k_operand<D, FP8, KPITCH>(kl, kb + kSub * n, j, lane), bq, s[n]);
  }
}

// Mask the scores of one tile: key index of s[i] in this lane, keys >= klim
// (this lane's query row) become -inf.  Applied only on tiles that cross a
// row's causal limit or the live length.
__device__ __forceinline__ void mask_tile(f32x16& s, int key0, int klim, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = key0 + acc_key(i, lane) < klim ? s[i] : neg_inf();
}

// Logit soft-capping on raw MFMA scores.  The scaled score is r * c / log2(e)
// (c = softmax_scale * log2(e), times k_descale for fp8); capping it to
// cap * tanh(scaled / cap) is the same as replacing r by tanh(b r) / b with
// b = c / (cap * log2(e)), which leaves the rest of the exp2-domain softmax
// unchanged.  tanh(x) = 1 - 2 / (exp(2x) + 1): saturates to +-1 through
// exp2 = inf or 0.
struct SoftCap {
  float k2;      // 2 b log2(e) = 2 c / cap; 0 means no capping
  float inv_b;   // cap log2(e) / c
  __device__ SoftCap(float cap, float c)
      : k2(cap > 0.f ? 2.f * c / cap : 0.f), inv_b(cap > 0.f ? cap * 1.44269504088896341f / c : 0.f) {}
  __device__ bool on() const { return k2 != 0.f; }
};

__device__ __forceinline__ void cap_tile(f32x16& s, const SoftCap& sc) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = __builtin_amdgcn_exp2f(s[i] * sc.k2);
    s[i] = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f) * sc.inv_b;
  }
}

// Growth of the row max (log2 units) tolerated before the accumulator is
// rescaled: probabilities are exp2(score - m) with m possibly stale by up to
// this much, i.e. at most 2^8, harmless in fp32 and bf16.  The result is exact
// for any reference m; the slack only skips most of the per-tile rescales.
constexpr float kRescaleSlack = 8.0f;

// Online softmax update for NS consecutive 32-key tiles of raw scores of one
// 32-row column tile (masked entries already -inf): updates (m, l), rescales the
// accumulator when the row max grew by more than the slack, and returns the
// probabilities as bf16 PV B-operands.  c = softmax_scale * log2(e) (*
// k_descale), c > 0.
template <int D, int NS, bool INT_M = false>
__device__ __forceinline__ void max_update(SoftmaxState<D>& st, const f32x16 (&s)[NS], float c) {
  float mx = neg_inf();
#pragma unroll
  for (int n = 0; n < NS; ++n)
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[n][i]), s[n][i + 1]);
  mx = fmaxf(mx, xor32(mx));
  const float mxs = mx * c;
  if (__builtin_amdgcn_ballot_w64(mxs > st.m + kRescaleSlack)) {
    // INT_M: the reference is rounded up to an integer, so that every rescale
    // factor is a power of two
    const float m_new = INT_M ? __builtin_ceilf(fmaxf(st.m, mxs)) : fmaxf(st.m, mxs);
    const float alpha = __builtin_amdgcn_exp2f(st.m - (m_new == neg_inf() ? 0.f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[t][i] *= alpha;
    st.m = m_new;
  }
}

// Probabilities of NS tiles under the current running max, added to the row
// sum and packed as bf16 PV B-operands.
template <int D, int NS>
__device__ __forceinline__ void probs(SoftmaxState<D>& st, const f32x16 (&s)[NS], float c,
                                      bf16x8 (&pb)[NS][2]) {
  // nothing visible yet: reference 0 so that exp2(-inf) = 0 instead of NaN
  const float nref = st.m == neg_inf() ? 0.f : -st.m;
  float psum = 0.f;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][i], c, nref));
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = p[i] + p[i + 8];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] += q[i + 4];
    psum += (q[0] + q[2]) + (q[1] + q[3]);
    pb[n][0] = pack_bf16x8(p);
    pb[n][1] = pack_bf16x8(p + 8);
  }
  st.l += psum;
}

// max_update for one tile of the streamed schedule, with the slack test done
// per lane first: each lane compares the max of its own 16 raw scores with
// thr = (m + slack) / c; only when some lane of the wave exceeds it is the row
// max taken over both lanes of the row and the accumulator rescaled.  The
// common case is then eight v_max3 and one compare.  thr and nref (the
// exponent offset of the probabilities, -m or 0 while m is -inf) follow st.m.
template <int D, bool INT_M>
__device__ __forceinline__ void max_update_lane(SoftmaxState<D>& st, const f32x16& s, float c, float& thr,
                                                float& nref) {
  float mx = neg_inf();
#pragma unroll
  for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
  if (__builtin_amdgcn_ballot_w64(mx > thr)) {
    mx = fmaxf(mx, xor32(mx));
    const float mxs = mx * c;
    const float m_new = INT_M ? __builtin_ceilf(fmaxf(st.m, mxs)) : fmaxf(st.m, mxs);
    const float alpha = __builtin_amdgcn_exp2f(st.m - (m_new == neg_inf() ? 0.f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[t][i] *= alpha;
    st.m = m_new;
    thr = (m_new + kRescaleSlack) / c;
    nref = m_new == neg_inf() ? 0.f : -m_new;
  }
}

template <int D, int NS>
__device__ __forceinline__ void softmax_p(SoftmaxState<D>& st, const f32x16 (&s)[NS], float c,
                                          bf16x8 (&pb)[NS][2]) {
  max_update<D, NS>(st, s, c);
  probs<D, NS>(st, s, c, pb);
}

// O^T += V^T P^T for NS tiles whose V rows start at row kb of the stage, for
// NCT column tiles at once: each V operand read from LDS feeds NCT MFMAs.
template <int D, bool FP8, int VPITCH, int NS, int NCT>
__device__ __forceinline__ void pv_accum(SoftmaxState<D> (&st)[NCT], const bf16x8 (&pb)[NCT][NS][2],
                                         const uint8_t* vl, int kb, int lane) {
#pragma unroll
  for (int n = 0; n < NS; ++n)
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 a = v_operand<FP8, VPITCH>(vl, kb + kSub * n, t, h, lane);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) st[ct].o[t] = mfma32(a, pb[ct][n][h], st[ct].o[t]);
      }
}

// ---------------------------------------------------------------------------
// output
// ---------------------------------------------------------------------------

struct RowMap {
  int t0;       // absolute token index of the block's first query token
  int ntok;     // query tokens in the block
  int pos0;     // absolute position of the first token in its sequence
  int g;        // KV head
  int G;        // query heads per KV head
};

// Write one wave's 32 query rows (columns) starting at packed row r0.  l is
// already the full row sum (both lane halves).  The wave's accumulator covers
// head-dim columns [col0, col0 + DS) of rows of width D; the LSE is written
// only by the wave that owns it (lse_owner).
template <int D, int DS = D>
__device__ void write_rows(const AttnParams& p, const SoftmaxState<DS>& st, float l_tot, int r0,
                           const RowMap& rm, int slot, float vdesc, int lane, int col0 = 0,
                           bool lse_owner = true) {
  lane = item_tid() & (kWave - 1);       // re-derived here: nothing per-lane stays live for the epilogue
  const int r = r0 + (lane & 31);
  const int tok = r / rm.G;
  if (tok >= rm.ntok) return;
  const int t = rm.t0 + tok;
  if (t >= p.max_total_q) return;
  const int h = rm.g * rm.G + (r - tok * rm.G);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : vdesc / l_tot;
  const float lse2 = empty ? neg_inf() : st.m + __builtin_amdgcn_logf(l_tot);  // v_log_f32 is log2
  if (slot >= 0) {
    // partial (O / l, log2 LSE): split-KV slots hold [split][token][head]
    // records; balanced decode slots hold the G rows of one item
    const int64_t row = p.balanced ? (int64_t)slot * rm.G + r
                                   : ((int64_t)slot * p.max_total_q + t) * p.num_q_heads + h;
    if (lse_owner && (lane >> 5) == 0) p.part_lse[row] = lse2;
    if (empty) return;
    float* dst = p.part_o + row * D + col0;
#pragma unroll
    for (int tt = 0; tt < DS / 32; ++tt)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = 32 * tt + 8 * ig + (lane >> 5) * 4;
        f32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = st.o[tt][4 * ig + k] * inv;
        *reinterpret_cast<f32x4*>(dst + d0) = v;
      }
  } else {
    uint16_t* dst = p.out + (int64_t)t * p.o_stride_t + (int64_t)h * D + col0;
#pragma unroll
    for (int tt = 0; tt < DS / 32; ++tt)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = 32 * tt + 8 * ig + (lane >> 5) * 4;
        const u32x2 v{pack_bf16x2(st.o[tt][4 * ig] * inv, st.o[tt][4 * ig + 1] * inv),
                      pack_bf16x2(st.o[tt][4 * ig + 2] * inv, st.o[tt][4 * ig + 3] * inv)};
        *reinterpret_cast<u32x2*>(dst + d0) = v;
      }
    if (lse_owner && p.lse && (lane >> 5) == 0) p.lse[(int64_t)t * p.num_q_heads + h] = lse2 * kLn2;
  }
}

// ---------------------------------------------------------------------------
// decode schedule: waves split the key range of one block of <= 32 query rows
// ---------------------------------------------------------------------------

template <int D, bool FP8, int MODE>
__device__ void keysplit_item(const AttnParams& p, uint8_t* smem, int32_t* pcache, const RowMap& rm,
                              const PageWalk& pw, int L, int klo, int khi, int slot, float c,
                              float vdesc) {
  using Gm = Geo<D, FP8>;
  const SoftCap sc(p.softcap, c);
  constexpr int NWB = Block<MODE, D>::waves;             // waves in the workgroup
  constexpr int NW = Gm::template DecWaves<NWB>::value;   // waves that stage K/V
  constexpr int NK = Gm::dec_keys_per_lane;
  const int lane = item_tid() & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(item_tid() >> 6);
  const int nrows = rm.ntok * rm.G;

  // key window [klo, khi), clipped by the causal limit of the last token
  if (p.causal) khi = min(khi, rm.pos0 + rm.ntok);

  SoftmaxState<D> st[1];
  state_init(st[0]);
  if (khi <= klo) {
    // empty window: the (partial) rows are empty, nothing to stage or stream
    if (wave == 0) write_rows<D>(p, st[0], 0.f, 0, rm, slot, vdesc, lane);
    return;
  }

  // The block's query rows (zero padded to 32) and the page ids of the first
  // chunk of keys are fetched together and published with one barrier.
  uint8_t* ql = smem;
  PageWalk w = pw;
  const int chunk_keys = kPcacheEntries << w.shift;
  {
    constexpr int cpr = D * 2 / 16;
    constexpr int NTH = Block<MODE, D>::threads;
    constexpr int QPT = (kCols * cpr + NTH - 1) / NTH;   // 16-byte Q chunks per thread
    u32x4 qv[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int u = item_tid() + k * NTH;
      const int r = u / cpr, ch = u % cpr;
      qv[k] = u32x4{0u, 0u, 0u, 0u};
      if (u < kCols * cpr && r < nrows) {
        const int tok = r / rm.G;
        const int h = rm.g * rm.G + (r - tok * rm.G);
        qv[k] = *reinterpret_cast<const u32x4*>(p.q + (int64_t)(rm.t0 + tok) * p.q_stride_t +
                                                (int64_t)h * D + ch * 8);
      }
    }
    fill_pcache(w, pcache, klo, min(khi, klo + chunk_keys));
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int u = item_tid() + k * NTH;
      if (u < kCols * cpr) *reinterpret_cast<u32x4*>(ql + (u / cpr) * Gm::q_pitch + (u % cpr) * 16) = qv[k];
    }
  }
  __syncthreads();
  // this lane's query row sees keys < klim
  const int my_tok = min((lane & 31) / rm.G, max(rm.ntok - 1, 0));
  const int klim = p.causal ? min(khi, rm.pos0 + my_tok + 1) : khi;
  // keys below kfull are visible to every row of the block
  const int kfull = p.causal ? min(khi, rm.pos0 + 1) : khi;

  for (int cb = klo; cb < khi; cb += chunk_keys) {
    const int ce = min(khi, cb + chunk_keys);
    if (cb != klo) {
      __syncthreads();
      fill_pcache(w, pcache, cb, ce);
      __syncthreads();
    }
    constexpr int STEP = Gm::dec_step;
    constexpr int NT = Gm::dec_tiles;
    const int nsub = (ce - cb + STEP - 1) / STEP;
    if (wave < NW) {
      uint8_t* stage = smem + Gm::q_bytes + wave * Gm::stage_bytes;
      const int chunk = lane % Gm::chunks;
      const int kg = lane / Gm::chunks;      // key group of this lane
      u32x4 kr[NK], vr[NK];
      int n = wave;
      if (Gm::dec_prefetch && n < nsub) {
        load_unit<NK>(p.k_pool, w, cb + n * STEP + kg * NK, chunk, kr);
        load_unit<NK>(p.v_pool, w, cb + n * STEP + kg * NK, chunk, vr);
      }
      for (; n < nsub; n += NW) {
        const int key0 = cb + n * STEP;
        // Prefetch target: the wave's next step, or (last iteration) keys
        // already in cache.  Unconditional, so that the compiler's load
        // counters stay exact and no wait covers the prefetch itself.
        const int key_next = cb + min(n + NW, nsub - 1) * STEP;
        if (!Gm::dec_prefetch) load_unit<NK>(p.k_pool, w, key0 + kg * NK, chunk, kr);
        store_k<NK, Gm::k_pitch>(stage, kg * NK, chunk, kr);
        if (Gm::dec_prefetch) load_unit<NK>(p.k_pool, w, key_next + kg * NK, chunk, kr);
        __builtin_amdgcn_wave_barrier();
        f32x16 s[NT];
        score_tiles<D, FP8, Gm::k_pitch, true, NT>(s, stage, 0, nullptr, ql, Gm::q_pitch, lane);
        if (sc.on()) {
#pragma unroll
          for (int t = 0; t < NT; ++t) cap_tile(s[t], sc);
        }
        if (key0 + STEP > kfull) {
#pragma unroll
          for (int t = 0; t < NT; ++t) mask_tile(s[t], key0 + kSub * t, klim, lane);
        }
        __builtin_amdgcn_wave_barrier();
        if (!Gm::dec_prefetch) load_unit<NK>(p.v_pool, w, key0 + kg * NK, chunk, vr);
        store_k<NK, Gm::v_pitch>(stage, kg * NK, chunk, vr);
        if (Gm::dec_prefetch) load_unit<NK>(p.v_pool, w, key_next + kg * NK, chunk, vr);
        __builtin_amdgcn_wave_barrier();
        bf16x8 pb[1][NT][2];
        softmax_p<D, NT>(st[0], s, c, pb[0]);
        pv_accum<D, FP8, Gm::v_pitch, NT, 1>(st, pb, stage, 0, lane);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }

  // merge the per-wave states pairwise through LDS: (m, l, O) of a writer wave
  // folded into a reader wave with the usual max-rescale.
  __syncthreads();
  constexpr int lds_avail = Lds<D, FP8, MODE>::base;
  constexpr int nbuf_raw = lds_avail / Gm::red_bytes;
  constexpr int nbuf = nbuf_raw < 1 ? 1 : nbuf_raw;
  static_assert(nbuf_raw >= 1, "no LDS for the wave merge");
  float* red = reinterpret_cast<float*>(smem);
  int active = NW;
  while (active > 1) {
    const int half = active / 2;
    const int cnt = half < nbuf ? half : nbuf;
    const int w_lo = active - cnt;         // writers [w_lo, active)
    const int r_lo = active - 2 * cnt;     // readers [r_lo, w_lo)
    // a wave's state as 16-byte records [record][lane]: O in D/8 records, then (l, m)
    if (wave >= w_lo && wave < active) {
      f32x4* buf = reinterpret_cast<f32x4*>(red + (wave - w_lo) * Gm::red_floats * kWave);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          buf[(4 * t + q) * kWave + lane] = f32x4{st[0].o[t][4 * q], st[0].o[t][4 * q + 1],
                                                  st[0].o[t][4 * q + 2], st[0].o[t][4 * q + 3]};
      buf[(D / 8) * kWave + lane] = f32x4{st[0].l, st[0].m, 0.f, 0.f};
    }
    __syncthreads();
    if (wave >= r_lo && wave < w_lo) {
      const f32x4* buf = reinterpret_cast<const f32x4*>(red + (wave - r_lo) * Gm::red_floats * kWave);
      const f32x4 lm = buf[(D / 8) * kWave + lane];
      const float l2 = lm[0];
      const float m2 = lm[1];
      const float mm = fmaxf(st[0].m, m2);
      const float ref = mm == neg_inf() ? 0.f : mm;
      const float a1 = __builtin_amdgcn_exp2f(st[0].m - ref);
      const float a2 = __builtin_amdgcn_exp2f(m2 - ref);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = buf[(4 * t + q) * kWave + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) st[0].o[t][4 * q + e] = st[0].o[t][4 * q + e] * a1 + v[e] * a2;
        }
      st[0].l = st[0].l * a1 + l2 * a2;
      st[0].m = mm;
    }
    __syncthreads();
    active = w_lo;
  }
  if (wave == 0) {
    const float l_tot = st[0].l + xor32(st[0].l);
    write_rows<D>(p, st[0], l_tot, 0, rm, slot, vdesc, lane);
  }
}

// ---------------------------------------------------------------------------
// prefill schedule: each wave owns 32 packed query rows; K/V tiles shared in LDS
// ---------------------------------------------------------------------------

template <int D, bool FP8, int MODE>
__device__ void rowsplit_item(const AttnParams& p, uint8_t* smem, int32_t* pcache, const RowMap& rm,
                              const PageWalk& pw, int L, int split, float c, float vdesc) {
  using Gm = Geo<D, FP8>;
  const SoftCap sc(p.softcap, c);
  constexpr int NTH = Block<MODE, D>::threads;
  // a loader unit: NK consecutive keys x one 16-byte chunk, one unit per thread
  constexpr int NK = (kTile * Gm::chunks) / NTH > 0 ? (kTile * Gm::chunks) / NTH : 1;
  constexpr int NUNITS = (kTile * Gm::chunks) / NK;
  constexpr int NCT = Block<MODE, D>::nct;               // 32-row column tiles per wave
  constexpr int NS = kTile / kSub;                       // score tiles per LDS tile
  const int lane = item_tid() & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(item_tid() >> 6);
  const int nrows = rm.ntok * rm.G;
  const int r0 = wave * kCols * NCT;                     // this wave's first packed row
  const int last_tok = max(rm.ntok - 1, 0);

  // Q operands of this wave's rows, in registers
  bf16x8 qreg[NCT][D / 16];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int r = r0 + ct * kCols + (lane & 31);
    const bool ok = r < nrows;
    const int tok = ok ? r / rm.G : 0;
    const int h = rm.g * rm.G + (r - tok * rm.G);
    const uint16_t* src = p.q + (int64_t)(rm.t0 + tok) * p.q_stride_t + (int64_t)h * D + (lane >> 5) * 8;
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
      qreg[ct][j] = ok ? as_bf16x8(*reinterpret_cast<const u32x4*>(src + 16 * j))
                       : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }
  // Let the Q loads land here, once.  Vector-memory loads retire in order on
  // one counter; if Q were still counted as outstanding at the first score
  // product, the wait placed there (inside the tile loop) would also cover the
  // K/V prefetch issued just before it, on every tile.
  wait_vmem_all();

  const int klo = split * p.split_keys;
  // the last window takes every remaining key
  int khi = split == p.num_splits - 1 ? L : min(L, klo + p.split_keys);
  if (p.causal) khi = min(khi, rm.pos0 + rm.ntok);

  // visibility: the wave's rows are tokens [tok_a, tok_b]; lane rows per column tile
  const bool wave_active = r0 < nrows;
  const int tok_a = min(r0 / rm.G, last_tok);
  const int tok_b = min((r0 + kCols * NCT - 1) / rm.G, last_tok);
  const int wave_kmax = p.causal ? min(khi, rm.pos0 + tok_b + 1) : khi;   // no key >= this is visible
  const int wave_kfull = p.causal ? min(khi, rm.pos0 + tok_a + 1) : khi;  // keys < this visible to all
  int klim[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int my_tok = min((r0 + ct * kCols + (lane & 31)) / rm.G, last_tok);
    klim[ct] = p.causal ? min(khi, rm.pos0 + my_tok + 1) : khi;
  }

  SoftmaxState<D> st[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) state_init(st[ct]);

  const int unit = item_tid();
  const bool loader = unit < NUNITS;
  const int chunk = unit % Gm::chunks;
  const int kg = unit / Gm::chunks;
  u32x4 kr[NK], vr[NK];
  PageWalk w = pw;
  const int chunk_keys = kPcacheEntries << w.shift;
  // Two LDS tile buffers: tile t is read from buffer t&1 while tile t+1 is
  // stored into the other one and tile t+2 is in flight in registers, so each
  // tile costs one workgroup barrier.
  for (int cb = klo; cb < khi; cb += chunk_keys) {
    const int ce = min(khi, cb + chunk_keys);
    __syncthreads();
    fill_pcache(w, pcache, cb, ce);
    __syncthreads();
    const int ntiles = (ce - cb + kTile - 1) / kTile;
    if (loader) {
      load_kv_unit<NK>(p.k_pool, p.v_pool, w, cb + kg * NK, chunk, kr, vr);
      store_k<NK, Gm::k_pitch>(smem, kg * NK, chunk, kr);
      store_k<NK, Gm::v_pitch>(smem + Gm::tile_k_bytes, kg * NK, chunk, vr);
      const int key1 = cb + min(1, ntiles - 1) * kTile;
      load_kv_unit<NK>(p.k_pool, p.v_pool, w, key1 + kg * NK, chunk, kr, vr);
    }
    __syncthreads();
    for (int tix = 0; tix < ntiles; ++tix) {
      const int key0 = cb + tix * kTile;
      const uint8_t* kl = smem + (tix & 1) * Gm::tile_bytes;
      const uint8_t* vl = kl + Gm::tile_k_bytes;
      if (wave_active && key0 < wave_kmax) {
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const int k0 = key0 + kSub * n;
          // K operands of the tile: all of them first (head dim <= 128), so the
          // score MFMAs do not wait on LDS one by one; at head dim 256 eight
          // ahead of their MFMAs, which keeps the operands out of scratch
          constexpr int KA = D <= 128 ? D / 16 : 8;
          bf16x8 ka[D / 16];
#pragma unroll
          for (int j = 0; j < KA; ++j) ka[j] = k_operand<D, FP8, Gm::k_pitch>(kl, kSub * n, j, lane);
          // two independent accumulation chains (even / odd k-steps) halve the
          // dependent-MFMA latency of the score product
          f32x16 s[NCT][1], s2[NCT];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[ct][0][i] = s2[ct][i] = 0.f;
#pragma unroll
          for (int j = 0; j < D / 16; j += 2) {
            if (KA < D / 16 && j + KA < D / 16) {
              ka[j + KA] = k_operand<D, FP8, Gm::k_pitch>(kl, kSub * n, j + KA, lane);
              ka[j + KA + 1] = k_operand<D, FP8, Gm::k_pitch>(kl, kSub * n, j + KA + 1, lane);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              s[ct][0] = mfma32(ka[j], qreg[ct][j], s[ct][0]);
              s2[ct] = mfma32(ka[j + 1], qreg[ct][j + 1], s2[ct]);
            }
          }
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) s[ct][0] += s2[ct];
          // V operands requested before the softmax, so that their LDS latency
          // hides under the exp work: all of them (head dim <= 128), or the
          // first eight, the rest eight ahead of their MFMAs
          constexpr int VA = D <= 128 ? D / 16 : 8;
          bf16x8 va[D / 32][2];
#pragma unroll
          for (int v = 0; v < VA; ++v) va[v >> 1][v & 1] = v_operand<FP8, Gm::v_pitch>(vl, kSub * n, v >> 1, v & 1, lane);
          if (sc.on()) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) cap_tile(s[ct][0], sc);
          }
          if (k0 + kSub > wave_kfull) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) mask_tile(s[ct][0], k0, klim[ct], lane);
          }
          bf16x8 pb[NCT][1][2];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) softmax_p<D, 1>(st[ct], s[ct], c, pb[ct]);
#pragma unroll
          for (int v = 0; v < D / 16; ++v) {
            if (VA < D / 16 && v + VA < D / 16)
              va[(v + VA) >> 1][(v + VA) & 1] = v_operand<FP8, Gm::v_pitch>(vl, kSub * n, (v + VA) >> 1, (v + VA) & 1, lane);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) st[ct].o[v >> 1] = mfma32(va[v >> 1][v & 1], pb[ct][0][v & 1], st[ct].o[v >> 1]);
          }
        }
      }
      if (loader) {
        // tile tix+1 (already in registers) into the other buffer, then fetch
        // tile tix+2 -- or, near the end, a tile already in cache: the loads
        // are unconditional so the compiler's load counters stay exact
        uint8_t* kn = smem + ((tix + 1) & 1) * Gm::tile_bytes;
        store_k<NK, Gm::k_pitch>(kn, kg * NK, chunk, kr);
        store_k<NK, Gm::v_pitch>(kn + Gm::tile_k_bytes, kg * NK, chunk, vr);
        const int key2 = cb + min(tix + 2, ntiles - 1) * kTile;
        load_kv_unit<NK>(p.k_pool, p.v_pool, w, key2 + kg * NK, chunk, kr, vr);
      }
      __syncthreads();
    }
  }
  if (wave_active) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float l_tot = st[ct].l + xor32(st[ct].l);
      write_rows<D>(p, st[ct], l_tot, r0 + ct * kCols, rm, p.num_splits > 1 ? split : -1, vdesc, lane);
    }
  }
}


// ---------------------------------------------------------------------------
// streamed prefill schedule (head dim <= 128): each wave owns 32 packed
// query rows; 64-key K/V tiles stream through a ring of LDS buffers
// ---------------------------------------------------------------------------

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Direct global->LDS load of 16 bytes per lane: lane l's 16 bytes from src
// land at LDS address lds + 16 l (lds wave-uniform).  Written as asm so that
// the compiler does not track it as an LDS write: it would otherwise wait for
// every such load in flight before each transposing LDS read, including the
// tiles fetched ahead.  No register receives data (nothing to be reused while
// the load is in flight); completion is waited for explicitly (wait_vmem)
// before the barrier that publishes a tile.
__device__ __forceinline__ void dma_load_16(const uint8_t* src, uint8_t* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// Same, with the LDS destination given by its generic address: the low 32
// bits of a generic pointer into the LDS aperture are the LDS address, which
// spares the address-space cast (whose null check some inlining contexts
// could not fold).
__device__ __forceinline__ void dma_load_16_g(const uint8_t* src, const uint8_t* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// Workgroup barrier for the ring.  No memory fence: the K/V tiles arrive by
// direct global->LDS loads whose completion each wave has already waited for
// (a fence would wait for every load in flight, including the tiles fetched
// ahead).  The empty asm statements keep the compiler from moving LDS
// accesses across the barrier, and the wait retires this wave's LDS reads
// before any wave may refill the buffer they read.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this wave's LDS reads have returned
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS loads of one 64-key tile.  The tile's LDS image (64 K
// rows at k_pitch, then 64 V rows at v_pitch) is a run of 16-byte slots; load
// i of the tile writes slots [64 i, 64 i + 64), lane l slot 64 i + l, so the
// lane fetches whichever 16 bytes belong there: the chunk of its row, or for a
// pad slot chunk 0 again (in bounds, never read).  Wave w issues loads w,
// w + NW, ...; per load it keeps its lane's row in the tile (high half) and
// the byte offset of its chunk in the row (low half) in one register.
template <int D, bool FP8, int NW>
struct TileLoads {
  using Gm = Geo<D, FP8>;
  static constexpr int per_wave = (Gm::ring_loads + NW - 1) / NW;
  static constexpr int min_per_wave = Gm::ring_loads / NW;
  static_assert(min_per_wave >= 1, "every wave issues loads of every tile");
  uint32_t slot_rc[per_wave];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
      const int i = wave + j * NW;
      const bool kreg = i < Gm::k_slots;
      const int slot = 64 * (kreg ? i : i - Gm::k_slots) + lane;
      const int per_row = kreg ? Gm::k_slots : Gm::v_slots;
      const int row = slot / per_row;
      const int ch = slot - row * per_row;
      slot_rc[j] = ((uint32_t)row << 16) | (ch < Gm::chunks ? (uint32_t)ch * 16u : 0u);
    }
  }

  __device__ __forceinline__ void issue(const uint8_t* __restrict__ kpool, const uint8_t* __restrict__ vpool,
                                        const PageWalk& w, int key0, uint8_t* buf, int wave) const {
    const int slot_mask = (1 << w.shift) - 1;
    // page ids of all loads first (one LDS round trip), then the loads; a
    // page base is one 32 x 32 -> 64-bit multiply-add and a slot offset one
    // 24-bit multiply-add (page bytes < 2^32, slot stride < 2^24: the plan
    // refuses larger geometry).  The fp8 instance keeps the 64-bit product:
    // there the shorter form gains nothing and its registers tip the kernel
    // into scratch.
    int key[per_wave];
    uint32_t page[per_wave];
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
      key[j] = min(key0 + (int)(slot_rc[j] >> 16), w.kend - 1);
      page[j] = (uint32_t)w.pcache[(key[j] >> w.shift) - w.first_page];
    }
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
      const int i = wave + j * NW;
      if (i < Gm::ring_loads) {
        const uint8_t* pool = (i < Gm::k_slots ? kpool : vpool) + w.head_off;
        if constexpr (FP8) {
          dma_load_16(pool + (int64_t)(int32_t)page[j] * w.page_bytes +
                          ((uint32_t)(key[j] & slot_mask) * (uint32_t)w.row_stride_b + (slot_rc[j] & 0xFFFFu)),
                      buf + 1024 * i);
        } else {
          const uint32_t in_page = __umul24((uint32_t)(key[j] & slot_mask), (uint32_t)w.row_stride_b) +
                                   (slot_rc[j] & 0xFFFFu);
          dma_load_16(pool + ((uint64_t)page[j] * (uint32_t)w.page_bytes + in_page), buf + 1024 * i);
        }
      }
    }
  }
};

// Raw scores of the 32 keys whose K rows start at kl: one MFMA chain.
template <int D, bool FP8, int KPITCH>
__device__ __forceinline__ f32x16 qk_tile(const uint8_t* kl, const bf16x8 (&qreg)[D / 16], int lane) {
  f32x16 s;
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) s = mfma32(k_operand<D, FP8, KPITCH>(kl, 0, j, lane), qreg[j], s);
  return s;
}

// O^T += V^T P^T for the 32 keys whose V rows start at vl.
template <int D, bool FP8, int VPITCH>
__device__ __forceinline__ void pv_tile(SoftmaxState<D>& st, const bf16x8 (&pb)[1][2], const uint8_t* vl,
                                        int lane) {
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) st.o[t] = mfma32(v_operand<FP8, VPITCH>(vl, 0, t, h, lane), pb[0][h], st.o[t]);
}

// One pipelined 32-key step of a wave: the score product of the NEXT step
// (K rows at kl) interleaved with the exp work of THIS step (raw scores sc),
// then this step's PV product (V rows at vl) interleaved with its row sum.
// The instruction order is fixed with scheduling barriers: each MFMA is
// preceded by the LDS read of the operand two MFMAs ahead and followed by its
// share of the VALU work, so that one wave keeps its matrix core fed while its
// VALU works through the softmax.
// Query operands of the streamed schedule: bf16 (16-wide k-steps) or, with
// fp8 queries, E4M3 (64-wide k-steps of the fp8 product).
template <bool QF8>
struct QOp {
  using reg = bf16x8;
  template <int D> struct n { static constexpr int value = D / 16; };
};
template <>
struct QOp<true> {
  using reg = i32x8;
  template <int D> struct n { static constexpr int value = D / 64; };
};

// With fp8 queries (QF8) the query operands are read from the wave's rows in
// LDS (qrow: this lane's row, 16-byte aligned) instead of qreg.
template <int D, bool FP8, int KPITCH, int VPITCH, bool QF8>
__device__ __forceinline__ void stream_step(SoftmaxState<D>& st, const f32x16& sc, f32x16& sn,
                                            const uint8_t* kl, const uint8_t* vl,
                                            const typename QOp<QF8>::reg (&qreg)[QOp<QF8>::template n<D>::value],
                                            const uint8_t* qrow, float c, float nref, int lane) {
  constexpr int NQ = QOp<QF8>::template n<D>::value;   // score MFMAs (k-steps over the head dim)
  constexpr int NT = D / 32;            // 32-wide d tiles of O
  constexpr int NV = 2 * NT;            // PV MFMAs; operand v = (tile v % NT, half v / NT)
  constexpr int EPQ = 16 / NQ;          // exps per score MFMA
  typename QOp<QF8>::reg ka[NQ];
  bf16x8 va[NV];
  float p[16];
  // operands are fetched two ahead of their MFMA: the K operands of the score
  // product, then the V operands of the PV product
  auto fetch = [&](int idx) {
    if (idx < NQ) {
      if constexpr (QF8) ka[idx] = k_operand_f8<KPITCH>(kl, 0, idx, lane);
      else ka[idx] = k_operand<D, FP8, KPITCH>(kl, 0, idx, lane);
    } else if (idx < NQ + NV) {
      const int v = idx - NQ;
      va[v] = v_operand<FP8, VPITCH>(vl, 0, v % NT, v / NT, lane);
    }
  };
#pragma unroll
  for (int i = 0; i < 16; ++i) sn[i] = 0.f;
  fetch(0);
  fetch(1);
  __builtin_amdgcn_sched_barrier(0);
  // Wave priorities: the score phase (MFMAs interleaved with this step's
  // exps) goes first, the PV burst second, the row max, mask and loop work
  // last, so that of the waves sharing a SIMD the one that can feed the
  // matrix core and the VALU at once is issued first.
  __builtin_amdgcn_s_setprio(3);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    fetch(j + 2);
    if constexpr (QF8) sn = mfma32_f8(ka[j], q8_operand(qrow, j), sn);
    else sn = mfma32(ka[j], qreg[j], sn);
#pragma unroll
    for (int e = 0; e < EPQ; ++e) {
      const int i = j * EPQ + e;
      p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c, nref));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  bf16x8 pb[2];
  pb[0] = pack_bf16x8(p);
  pb[1] = pack_bf16x8(p + 8);
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = p[i] + p[i + 8];
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    fetch(NQ + v + 2);
    st.o[v % NT] = mfma32(va[v], pb[v / NT], st.o[v % NT]);
    if (v == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] += q[i + 4];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  st.l += (q[0] + q[2]) + (q[1] + q[3]);
}

// Rows whose probabilities may go through the E4M3 PV product see at least
// this many keys.  An E4M3 probability is off by up to 2^-4 of itself; with
// hundreds of keys no single weight is large enough for that to move the
// output by more than a few 1e-3 on standard-normal data, while a row with a
// handful of keys could be moved by several 1e-2.
constexpr int kMinKeysF8Pv = 256;

// V^T operand of the E4M3 PV product for d-tile t of a 64-key tile (V rows
// of the tile from vl, fp8, row-major at VPITCH): lane l takes column
// 32 t + l % 32 and the 32 keys 32 (l / 32) + {0..7, 16..23, 8..15, 24..31}
// of the tile -- the order in which the probabilities of one 32-key step
// sit in a lane after pair_probs -- from four transposing reads (lane L of a
// 16-lane group receives 8 consecutive keys of one column).
template <int VPITCH>
__device__ __forceinline__ i32x8 v_operand_f8pair(const uint8_t* vl, int t, int lane) {
  const int L = lane & 15;
  const int d0 = 32 * t + 16 * ((lane >> 4) & 1);
  const uint8_t* src = vl + (32 * (lane >> 5) + (L >> 1)) * VPITCH + d0 + 8 * (L & 1);
  const i32x2 a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(src));
  const i32x2 b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(src + 16 * VPITCH));
  const i32x2 c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(src + 8 * VPITCH));
  const i32x2 d = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(src + 24 * VPITCH));
  return i32x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 16 probabilities (0 <= p <= 2^8) -> 16 E4M3 codes, byte i = code of p[i]
// (round to nearest even; the range needs no saturation).
__device__ __forceinline__ void pack_e4m3x16(const float* p, uint32_t (&w)[4]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * d], p[4 * d + 1], 0, false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * d + 2], p[4 * d + 3], x, true);
    w[d] = (uint32_t)x;
  }
}

// The E4M3 probabilities of two consecutive 32-key steps (x: the earlier one,
// y: the later one, each as this lane's 16 keys) rearranged for the B operand
// of one 32x32x64 product: lanes < 32 end with all 32 keys of the earlier
// step, lanes >= 32 with all 32 of the later one (one v_permlane32_swap per
// dword: the upper half-wave of x trades places with the lower half of y).
__device__ __forceinline__ i32x8 pair_probs(const uint32_t (&x)[4], const uint32_t (&y)[4]) {
  i32x8 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const auto s = __builtin_amdgcn_permlane32_swap((int)x[d], (int)y[d], false, false);
    r[d] = (int)s[0];
    r[4 + d] = (int)s[1];
  }
  return r;
}

// One pipelined 32-key step of the streamed schedule with fp8 queries whose
// probabilities go through the E4M3 PV product: as stream_step, the score
// product of the next step (K rows at kl) interleaved with the exp work of
// this step (raw scores sc); then, by MODE:
//   1  the first step of a 64-key tile: no PV product; the probabilities are
//      kept in E4M3 (stash) with the running max they were taken against;
//   2  the second step: its probabilities in E4M3 paired with the stash, one
//      v_mfma_scale_f32_32x32x64_f8f6f4 per 32-wide d tile over the tile's 64
//      V rows (from vl_tile).  The running max is an integer (log2 units), so
//      the stash's rescale since it was taken, 2^(m_stash - m), is a power of
//      two: the E8M0 block scale of its half of the keys (lanes < 32 supply
//      the scale of k-block 0 of their column, lanes >= 32 of k-block 1).
template <int D, int KPITCH, int VPITCH, int MODE>
__device__ __forceinline__ void stream_step_f8(SoftmaxState<D>& st, const f32x16& sc, f32x16& sn,
                                               const uint8_t* kl, const uint8_t* vl_tile,
                                               const uint8_t* qrow, float c, float nref,
                                               uint32_t (&stash)[4], float& m_stash, int lane) {
  static_assert(MODE == 1 || MODE == 2, "first or second step of a tile");
  constexpr int NQ = D / 64;            // score MFMAs
  constexpr int NT = D / 32;            // 32-wide d tiles of O
  constexpr int EPQ = 16 / NQ;          // exps per score MFMA
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) sn[i] = 0.f;
  i32x8 ka = k_operand_f8<KPITCH>(kl, 0, 0, lane);
  __builtin_amdgcn_sched_barrier(0);
  // wave priorities by phase, as in stream_step
  __builtin_amdgcn_s_setprio(3);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    sn = mfma32_f8(ka, q8_operand(qrow, j), sn);
    if (j + 1 < NQ) ka = k_operand_f8<KPITCH>(kl, 0, j + 1, lane);
#pragma unroll
    for (int e = 0; e < EPQ; ++e) {
      const int i = j * EPQ + e;
      p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c, nref));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(1);
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = p[i] + p[i + 8];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] += q[i + 4];
  st.l += (q[0] + q[2]) + (q[1] + q[3]);
  if constexpr (MODE == 1) {
    pack_e4m3x16(p, stash);
    m_stash = st.m;
  } else {
    uint32_t cur[4];
    pack_e4m3x16(p, cur);
    const i32x8 pb = pair_probs(stash, cur);
    int e = 127;
    if (lane < 32) {
      const float dm = m_stash - st.m;                 // an integer <= 0, or -inf/NaN when empty
      e = dm > -127.f ? 127 + (int)dm : 0;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const i32x8 va = v_operand_f8pair<VPITCH>(vl_tile, t, lane);
      st.o[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, st.o[t], 0, 0, 0, 127, 0, e);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// Tiles are issued NB-2 ahead: at the top of tile t every wave has waited for
// its loads of tiles t and t+1 and passed the barrier, so both are resident and
// every wave is done with tile t-1, whose buffer then receives tile t+NB-1.
// Within a tile each wave runs 32-key steps; step u issues the score product
// of step u+1 (K rows of tile t or t+1) before the softmax and PV product of
// step u, so the two products of a wave overlap its exp work.
template <int D, bool FP8, int MODE, bool QF8>
__device__ void stream_item(const AttnParams& p, uint8_t* smem, int32_t* pcache, const RowMap& rm,
                            const PageWalk& pw, int L, float c, float vdesc) {
  using Gm = Geo<D, FP8>;
  const SoftCap sc(p.softcap, c);
  constexpr int NW = Block<MODE, D, QF8>::waves;
  constexpr int NB = Gm::ring_bufs;
  static_assert(NB >= 3 && NB <= 4, "ring of three or four tiles");
  using TL = TileLoads<D, FP8, NW>;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrows = rm.ntok * rm.G;
  const int r0 = wave * kCols;
  const int last_tok = max(rm.ntok - 1, 0);

  // Q operands of this wave's rows, in registers (bf16, or E4M3 codes)
  typename QOp<QF8>::reg qreg[QOp<QF8>::template n<D>::value];   // bf16 queries only
  // fp8 queries: the wave's E4M3 query rows live in LDS (registers go to the
  // E4M3 PV product's state); this lane reads row lane % 32 from qrow
  const uint8_t* qrow = nullptr;
  {
    const int r = r0 + (lane & 31);
    const bool ok = r < nrows;
    const int tok = ok ? r / rm.G : 0;
    const int h = rm.g * rm.G + (r - tok * rm.G);
    if constexpr (QF8) {
      using LD = Lds<D, FP8, MODE>;
      uint8_t* qw = smem + LD::q8_off + (wave * kCols + (lane & 31)) * LD::q8_pitch + 32 * (lane >> 5);
      qrow = qw;
      // the loads are unconditional: a lane past the block's rows reads from
      // the first query row (head 0 of token 0 always exists), then drops it
      const int64_t off = ok ? (int64_t)(rm.t0 + tok) * p.q_stride_t + (int64_t)h * D : 0;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(p.q) + off + 32 * (lane >> 5);
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        u32x4 a = *reinterpret_cast<const u32x4*>(src + 64 * j);
        u32x4 b = *reinterpret_cast<const u32x4*>(src + 64 * j + 16);
        if (!ok) a = b = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(qw + 64 * j) = a;
        *reinterpret_cast<u32x4*>(qw + 64 * j + 16) = b;
      }
    } else {
      const uint16_t* src = p.q + (int64_t)(rm.t0 + tok) * p.q_stride_t + (int64_t)h * D + (lane >> 5) * 8;
#pragma unroll
      for (int j = 0; j < D / 16; ++j)
        qreg[j] = ok ? as_bf16x8(*reinterpret_cast<const u32x4*>(src + 16 * j)) : as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }

  int khi = L;
  if (p.causal) khi = min(khi, rm.pos0 + rm.ntok);
  const bool wave_active = r0 < nrows;
  const int tok_a = min(r0 / rm.G, last_tok);
  const int tok_b = min((r0 + kCols - 1) / rm.G, last_tok);
  const int wave_kmax = !wave_active ? 0 : (p.causal ? min(khi, rm.pos0 + tok_b + 1) : khi);
  const int wave_kfull = p.causal ? min(khi, rm.pos0 + tok_a + 1) : khi;   // keys < this visible to all rows
  const int my_tok = min((r0 + (lane & 31)) / rm.G, last_tok);
  const int klim = p.causal ? min(khi, rm.pos0 + my_tok + 1) : khi;       // this lane's row sees keys < klim

  SoftmaxState<D> st;
  state_init(st);
  float thr = neg_inf();                  // (st.m + slack) / c, raw-score units
  float nref = 0.f;                       // -st.m, or 0 while st.m is -inf
  TL tl;
  tl.init(wave, lane);
  PageWalk w = pw;
  const int chunk_keys = kPcacheEntries << w.shift;
  for (int cb = 0; cb < khi; cb += chunk_keys) {
    const int ce = min(khi, cb + chunk_keys);
    __syncthreads();
    fill_pcache(w, pcache, cb, ce);
    // The Q loads (first chunk) overlapped the page-table reads; let them land
    // here, once: vector-memory loads retire in order on one counter, and a Q
    // load still counted as outstanding at the first score product would make
    // the wait placed there (inside the tile loop) cover every tile's loads.
    wait_vmem_all();
    __syncthreads();
    const int ntiles = (ce - cb + kTile - 1) / kTile;
    const int kvis = min(wave_kmax, ce) - cb;                     // this wave's keys in the chunk
    const int nsub = kvis > 0 ? (kvis + kSub - 1) / kSub : 0;     // its 32-key steps
#pragma unroll
    for (int t = 0; t < NB - 1; ++t)
      if (t < ntiles) tl.issue(p.k_pool, p.v_pool, w, cb + t * kTile, smem + t * Gm::tile_bytes, wave);
    // Step u (u = -1 .. nsub-1) issues the scores of step u+1 and the softmax
    // and PV product of step u.  Step -1 has no keys of its own (scores -inf,
    // probabilities 0, its PV product adds nothing) and the scores issued by
    // the last step are dropped, so every step runs the same code.
    f32x16 s_cur;
#pragma unroll
    for (int i = 0; i < 16; ++i) s_cur[i] = neg_inf();
    int u = -1;
    for (int t = 0; t < ntiles; ++t) {
      if (NB == 4 && t + 2 < ntiles)
        wait_vmem<TL::min_per_wave>();      // tile t+2 may stay in flight
      else
        wait_vmem<0>();
      ring_barrier();
      if (t + NB - 1 < ntiles)
        tl.issue(p.k_pool, p.v_pool, w, cb + (t + NB - 1) * kTile, smem + ((t + NB - 1) % NB) * Gm::tile_bytes,
                 wave);
      // steps 2t and 2t+1 read tiles t and t+1 (step -1 also reads tile 0)
      const int u_end = min(2 * t + 2, nsub);
      // the scores of step u+1 (just computed into sn): cap, mask, row max
      auto next_scores = [&](f32x16 (&sn)[1]) {
        if (u + 1 < nsub) {
          const int k1 = cb + (u + 1) * kSub;
          if (sc.on()) cap_tile(sn[0], sc);
          if (k1 + kSub > wave_kfull) mask_tile(sn[0], k1, klim, lane);
          max_update_lane<D, QF8>(st, sn[0], c, thr, nref);
        }
        s_cur = sn[0];
      };
      auto k_rows = [&]() {                                  // K rows of step u+1's keys
        const int tk = (u + 1) >> 1;
        return smem + (tk % NB) * Gm::tile_bytes + ((u + 1) & 1) * kSub * Gm::k_pitch;
      };
      if constexpr (QF8) {
        // Tile t visible to every row of the wave, and every row seeing at
        // least kMinKeysF8Pv keys: its two steps' probabilities go through
        // the E4M3 PV product together.  Steps of a masked (diagonal or
        // tail) tile, and rows with few keys, keep the bf16 product.
        if (wave_kfull >= kMinKeysF8Pv && cb + kTile * (t + 1) <= wave_kfull) {
          if (u < 2 * t) {                                   // step -1 (t == 0): no keys of its own
            f32x16 sn[1];
            const uint8_t* vl = smem + Gm::tile_k_bytes + kSub * Gm::v_pitch;
            stream_step<D, FP8, Gm::k_pitch, Gm::v_pitch, QF8>(st, s_cur, sn[0], k_rows(), vl, qreg, qrow, c, nref, lane);
            next_scores(sn);
            ++u;
          }
          const uint8_t* vl_tile = smem + (t % NB) * Gm::tile_bytes + Gm::tile_k_bytes;
          uint32_t stash[4];
          float m_stash;
          __builtin_amdgcn_sched_barrier(0);
          {
            f32x16 sn[1];
            stream_step_f8<D, Gm::k_pitch, Gm::v_pitch, 1>(st, s_cur, sn[0], k_rows(), vl_tile, qrow, c, nref, stash,
                                                         m_stash, lane);
            next_scores(sn);
            ++u;
          }
          __builtin_amdgcn_sched_barrier(0);
          {
            f32x16 sn[1];
            stream_step_f8<D, Gm::k_pitch, Gm::v_pitch, 2>(st, s_cur, sn[0], k_rows(), vl_tile, qrow, c, nref, stash,
                                                         m_stash, lane);
            next_scores(sn);
            ++u;
          }
          continue;
        }
      }
#pragma unroll 1
      for (; u < u_end; ++u) {
        const int tv = max(u, 0) >> 1;                      // tile of step u's keys
        const uint8_t* vl = smem + (tv % NB) * Gm::tile_bytes + Gm::tile_k_bytes + (u & 1) * kSub * Gm::v_pitch;
        f32x16 sn[1];
        stream_step<D, FP8, Gm::k_pitch, Gm::v_pitch, QF8>(st, s_cur, sn[0], k_rows(), vl, qreg, qrow, c, nref, lane);
        next_scores(sn);
      }
    }
  }
  if (wave_active) {
    const float l_tot = st.l + xor32(st.l);
    write_rows<D>(p, st, l_tot, r0, rm, -1, vdesc, lane);
  }
}

// ---------------------------------------------------------------------------
// ring decode schedule (fp8 cache, head dim 256): waves split the key range of
// one block of <= 32 query rows; each wave streams its steps through a private
// ring of LDS half-step buffers filled by direct global->LDS loads
// ---------------------------------------------------------------------------

// Direct loads of one half-step (the K or the V rows of 32 keys from key0)
// into a swizzled buffer: load i fills bytes [1024 i, 1024 i + 1024), lane l
// the 16 bytes of slot 64 i + l, i.e. row r = (64 i + l) / 16 at chunk
// position l mod 16, which holds chunk (l mod 16) ^ (r mod 16) of that row.
// Keys past the live window are clamped to its last key (in bounds; the
// score mask gives them probability 0).
template <int D, bool FP8>
__device__ __forceinline__ void ring_issue(const uint8_t* __restrict__ pool, const PageWalk& w, int key0,
                                           uint8_t* buf, int lane) {
  using R = RingGeo<D, FP8>;
  const int slot_mask = (1 << w.shift) - 1;
  const int pos = lane & 15;
  if (w.shift >= 5 && key0 + kSub <= w.kend) {
    // 32 whole keys on one page (key0 is a multiple of 32): one page id
    const uint8_t* base = pool + (int64_t)w.pcache[(key0 >> w.shift) - w.first_page] * w.page_bytes +
                          w.head_off + (uint32_t)(key0 & slot_mask) * (uint32_t)w.row_stride_b;
#pragma unroll
    for (int i = 0; i < R::half_loads; ++i) {
      const int row = 4 * i + (lane >> 4);
      dma_load_16_g(base + ((uint32_t)row * (uint32_t)w.row_stride_b + (uint32_t)((pos ^ (row & 15)) * 16)),
                    buf + 1024 * i);
    }
    return;
  }
  int page[R::half_loads];
#pragma unroll
  for (int i = 0; i < R::half_loads; ++i)
    page[i] = w.pcache[(min(key0 + 4 * i + (lane >> 4), w.kend - 1) >> w.shift) - w.first_page];
#pragma unroll
  for (int i = 0; i < R::half_loads; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int key = min(key0 + row, w.kend - 1);
    const uint8_t* src = pool + (int64_t)page[i] * w.page_bytes + w.head_off +
                         ((uint32_t)(key & slot_mask) * (uint32_t)w.row_stride_b + (uint32_t)((pos ^ (row & 15)) * 16));
    dma_load_16_g(src, buf + 1024 * i);
  }
}

// K operand of k-step j from a swizzled half-step: K[key = kperm(lane%32)][d =
// 16 j + 8 (lane/32) .. +8] as bf16 (fp8 bytes widened exactly).
template <int D, bool FP8>
__device__ __forceinline__ bf16x8 k_operand_r(const uint8_t* kl, int j, int lane) {
  static_assert(FP8, "the ring buffers hold fp8 rows");
  using R = RingGeo<D, FP8>;
  const int row = kperm(lane & 31);
  const u32x2 v = *reinterpret_cast<const u32x2*>(kl + row * R::row_bytes + (j ^ (row & 15)) * 16 + 8 * (lane >> 5));
  return fp8x8_to_bf16(v[0], v[1]);
}

// V^T operand of d-tile t, k-step h from a swizzled half-step (the lane
// mapping of the transposing read is that of v_operand).
template <int D, bool FP8>
__device__ __forceinline__ bf16x8 v_operand_r(const uint8_t* vl, int t, int h, int lane) {
  static_assert(FP8, "the ring buffers hold fp8 rows");
  using R = RingGeo<D, FP8>;
  const int L = lane & 15;
  const int row = 16 * h + 8 * (lane >> 5) + (L >> 1);
  const int c = (2 * t + ((lane >> 4) & 1)) ^ (row & 15);
  const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vl + row * R::row_bytes + c * 16 + 8 * (L & 1)));
  return fp8x8_to_bf16((uint32_t)w[0], (uint32_t)w[1]);
}

// Merge the softmax states of the NW waves of a workgroup pairwise through
// LDS (lds_avail bytes from smem): the (m, l, O) of a writer wave is folded
// into a reader wave with the usual max-rescale; wave 0 ends with the total.
template <int D, int NW>
__device__ void merge_waves(SoftmaxState<D>& st, uint8_t* smem, int lds_avail, int wave, int lane) {
  constexpr int red_floats = D / 2 + 4;               // O registers, then (l, m), per lane
  const int nbuf = max(1, lds_avail / (red_floats * kWave * 4));
  float* red = reinterpret_cast<float*>(smem);
  int active = NW;
  while (active > 1) {
    const int half = active / 2;
    const int cnt = half < nbuf ? half : nbuf;
    const int w_lo = active - cnt;         // writers [w_lo, active)
    const int r_lo = active - 2 * cnt;     // readers [r_lo, w_lo)
    if (wave >= w_lo && wave < active) {
      f32x4* buf = reinterpret_cast<f32x4*>(red + (wave - w_lo) * red_floats * kWave);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          buf[(4 * t + q) * kWave + lane] = f32x4{st.o[t][4 * q], st.o[t][4 * q + 1], st.o[t][4 * q + 2], st.o[t][4 * q + 3]};
      buf[(D / 8) * kWave + lane] = f32x4{st.l, st.m, 0.f, 0.f};
    }
    __syncthreads();
    if (wave >= r_lo && wave < w_lo) {
      const f32x4* buf = reinterpret_cast<const f32x4*>(red + (wave - r_lo) * red_floats * kWave);
      const f32x4 lm = buf[(D / 8) * kWave + lane];
      const float mm = fmaxf(st.m, lm[1]);
      const float ref = mm == neg_inf() ? 0.f : mm;
      const float a1 = __builtin_amdgcn_exp2f(st.m - ref);
      const float a2 = __builtin_amdgcn_exp2f(lm[1] - ref);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = buf[(4 * t + q) * kWave + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) st.o[t][4 * q + e] = st.o[t][4 * q + e] * a1 + v[e] * a2;
        }
      st.l = st.l * a1 + lm[0] * a2;
      st.m = mm;
    }
    __syncthreads();
    active = w_lo;
  }
}

// One (sequence, KV head, key window [klo, khi)) item whose packed query rows
// fit one MFMA column tile, on an fp8 cache at head dim 256.  Eight waves, two
// per SIMD; wave w takes the 32-key steps w, w + 8, ... of the window.  The
// block's query rows are staged once in LDS and read as the B operand of each
// score k-step (in registers they would take 64 of the 256 registers two
// waves per SIMD leave).  A wave's private LDS holds the K and V rows of one
// step: the K rows of step s + 1 are requested as soon as the score product
// of step s has read its K buffer, the V rows as soon as its PV product has
// read the V buffer, with no register holding data in flight and no
// workgroup barrier in the key loop; a wave waiting for its rows or for the
// load path leaves its SIMD to the other wave.  Every step converts each fp8
// byte once; the eight waves' softmax states are merged at the end.
template <int D, bool FP8, int MODE>
__device__ void ring_item(const AttnParams& p, uint8_t* smem, int32_t* pcache, const RowMap& rm,
                          const PageWalk& pw, int L, int klo, int khi, int slot, float c, float vdesc) {
  using R = RingGeo<D, FP8>;
  constexpr int NW = kRingWaves;
  constexpr int HL = R::half_loads;
  const SoftCap sc(p.softcap, c);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrows = rm.ntok * rm.G;

  if (p.causal) khi = min(khi, rm.pos0 + rm.ntok);
  SoftmaxState<D> st;
  state_init(st);
  if (khi <= klo) {
    if (wave == 0) write_rows<D>(p, st, 0.f, 0, rm, slot, vdesc, lane);
    return;
  }

  // the block's query rows (zero past the last row) into LDS: 32 rows of
  // D / 8 16-byte chunks, two chunks per thread
  uint8_t* qlds = smem + R::q_off;
  {
    constexpr int QCH = D / 8;
    for (int i = threadIdx.x; i < kCols * QCH; i += NW * kWave) {
      const int r = i / QCH, ch = i - r * QCH;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (r < nrows) {
        const int tok = r / rm.G;
        const int h = rm.g * rm.G + (r - tok * rm.G);
        v = *reinterpret_cast<const u32x4*>(p.q + (int64_t)(rm.t0 + tok) * p.q_stride_t + (int64_t)h * D + 8 * ch);
      }
      *reinterpret_cast<u32x4*>(qlds + r * R::q_pitch + 16 * ch) = v;
    }
  }
  // B operand of k-step j: row lane % 32, columns 16 j + 8 (lane / 32) .. +7
  const uint8_t* qsrc = qlds + (lane & 31) * R::q_pitch + 16 * (lane >> 5);
  const int my_tok = min((lane & 31) / rm.G, max(rm.ntok - 1, 0));
  const int klim = p.causal ? min(khi, rm.pos0 + my_tok + 1) : khi;   // this lane's row sees keys < klim
  const int kfull = p.causal ? min(khi, rm.pos0 + 1) : khi;           // keys < kfull visible to every row

  uint8_t* kl = smem + wave * R::wave_bytes;           // K, then V
  uint8_t* vl = kl + R::half_bytes;
  PageWalk w = pw;
  const int chunk_keys = kPcacheEntries << w.shift;
  for (int cb = klo; cb < khi; cb += chunk_keys) {
    const int ce = min(khi, cb + chunk_keys);
    __syncthreads();                                     // the buffers and page cache are free; Q staged
    fill_pcache(w, pcache, cb, ce);
    wait_vmem_all();                                     // page-table reads
    __syncthreads();
    const int nsteps = (ce - cb + kSub - 1) / kSub;
    const int mine = nsteps > wave ? (nsteps - wave + NW - 1) / NW : 0;   // this wave's steps
    if (mine > 0) {
      // Steps past the wave's last are requested too (clamped to the window's
      // last key): every iteration then has the same loads in flight and the
      // same wait counts.
      auto key_of = [&](int i) { return cb + kSub * min(wave + NW * i, nsteps - 1); };
      ring_issue<D, FP8>(p.k_pool, w, key_of(0), kl, lane);
      ring_issue<D, FP8>(p.v_pool, w, key_of(0), vl, lane);
      for (int i = 0; i < mine; ++i) {
        const int key0 = cb + kSub * (wave + NW * i);
        // the operand addresses (swizzled per lane) are recomputed every step
        // from an opaque copy of the lane id: hoisted, they would hold some
        // 32 registers for the whole kernel
        const int ln = item_tid() & (kWave - 1);
        wait_vmem<HL>();                                 // K(i) landed; V(i) may fly
        f32x16 sv[1];
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[0][e] = 0.f;
        u32x4 qb = *reinterpret_cast<const u32x4*>(qsrc);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const u32x4 qn = j + 1 < D / 16 ? *reinterpret_cast<const u32x4*>(qsrc + 32 * (j + 1)) : qb;
          sv[0] = mfma32(k_operand_r<D, FP8>(kl, j, ln), as_bf16x8(qb), sv[0]);
          qb = qn;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): the K reads have returned
        ring_issue<D, FP8>(p.k_pool, w, key_of(i + 1), kl, lane);
        if (sc.on()) cap_tile(sv[0], sc);
        if (key0 + kSub > kfull) mask_tile(sv[0], key0, klim, lane);
        wait_vmem<HL>();                                 // V(i) landed; K(i+1) may fly
        bf16x8 pb[1][2];
        softmax_p<D, 1>(st, sv, c, pb);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h) st.o[t] = mfma32(v_operand_r<D, FP8>(vl, t, h, ln), pb[0][h], st.o[t]);
        __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): the V reads have returned
        ring_issue<D, FP8>(p.v_pool, w, key_of(i + 1), vl, lane);
      }
      wait_vmem_all();                                   // nothing lands in the buffers later
    }
  }
  __syncthreads();
  merge_waves<D, NW>(st, smem, R::ring_bytes, wave, lane);
  if (wave == 0) {
    const float l_tot = st.l + xor32(st.l);
    write_rows<D>(p, st, l_tot, 0, rm, slot, vdesc, lane);
  }
}

// ---------------------------------------------------------------------------
// the kernel: work-item decode, then one of the schedules
// ---------------------------------------------------------------------------

// Row map and page walk of the item (sequence b, KV head g, query tokens
// t0 .. t0+ntok-1 at offset i0 of its q_len); returns the live key count.
template <int D, bool FP8>
__device__ __forceinline__ int item_setup(const AttnParams& p, int b, int g, int t0, int ntok, int q_len,
                                          int i0, RowMap& rm, PageWalk& pw) {
  const int L = min(p.seq_lens[b], p.pt_cols << p.page_shift);
  rm.t0 = t0;
  rm.ntok = ntok;
  // position of the block's first token: the queries are the last q_len keys
  rm.pos0 = L - q_len + i0;
  rm.g = g;
  rm.G = p.group;
  pw.pt_row = p.page_table + (int64_t)b * p.pt_row_stride;
  pw.page_bytes = p.kv_page_bytes;
  pw.head_off = (int64_t)g * Geo<D, FP8>::row_bytes;
  pw.row_stride_b = p.num_kv_heads * Geo<D, FP8>::row_bytes;
  pw.shift = p.page_shift;
  pw.klimit = L;
  return L;
}

// Exp2-domain score scale (softmax_scale * log2 e, times k_descale for fp8)
// and the factor applied to O at the end (v_descale for fp8).
template <bool FP8>
__device__ __forceinline__ void score_scales(const AttnParams& p, float& c, float& vdesc) {
  c = p.scale_log2;
  vdesc = 1.f;
  if (FP8) {
    c *= *p.k_descale;
    vdesc = *p.v_descale;
  }
}

// Balanced (persistent) decode.  The items (sequence b, KV head g) are laid
// end to end in units of kUnitKeys keys, b-major: item (b, g) covers units
// [Hkv S_b + g s_b, + s_b) with s_b = ceil(L_b / kUnitKeys) (0 when the
// sequence has no query token) and S_b the prefix sum of s.  The grid holds
// exactly the workgroups that fit on the device at once; workgroup w takes
// units [w U, (w+1) U), U = ceil(total / grid), and runs them piece by piece
// (a piece = the part of one item inside the range) with the decode schedule.
// A piece that is a whole item writes its rows; a cut piece writes a partial
// record into slot 2w (the range's first piece) or 2w+1 (its last), and
// merge_balanced_kernel combines the pieces of cut items.  Every workgroup
// has the same number of keys to stream, so no tail of long items is left to
// a few compute units.  Workgroup 0 publishes U, the total and S_b for the
// merge in p.sched.
constexpr int kUnitKeys = 128;
constexpr int kUnitShift = 7;

__device__ __forceinline__ int seq_units(const AttnParams& p, int b) {
  const int qn = p.cu_q_lens ? p.cu_q_lens[b + 1] - p.cu_q_lens[b] : 1;
  const int L = min(p.seq_lens[b], p.pt_cols << p.page_shift);
  return (qn > 0 && L > 0) ? (L + kUnitKeys - 1) >> kUnitShift : 0;
}

// Balanced schedule prologue: the unit scan (block-wide prefix sum of
// seq_units over the batch, NTH threads), this workgroup's units [u0, u1)
// with U = ceil(total / grid) and the sequence b holding u0 with its unit
// offset S_b; workgroup 0 publishes U, the total and every S_b in p.sched.
// `per_seq` is the number of items per sequence (KV heads, or MLA head
// groups).  Returns false when the workgroup has no units.
template <int NTH>
__device__ bool balanced_start(const AttnParams& p, uint8_t* smem, int* meta, int per_seq, int& u0, int& u1,
                               int& b, int& S) {
  const int tid = threadIdx.x;
  const int B = p.num_seqs;
  // units per thread chunk of sequences, then an exclusive scan over threads
  const int per = (B + NTH - 1) / NTH;
  const int j0 = min(B, tid * per), j1 = min(B, j0 + per);
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += seq_units(p, j);
  int* scan = reinterpret_cast<int*>(smem);
  scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < NTH; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int excl = scan[tid] - mine;           // sequence units before this chunk
  const int total = scan[NTH - 1] * per_seq;   // item units in the whole batch
  const int W = gridDim.x;
  const int U = (total + W - 1) / max(W, 1);
  const int w = blockIdx.x;
  u0 = min(total, w * U);
  u1 = min(total, u0 + U);
  if (w == 0) {
    if (tid == 0) {
      p.sched[0] = U;
      p.sched[1] = total;
    }
    int acc = excl;
    for (int j = j0; j < j1; ++j) {
      p.sched[4 + j] = acc;
      acc += seq_units(p, j);
    }
    if (tid == NTH - 1) p.sched[4 + B] = acc;
  }
  // the sequence holding unit u0
  if (u0 < u1 && per_seq * excl <= u0 && u0 < per_seq * (excl + mine)) {
    int acc = excl;
    for (int j = j0; j < j1; ++j) {
      const int sj = seq_units(p, j);
      if (u0 < per_seq * (acc + sj)) {
        meta[0] = j;
        meta[1] = acc;
        break;
      }
      acc += sj;
    }
  }
  __syncthreads();
  if (u0 >= u1) return false;
  b = __builtin_amdgcn_readfirstlane(meta[0]);
  S = __builtin_amdgcn_readfirstlane(meta[1]);
  return true;
}

template <int D, bool FP8, int MODE>
__device__ void balanced_decode(const AttnParams& p, uint8_t* smem, int32_t* pcache, int* meta) {
  const int Hkv = p.num_kv_heads;
  const int w = blockIdx.x;
  int u0, u1, b, S;
  if (!balanced_start<Shape<D, FP8, MODE>::threads>(p, smem, meta, Hkv, u0, u1, b, S)) return;
  float c, vdesc;
  score_scales<FP8>(p, c, vdesc);
  int u = u0;
  int piece = 0;
  while (u < u1) {
    const int sb = seq_units(p, b);
    const int item0 = Hkv * S;
    if (sb == 0 || u >= item0 + Hkv * sb) {     // past this sequence's items
      S += sb;
      ++b;
      continue;
    }
    const int g = (u - item0) / sb;
    const int a0 = item0 + g * sb;
    const int a1 = a0 + sb;
    const int pu1 = min(u1, a1);
    const int t0 = p.cu_q_lens ? p.cu_q_lens[b] : b;
    RowMap rm;
    PageWalk pw;
    const int L = item_setup<D, FP8>(p, b, g, t0, 1, 1, 0, rm, pw);
    const int klo = (u - a0) << kUnitShift;
    const int khi = min(L, (pu1 - a0) << kUnitShift);
    const int slot = (u == a0 && pu1 == a1) ? -1 : 2 * w + (piece == 0 ? 0 : 1);
    if constexpr (RingDec<D, FP8, MODE>::value)
      ring_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, klo, khi, slot, c, vdesc);
    else
      keysplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, klo, khi, slot, c, vdesc);
    __syncthreads();                            // LDS is reused by the next piece
    u = pu1;
    ++piece;
  }
}

// Task-queue schedule of a mixed batch.  Work items are split into two lists
// by the kind of work: prefill-type items (sequence b with q_len_b * G > 32:
// one per (q-block, KV head); within a sequence KV-head major, each head's
// q-blocks last-first, i.e. most keys first) are compute-bound, decode-type
// items (one per (sequence, KV head)) are memory-bound.  queue_setup_kernel
// lays both lists out (per sequence offsets) and zeroes the counters.  The
// grid holds the workgroups that fit on the device at once; each one draws
// items from the two lists with atomic counters until both are empty.  The
// first workgroup to arrive on a compute unit prefers the prefill list and
// the second the decode list, so that a compute-bound and a memory-bound item
// tend to share each compute unit; a workgroup whose preferred list is empty
// takes the other.  The prefill list is cut into kQueueShares contiguous
// shares with a counter each: a workgroup draws from the share of its own
// XCD (workgroups are dealt to the XCDs round-robin by linear id) and only
// when that is empty from the next ones, so the q-blocks of one (sequence,
// KV head), which read the same K/V rows, run under one L2.  Every draw
// either claims one of the finitely many items or finds all lists empty, so
// every workgroup ends without waiting on another.
constexpr int kQmPref = 8;      // LDS metadata words used by the queue loop
constexpr int kQmWhich = 9;
constexpr int kQmItem = 10;
constexpr int kQmSeq = 11;

// Claim a prefill-type item: the own share first, then the others in turn;
// -1 when every share is empty.
__device__ __forceinline__ int draw_prefill(int32_t* ctr, int n, int xcd) {
  for (int s = 0; s < kQueueShares; ++s) {
    const int y = (xcd + s) % kQueueShares;
    const int lo = (int)((int64_t)y * n / kQueueShares);
    const int hi = (int)((int64_t)(y + 1) * n / kQueueShares);
    if (lo >= hi) continue;
    const int k = atomicAdd(&ctr[y], 1);
    if (lo + k < hi) return lo + k;
  }
  return -1;
}

template <int D, bool FP8, int MODE>
__device__ void queue_mixed(const AttnParams& p, uint8_t* smem, int32_t* pcache, int* meta) {
  constexpr int NTH = Block<MODE, D>::threads;
  const int B = p.num_seqs;
  const int xcd = blockIdx.x % kQueueShares;
  if (threadIdx.x == 0)
    meta[kQmPref] = atomicAdd(&p.sched[kQueueCtrs + (__smid() & (kQueueSlots - 1))], 1) & 1;
  __syncthreads();
  int pref = meta[kQmPref];
  for (;;) {
    __syncthreads();                            // the previous item is done with LDS and meta
    if (threadIdx.x == 0) {
      // list l's offsets start at sched + kQueueCtrs + kQueueSlots + l (B + 1);
      // its item count is the last offset
      const int32_t* lists = p.sched + kQueueCtrs + kQueueSlots;
      const int np = lists[B], nd = lists[(B + 1) + B];
      int which = pref, k = -1;
      for (int attempt = 0; attempt < 2 && k < 0; ++attempt, which ^= 1) {
        if (which == 0) {
          k = draw_prefill(p.sched, np, xcd);
        } else {
          k = atomicAdd(&p.sched[kQueueDecodeCtr], 1);
          if (k >= nd) k = -1;
        }
        if (k >= 0) break;
      }
      meta[kQmWhich] = which;
      meta[kQmItem] = k;
      meta[kQmSeq] = -1;
    }
    __syncthreads();
    const int which = meta[kQmWhich];
    const int k = meta[kQmItem];
    if (k < 0) break;
    pref = which;
    // the sequence whose range [off[b], off[b+1]) holds item k
    const int32_t* off = p.sched + kQueueCtrs + kQueueSlots + which * (B + 1);
    for (int j = threadIdx.x; j < B; j += NTH)
      if (off[j] <= k && k < off[j + 1]) meta[kQmSeq] = j;
    __syncthreads();
    const int b = meta[kQmSeq];
    if (b < 0) break;                           // counters not set up: nothing to claim
    const int r = k - off[b];
    const int t0 = p.cu_q_lens[b];
    const int q_len = p.cu_q_lens[b + 1] - t0;
    const int BQ = p.q_block_tokens;
    int g, i0, ntok;
    if (which == 0) {
      const int nb = (q_len + BQ - 1) / BQ;
      g = r / nb;
      i0 = (nb - 1 - (r - g * nb)) * BQ;
      ntok = min(BQ, q_len - i0);
    } else {
      g = r;
      i0 = 0;
      ntok = q_len;
    }
    RowMap rm;
    PageWalk pw;
    const int L = item_setup<D, FP8>(p, b, g, t0 + i0, ntok, q_len, i0, rm, pw);
    float c, vdesc;
    score_scales<FP8>(p, c, vdesc);
    if (which == 0)
      rowsplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, 0, c, vdesc);
    else
      keysplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, 0, L, -1, c, vdesc);
  }
}

// Lays out the two item lists of the task-queue schedule (one workgroup):
// per-sequence item counts, an exclusive scan over the batch, and zeroed
// draw and arrival counters.
__global__ __launch_bounds__(1024) void queue_setup_kernel(QueueSetupParams q) {
  __shared__ int sp[1024];
  __shared__ int sd[1024];
  const int B = q.num_seqs;
  const int t = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int j0 = min(B, t * per);
  const int j1 = min(B, j0 + per);
  auto counts = [&](int j, int& np, int& nd) {
    const int ql = q.cu_q_lens[j + 1] - q.cu_q_lens[j];
    np = nd = 0;
    if (ql <= 0) return;
    if (ql * q.group > kCols) np = (ql + q.q_block_tokens - 1) / q.q_block_tokens * q.num_kv_heads;
    else nd = q.num_kv_heads;
  };
  int cp = 0, cd = 0;
  for (int j = j0; j < j1; ++j) {
    int np, nd;
    counts(j, np, nd);
    cp += np;
    cd += nd;
  }
  sp[t] = cp;
  sd[t] = cd;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {       // inclusive scan
    const int a = t >= o ? sp[t - o] : 0;
    const int d = t >= o ? sd[t - o] : 0;
    __syncthreads();
    sp[t] += a;
    sd[t] += d;
    __syncthreads();
  }
  int32_t* offp = q.sched + kQueueCtrs + kQueueSlots;
  int32_t* offd = offp + B + 1;
  int ep = sp[t] - cp, ed = sd[t] - cd;
  for (int j = j0; j < j1; ++j) {
    int np, nd;
    counts(j, np, nd);
    offp[j] = ep;
    offd[j] = ed;
    ep += np;
    ed += nd;
  }
  if (t == 1023) {
    offp[B] = sp[1023];
    offd[B] = sd[1023];
  }
  if (t < kQueueCtrs) q.sched[t] = 0;
  for (int i = t; i < kQueueSlots; i += 1024) q.sched[kQueueCtrs + i] = 0;
}

// QF8: queries arrive as E4M3 codes (fp8 inputs); only the streamed prefill
// of an fp8 cache has that variant.  QUEUE: the task-queue schedule of a
// mixed batch (its own instance, so that its loop does not change the
// register allocation of the one-item-per-workgroup kernel).
template <int D, bool FP8, int MODE, bool QF8 = false, bool QUEUE = false>
__global__ __launch_bounds__((Shape<D, FP8, MODE, QF8>::threads))
__attribute__((amdgpu_waves_per_eu(Shape<D, FP8, MODE, QF8>::waves_per_eu, Shape<D, FP8, MODE, QF8>::waves_per_eu)))
void attn_kernel(AttnParams p) {
  static_assert(!QF8 || (FP8 && MODE == kPrefill && Block<MODE, D>::stream), "fp8 queries: streamed fp8 prefill only");
  static_assert(!QUEUE || MODE == kMixed, "task queues: mixed batches only");
  __shared__ __attribute__((aligned(16))) uint8_t smem[Lds<D, FP8, MODE>::bytes];
  int* meta = reinterpret_cast<int*>(smem + Lds<D, FP8, MODE>::base);
  int32_t* pcache = reinterpret_cast<int32_t*>(smem + Lds<D, FP8, MODE>::pcache_off);
  if constexpr (MODE == kDecode) {
    if (p.balanced) {
      balanced_decode<D, FP8, MODE>(p, smem, pcache, meta);
      return;
    }
  }
  if constexpr (QUEUE) {
    queue_mixed<D, FP8, MODE>(p, smem, pcache, meta);
    return;
  }
  const int split = blockIdx.z;
  int g = blockIdx.y;
  int b, t0, ntok, q_len, i0 = 0;
  if constexpr (MODE == kDecode) {
    b = blockIdx.x;
    if (p.cu_q_lens) {
      t0 = p.cu_q_lens[b];
      q_len = p.cu_q_lens[b + 1] - t0;
      ntok = min(q_len, 1);
    } else {
      t0 = b;
      q_len = 1;
      ntok = 1;
    }
  } else {
    // Work item -> (sequence, q-block).  Sequence b owns the block indices
    // [cu[b]/BQ + b, cu[b]/BQ + b + ceil(q_len_b/BQ)), which never overlap
    // and stay below cu[B]/BQ + B, so the grid can be sized from host bounds.
    const int BQ = p.q_block_tokens;
    // Workgroups are dealt to the XCDs round-robin by linear id.  Remap so that
    // each XCD takes a contiguous range of the logical list (KV head major,
    // then q-block): the q-blocks that stream the same K/V share one L2.
    // Prefill runs each sequence's q-blocks last-first (most keys first).
    // Mixed batches deal the two halves of each KV head's block range
    // alternately, so that with prefill chunks and decode rows in separate
    // halves a compute-bound and a memory-bound block tend to share a
    // compute unit (measured 2 % faster on the 1000-token serving mix).
    int x;
    {
      const int X = gridDim.x;
      const int n = X * gridDim.y;
      const int lin = blockIdx.x + X * blockIdx.y;
      const int full = n - n % kXcds;
      const int logical = lin < full ? (lin % kXcds) * (full / kXcds) + lin / kXcds : lin;
      g = logical / X;
      x = logical - g * X;
      if (MODE == kPrefill) x = X - 1 - x;
      // mixed: deal the two halves of each KV head's block range alternately
      // (a perfect shuffle)
      if (MODE == kMixed) {
        const int h2 = X >> 1;
        if (x < 2 * h2) x = (x & 1) ? h2 + (x >> 1) : (x >> 1);
      }
    }
    if (threadIdx.x == 0) meta[0] = 0;
    __syncthreads();
    int cnt = 0;
    for (int j = threadIdx.x; j < p.num_seqs; j += Block<MODE, D, QF8>::threads) cnt += (p.cu_q_lens[j] / BQ + j <= x) ? 1 : 0;
    if (cnt) atomicAdd(&meta[0], cnt);
    __syncthreads();
    b = meta[0] - 1;
    if (b < 0) return;
    t0 = p.cu_q_lens[b];
    q_len = p.cu_q_lens[b + 1] - t0;
    const int local = x - (t0 / BQ + b);
    i0 = local * BQ;
    if (i0 >= q_len) return;
    ntok = min(BQ, q_len - i0);
    t0 += i0;
  }
  if (ntok <= 0) {
    // no query row in this block; nothing to write
    return;
  }
  RowMap rm;
  PageWalk pw;
  const int L = item_setup<D, FP8>(p, b, g, t0, ntok, q_len, i0, rm, pw);
  float c, vdesc;
  score_scales<FP8>(p, c, vdesc);
  const int klo = split * p.split_keys;
  const int khi = split == p.num_splits - 1 ? L : min(L, klo + p.split_keys);   // the last window takes the rest
  const int slot = p.num_splits > 1 ? split : -1;
  if constexpr (MODE == kDecode) {
    if constexpr (RingDec<D, FP8, MODE>::value)
      ring_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, klo, khi, slot, c, vdesc);
    else
      keysplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, klo, khi, slot, c, vdesc);
  } else if constexpr (MODE == kPrefill) {
    if constexpr (Block<MODE, D>::stream)
      stream_item<D, FP8, MODE, QF8>(p, smem, pcache, rm, pw, L, QF8 ? c * *p.q_descale : c, vdesc);
    else
      rowsplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, 0, c, vdesc);
  } else {
    if (q_len * p.group <= kCols)
      keysplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, klo, khi, slot, c, vdesc);
    else
      rowsplit_item<D, FP8, MODE>(p, smem, pcache, rm, pw, L, split, c, vdesc);
  }
}

// ---------------------------------------------------------------------------
// MLA decode: one logical KV head whose 576-wide cached row (512 latent
// values, then the 64-wide RoPE key) is the key, and whose latent part is the
// value; up to 128 query heads share it
// ---------------------------------------------------------------------------

constexpr int kMlaLatent = 512;
constexpr int kMlaDk = 576;

// One 32-key tile of latent rows at a 1168-byte pitch (72 data slots of 16
// bytes and a pad slot per row), rounded up to whole 1 KB direct loads.
struct MlaGeo {
  static constexpr int row_bytes = kMlaDk * 2;
  static constexpr int chunks = row_bytes / 16;
  static constexpr int pitch = row_bytes + 32;
  static constexpr int slots = pitch / 16;
  static constexpr int loads = (kSub * slots + 63) / 64;
  static constexpr int tile_bytes = loads * 1024;
};

// Direct global->LDS loads of one 32-key tile: load i writes slots
// [64 i, 64 i + 64) of the tile; lane l fetches the 16 bytes that belong at
// slot 64 i + l (a pad slot re-fetches chunk 0 of its row, a slot past the 32
// rows chunk 0 of row 31: in bounds, never read).  Loader wave w of NW issues
// loads w, w + NW, ...
template <int NW>
struct MlaLoads {
  static constexpr int per_wave = (MlaGeo::loads + NW - 1) / NW;
  static constexpr int min_per_wave = MlaGeo::loads / NW;
  uint32_t slot_rc[per_wave];   // row in the tile (high half), byte offset in the row

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
      const int slot = 64 * (wave + j * NW) + lane;
      int row = slot / MlaGeo::slots;
      int ch = slot - row * MlaGeo::slots;
      if (row >= kSub) {
        row = kSub - 1;
        ch = 0;
      }
      slot_rc[j] = ((uint32_t)row << 16) | (ch < MlaGeo::chunks ? (uint32_t)ch * 16u : 0u);
    }
  }

  __device__ __forceinline__ void issue(const uint8_t* __restrict__ pool, const PageWalk& w, int key0,
                                        uint8_t* buf, int wave) const {
    const int slot_mask = (1 << w.shift) - 1;
    if (w.shift >= 5 && key0 + kSub <= w.kend) {
      // the tile's 32 keys are whole and share one page (key0 is a multiple
      // of 32): one page id, then each load is that row's base plus the
      // lane's offset
      const uint8_t* base = pool + (int64_t)w.pcache[(key0 >> w.shift) - w.first_page] * w.page_bytes +
                            (uint32_t)(key0 & slot_mask) * (uint32_t)MlaGeo::row_bytes;
#pragma unroll
      for (int j = 0; j < per_wave; ++j) {
        const int i = wave + j * NW;
        if (i < MlaGeo::loads)
          dma_load_16(base + ((slot_rc[j] >> 16) * (uint32_t)MlaGeo::row_bytes + (slot_rc[j] & 0xFFFFu)),
                      buf + 1024 * i);
      }
      return;
    }
    int key[per_wave], page[per_wave];
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
      key[j] = min(key0 + (int)(slot_rc[j] >> 16), w.kend - 1);
      page[j] = w.pcache[(key[j] >> w.shift) - w.first_page];
    }
#pragma unroll
    for (int j = 0; j < per_wave; ++j) {
      const int i = wave + j * NW;
      if (i < MlaGeo::loads) {
        const uint8_t* src = pool + (int64_t)page[j] * w.page_bytes +
                             ((uint32_t)(key[j] & slot_mask) * (uint32_t)MlaGeo::row_bytes + (slot_rc[j] & 0xFFFFu));
        dma_load_16(src, buf + 1024 * i);
      }
    }
  }
};

// One soft-capped value (same formula as cap_tile).
__device__ __forceinline__ float cap1(float x, const SoftCap& sc) {
  const float e = __builtin_amdgcn_exp2f(x * sc.k2);
  return __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f) * sc.inv_b;
}

__device__ __forceinline__ f32x4 mfma16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kMlaHeads = 16;                    // query heads per wave
constexpr int kMlaQSteps = kMlaDk / 32;          // 32-wide k-steps of the score product
constexpr int kMlaVTilesHalf = kMlaLatent / 32;  // 16-wide value tiles in half the columns

// Waves of a head-split MLA workgroup: eight, two per SIMD (waves w and
// w + 4 share 16 heads and split each tile's keys for the scores and the
// value columns for the output), so that one wave's LDS reads and softmax
// overlap the other's MFMAs.  (One wave per SIMD holding all 512 columns of
// its heads left every latency of the loop exposed.)
constexpr int kMlaHsWaves = 8;

// Running state of one wave: its 16 heads over its keys and NVT 16-wide value
// tiles.  Lane l holds head l % 16; o[t][i] is value column
// col0 + 16 t + 4 (l / 16) + i; l is this lane's part of the row sum (its
// eight keys of each tile); m is the same on the four lanes of a head.
template <int NVT>
struct MlaState {
  f32x4 o[NVT];
  float m, l;
};

__device__ __forceinline__ bf16x8 join_bf16x4(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// LDS of a key-pair MLA workgroup: a ring of four 32-key tiles, the score
// exchange buffer (one 1 KB record per wave), then a page-id cache of 512
// entries (half the usual, so that all of it fits in 160 KB).
struct MlaPairLds {
  static constexpr int ring = 4;
  static constexpr int pcache_entries = 512;
  static constexpr int xbuf_off = ring * MlaGeo::tile_bytes;
  static constexpr int pcache_off = xbuf_off + kMlaHsWaves * kWave * 16 + 64;
  static constexpr int bytes = pcache_off + pcache_entries * 4;
  static_assert(bytes <= kLdsMax, "MLA LDS budget exceeded");
};

// Scores S^T = K Q^T of one 16-key half of a tile (rows 16 kh .. 16 kh + 15
// of the LDS tile at kl) for this wave's 16 heads, on 16x16x32 MFMAs: lane l
// gets head l % 16, keys 4 (l / 16) .. +3 of the half.  Operand reads run one
// k-step pair ahead of their MFMAs.
__device__ __forceinline__ f32x4 mla_half_scores(const uint8_t* kl, int kh, const bf16x8 (&qreg)[kMlaQSteps],
                                                 int lane) {
  constexpr int NP = kMlaQSteps / 2;
  const uint8_t* krow = kl + (16 * kh + (lane & 15)) * MlaGeo::pitch + 16 * (lane >> 4);
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  u32x4 ka[NP][2];
  ka[0][0] = *reinterpret_cast<const u32x4*>(krow);
  ka[0][1] = *reinterpret_cast<const u32x4*>(krow + 64);
#pragma unroll
  for (int jp = 0; jp < NP; ++jp) {
    if (jp + 1 < NP) {
      ka[jp + 1][0] = *reinterpret_cast<const u32x4*>(krow + 128 * (jp + 1));
      ka[jp + 1][1] = *reinterpret_cast<const u32x4*>(krow + 128 * (jp + 1) + 64);
    }
    s0 = mfma16_k32(as_bf16x8(ka[jp][0]), qreg[2 * jp], s0);
    s1 = mfma16_k32(as_bf16x8(ka[jp][1]), qreg[2 * jp + 1], s1);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s0 + s1;
}

// The softmax of one 32-key tile (keys k0 .. k0 + 31, those >= khi masked)
// from the scores of both halves (h0: keys 0 .. 15, h1: keys 16 .. 31, in
// the score layout: lane l holds head l % 16, keys 4 (l / 16) .. +3 of each
// half), then O^T += V^T P^T over NVT value tiles from column col0, on
// 16x16x32 MFMAs with the tile's 32 keys as the contraction.  The
// contraction order is a permutation of the keys: index 8 g + i is key
// 4 g + i for i < 4 and key 16 + 4 g + i - 4 otherwise, which is the order in
// which lane group g already holds its eight probabilities (the B operand)
// and in which two transposing LDS reads give the A operand (16-lane group g
// reads keys 4 g .. 4 g + 3 of 16 columns from each half; lane L receives
// column L's keys).  Every wave of a pair runs the same operations on the
// same values, so their running states stay equal.
template <bool CAP, int NVT>
__device__ __forceinline__ void mla_tile_pv(MlaState<NVT>& st, const uint8_t* kl, int k0, int khi, f32x4 h0,
                                            f32x4 h1, float c, const SoftCap& sc, int col0, int lane) {
  constexpr int VG = 4;                         // value tiles per step
  constexpr int half = 16 * MlaGeo::pitch;
  const int L = lane & 15;
  const uint8_t* vsrc = kl + (4 * (lane >> 4) + (L >> 2)) * MlaGeo::pitch + 8 * (L & 3) + 2 * col0;
  i16x4 va[NVT / VG][VG][2];
#pragma unroll
  for (int u = 0; u < VG; ++u) {
    va[0][u][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vsrc + 32 * u));
    va[0][u][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vsrc + half + 32 * u));
  }
  __builtin_amdgcn_sched_barrier(0);
  const int kb = k0 + 4 * (lane >> 4);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x0 = h0[i], x1 = h1[i];
    if constexpr (CAP) {
      x0 = cap1(x0, sc);
      x1 = cap1(x1, sc);
    }
    v[i] = kb + i < khi ? x0 : neg_inf();
    v[4 + i] = kb + 16 + i < khi ? x1 : neg_inf();
  }
  float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
  mx = fmaxf(mx, xor16(mx));
  mx = fmaxf(mx, xor32(mx));
  const float mxs = mx * c;
  if (__builtin_amdgcn_ballot_w64(mxs > st.m + kRescaleSlack)) {
    __asm__ volatile("" ::: "memory");
    const float m_new = fmaxf(st.m, mxs);
    const float alpha = __builtin_amdgcn_exp2f(st.m - (m_new == neg_inf() ? 0.f : m_new));
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < NVT; ++t) st.o[t] *= alpha;
    st.m = m_new;
  }
  const float nref = st.m == neg_inf() ? 0.f : -st.m;
  float pr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], c, nref));
  st.l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  const bf16x8 pb = pack_bf16x8(pr);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < NVT / VG; ++g) {
    if (g + 1 < NVT / VG) {
#pragma unroll
      for (int u = 0; u < VG; ++u) {
        const uint8_t* a = vsrc + 32 * (VG * (g + 1) + u);
        va[g + 1][u][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
        va[g + 1][u][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + half));
      }
    }
#pragma unroll
    for (int u = 0; u < VG; ++u)
      st.o[VG * g + u] = mfma16_k32(join_bf16x4(va[g][u][0], va[g][u][1]), pb, st.o[VG * g + u]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The key loop of a key-pair MLA item (eight waves, two per SIMD): waves w
// and w + 4 own the same 16 heads; wave w scores keys 0 .. 15 of every tile
// and wave w + 4 keys 16 .. 31, and they swap those scores through LDS, so no
// product is computed twice; then both run the same softmax over the 32 keys
// and each accumulates its half of the 512 value columns.  Software
// pipelined: after barrier A of step t, tile t + 1 has landed (tile t + 2 may
// still be in flight) and every wave's scores of tile t are in the exchange
// buffer; the key-half-1 waves issue the loads of tile t + 3 (into the
// buffer of tile t - 1, which every wave has left); each wave reads its
// partner's scores, runs the softmax and value product of tile t and scores
// its half of tile t + 1; barrier B (every partner read done) precedes the
// write of those scores.
template <bool CAP>
__device__ __forceinline__ void mla_pair_keys(const AttnParams& p, uint8_t* smem, int32_t* pcache, int b, int L,
                                              int klo, int khi, const bf16x8 (&qreg)[kMlaQSteps], float c,
                                              const SoftCap& sc, MlaState<kMlaVTilesHalf>& st, int kh, int col0,
                                              int wave, int lane) {
  constexpr int R = MlaPairLds::ring;
  static_assert(R == 4, "the waits below keep at most one more tile in flight");
  using Loads = MlaLoads<kMlaHsWaves / 2>;
  uint8_t* xbuf = smem + MlaPairLds::xbuf_off;
  const int xmine = (wave * kWave + lane) * 16;
  const int xpart = ((wave ^ 4) * kWave + lane) * 16;
  PageWalk w;
  w.pt_row = p.page_table + (int64_t)b * p.pt_row_stride;
  w.page_bytes = p.kv_page_bytes;
  w.head_off = 0;
  w.row_stride_b = MlaGeo::row_bytes;
  w.shift = p.page_shift;
  w.klimit = L;
  Loads ml;
  ml.init(wave & 3, lane);
  const bool loader = kh == 1;
  const int chunk_keys = MlaPairLds::pcache_entries << w.shift;
  for (int cb = klo; cb < khi; cb += chunk_keys) {
    const int ce = min(khi, cb + chunk_keys);
    __syncthreads();
    fill_pcache(w, pcache, cb, ce);
    wait_vmem_all();                            // Q loads and page-table reads
    __syncthreads();
    const int ntiles = (ce - cb + kSub - 1) / kSub;
    if (loader) {
#pragma unroll
      for (int t = 0; t < R - 1; ++t)
        if (t < ntiles) ml.issue(p.k_pool, w, cb + t * kSub, smem + t * MlaGeo::tile_bytes, wave & 3);
    }
    // tile 0 (tiles 1 and 2 may stay in flight)
    if (ntiles > 2)
      wait_vmem<2 * Loads::min_per_wave>();
    else if (ntiles > 1)
      wait_vmem<Loads::min_per_wave>();
    else
      wait_vmem<0>();
    ring_barrier();
    f32x4 mine = mla_half_scores(smem, kh, qreg, lane);
    *reinterpret_cast<f32x4*>(xbuf + xmine) = mine;
#pragma unroll 1
    for (int t = 0; t < ntiles; ++t) {
      if (t + 2 < ntiles)                       // tile t + 1 (tile t + 2 may stay in flight)
        wait_vmem<Loads::min_per_wave>();
      else
        wait_vmem<0>();
      ring_barrier();                           // A
      // the loads of tile t + 3 (into the buffer of tile t - 1, which every
      // wave has left), by the key-half-1 waves only: while they wait on the
      // load path, their partners on the same SIMDs run ahead
      const bool more = t + R - 1 < ntiles;
      if (loader && more)
        ml.issue(p.k_pool, w, cb + (t + R - 1) * kSub, smem + ((t + R - 1) % R) * MlaGeo::tile_bytes, wave & 3);
      const f32x4 part = *reinterpret_cast<const f32x4*>(xbuf + xpart);
      mla_tile_pv<CAP, kMlaVTilesHalf>(st, smem + (t % R) * MlaGeo::tile_bytes, cb + t * kSub, khi,
                                       kh == 0 ? mine : part, kh == 0 ? part : mine, c, sc, col0, lane);
      if (t + 1 < ntiles) {
        mine = mla_half_scores(smem + ((t + 1) % R) * MlaGeo::tile_bytes, kh, qreg, lane);
        ring_barrier();                         // B
        *reinterpret_cast<f32x4*>(xbuf + xmine) = mine;
      }
    }
  }
}

// One head-split MLA item: the keys [klo, khi) of sequence b for head group
// hg (p.group heads starting at hg * p.group), then its outputs -- final rows
// (slot < 0), a split-KV partial record (split schedule) or a balanced
// partial record in slot `slot`.  Wave w takes heads 16 (w % 4) .. +15 of the
// group, key half kh = w / 4 of every tile for the scores and value columns
// [256 kh, 256 kh + 256) for the output.
template <int NW>
__device__ void mla_hs_item(const AttnParams& p, uint8_t* smem, int32_t* pcache, int b, int hg, int L, int klo,
                            int khi, int slot, int wave, int lane) {
  static_assert(NW == kMlaHsWaves, "two waves per SIMD");
  constexpr int NVT = kMlaVTilesHalf;
  const int hl = (wave & 3) * kMlaHeads + (lane & 15);  // head within the group
  const int kh = wave >> 2;                              // key half
  const int col0 = 16 * NVT * kh;
  const int h = hg * p.group + hl;
  const bool hok = hl < p.group && h < p.num_q_heads;
  // the B operand of k-step j: head hl's query values 32 j + 8 (lane / 16) .. +7
  bf16x8 qreg[kMlaQSteps];
  {
    const uint16_t* src = p.q + (int64_t)b * p.q_stride_t + (int64_t)(hok ? h : 0) * kMlaDk + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < kMlaQSteps; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + 32 * j);
      qreg[j] = as_bf16x8(hok ? v : u32x4{0u, 0u, 0u, 0u});
    }
  }
  float c, vdesc;
  score_scales<false>(p, c, vdesc);
  const SoftCap sc(p.softcap, c);
  MlaState<NVT> st;
#pragma unroll
  for (int t = 0; t < NVT; ++t) st.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = neg_inf();
  st.l = 0.f;
  if (khi > klo) {
    if (sc.on())
      mla_pair_keys<true>(p, smem, pcache, b, L, klo, khi, qreg, c, sc, st, kh, col0, wave, lane);
    else
      mla_pair_keys<false>(p, smem, pcache, b, L, klo, khi, qreg, c, sc, st, kh, col0, wave, lane);
  }
  // the row sum: this lane's keys, then the head's four lanes
  st.l += __shfl_xor(st.l, 16);
  st.l += xor32(st.l);
  if (!hok) return;
  const bool empty = !(st.l > 0.f);
  const float inv = empty ? 0.f : vdesc / st.l;
  const float lse2 = empty ? neg_inf() : st.m + __builtin_amdgcn_logf(st.l);
  const int d_lane = col0 + 4 * (lane >> 4);
  const bool lse_lane = lane < 16 && col0 == 0;
  if (slot >= 0) {
    // balanced records hold the group's rows (p.group of them) per slot
    const int64_t row = p.balanced ? (int64_t)slot * p.group + hl
                                   : ((int64_t)slot * p.max_total_q + b) * p.num_q_heads + h;
    if (lse_lane) p.part_lse[row] = lse2;
    if (empty) return;
    float* dst = p.part_o + row * kMlaLatent + d_lane;
#pragma unroll
    for (int t = 0; t < NVT; ++t) *reinterpret_cast<f32x4*>(dst + 16 * t) = st.o[t] * inv;
  } else {
    uint16_t* dst = p.out + (int64_t)b * p.o_stride_t + (int64_t)h * kMlaLatent + d_lane;
#pragma unroll
    for (int t = 0; t < NVT; ++t)
      *reinterpret_cast<u32x2*>(dst + 16 * t) =
          u32x2{pack_bf16x2(st.o[t][0] * inv, st.o[t][1] * inv), pack_bf16x2(st.o[t][2] * inv, st.o[t][3] * inv)};
    if (p.lse && lse_lane) p.lse[(int64_t)b * p.num_q_heads + h] = lse2 * kLn2;
  }
}

// MLA decode.  Item = (sequence b, key window, head group of up to 64 query
// heads).  Each pair of waves owns 16 query heads of the group (their 576
// query values in registers, 72 VGPRs, in both waves) and splits every tile's
// keys for the scores (16x16x32 MFMAs, swapped through LDS) and the value
// columns for the output (16x16x32 MFMAs over the tile's 32 keys, P straight
// from the score registers); see mla_pair_keys.  A group of at most 48 heads
// leaves pairs without live heads, which still share the tile loads and the
// barriers (each pair has its own SIMD, so they cost the others nothing).
// More than 64 heads take several head groups; the cache is read from memory
// once per head group.
//   Split schedule: one workgroup per (b, window, group); items are ordered
//   (b, split, group) and dealt so that each XCD takes a contiguous run of
//   them, which puts the head groups of one window on one L2.
//   Balanced schedule (p.balanced): one workgroup per compute unit, each
//   taking an equal run of 128-key units over all (b, group) items laid end
//   to end (balanced_start), piece by piece; cut pieces become partial
//   records for merge_balanced_kernel.
template <int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void mla_hs_kernel(AttnParams p) {
  using LD = MlaPairLds;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LD::bytes];
  int32_t* pcache = reinterpret_cast<int32_t*>(smem + LD::pcache_off);
  int* meta = reinterpret_cast<int*>(smem + LD::pcache_off - 64);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (p.balanced) {
    const int HG = p.head_groups;
    const int w = blockIdx.x;
    int u0, u1, b, S;
    if (!balanced_start<NW * kWave>(p, smem, meta, HG, u0, u1, b, S)) return;
    int u = u0;
    int piece = 0;
    while (u < u1) {
      const int sb = seq_units(p, b);
      const int item0 = HG * S;
      if (sb == 0 || u >= item0 + HG * sb) {    // past this sequence's items
        S += sb;
        ++b;
        continue;
      }
      const int hg = (u - item0) / sb;
      const int a0 = item0 + hg * sb;
      const int a1 = a0 + sb;
      const int pu1 = min(u1, a1);
      const int L = min(p.seq_lens[b], p.pt_cols << p.page_shift);
      const int klo = (u - a0) << kUnitShift;
      const int khi = min(L, (pu1 - a0) << kUnitShift);
      const int slot = (u == a0 && pu1 == a1) ? -1 : 2 * w + (piece == 0 ? 0 : 1);
      mla_hs_item<NW>(p, smem, pcache, b, hg, L, klo, khi, slot, wave, lane);
      __syncthreads();                          // LDS is reused by the next piece
      u = pu1;
      ++piece;
    }
    return;
  }
  int hg, b, split;
  {
    const int n = gridDim.x;
    const int lin = blockIdx.x;
    const int full = n - n % kXcds;
    const int logical = lin < full ? (lin % kXcds) * (full / kXcds) + lin / kXcds : lin;
    hg = logical % p.head_groups;
    const int rest = logical / p.head_groups;
    split = rest % p.num_splits;
    b = rest / p.num_splits;
  }
  const int L = min(p.seq_lens[b], p.pt_cols << p.page_shift);
  const int klo = split * p.split_keys;
  // the last window takes every remaining key
  const int khi = split == p.num_splits - 1 ? L : min(L, klo + p.split_keys);
  mla_hs_item<NW>(p, smem, pcache, b, hg, L, klo, khi, p.num_splits > 1 ? split : -1, wave, lane);
}

// ---------------------------------------------------------------------------
// split-KV merge: LSE = log sum exp(LSE_s), O = sum exp(LSE_s - LSE) O_s
// ---------------------------------------------------------------------------

// Running log-sum-exp combination of partial records (exp2 domain), taken
// CH records at a time so that their loads are issued together: a merge row
// costs one memory round trip per CH records instead of one for the maxima and
// one per record.  A record whose LSE is -inf (an empty window) is skipped by
// selects, since its O slots were never written.  With all records in one
// chunk the arithmetic is the plain two-pass combination, in record order.
template <int PER, int CH>
struct MergeRow {
  float acc[PER];
  float wsum = 0.f, mx = neg_inf();

  __device__ __forceinline__ MergeRow() {
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  }

  __device__ __forceinline__ void add(const float (&ls)[CH], const float (&v)[CH][PER]) {
    float cm = mx;
#pragma unroll
    for (int u = 0; u < CH; ++u) cm = fmaxf(cm, ls[u]);
    if (cm == neg_inf()) return;
    if (cm != mx) {               // the first visible record sets mx; later growth rescales
      const float a = __builtin_amdgcn_exp2f(mx - cm);
      wsum *= a;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] *= a;
      mx = cm;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const bool live = ls[u] != neg_inf();
      const float w = live ? __builtin_amdgcn_exp2f(ls[u] - mx) : 0.f;
      wsum += w;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = live ? acc[k] + w * v[u][k] : acc[k];
    }
  }

  // bf16 O (lane's PER values) and natural-log LSE
  __device__ __forceinline__ void store(uint16_t* dst, float* lse_dst) const {
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const __bf16 v = (__bf16)(acc[k] * inv);
      dst[k] = __builtin_bit_cast(uint16_t, v);
    }
    if (lse_dst) *lse_dst = mx == neg_inf() ? neg_inf() : (mx + __builtin_amdgcn_logf(wsum)) * kLn2;
  }
};

constexpr int kMergeChunk = 4;        // partial records loaded together per merge row

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // t * Hq + h
  const int total_t = p.cu_q_lens ? p.cu_q_lens[p.num_seqs] : p.num_seqs;
  const int64_t nrows = (int64_t)min(total_t, p.max_total_q) * p.num_q_heads;
  if (row >= nrows) return;
  const int t = (int)(row / p.num_q_heads);
  const int h = (int)(row - (int64_t)t * p.num_q_heads);
  const int64_t plane = (int64_t)p.max_total_q * p.num_q_heads;
  constexpr int PER = D / 64;     // d values per lane
  constexpr int CH = kMergeChunk;
  MergeRow<PER, CH> m;
  for (int s0 = 0; s0 < p.num_splits; s0 += CH) {
    float ls[CH], v[CH][PER];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int s = min(s0 + u, p.num_splits - 1);     // past the last split: re-read it, unused
      ls[u] = s0 + u < p.num_splits ? p.part_lse[s * plane + row] : neg_inf();
      const float* src = p.part_o + (s * plane + row) * D + lane * PER;
#pragma unroll
      for (int k = 0; k < PER; ++k) v[u][k] = src[k];
    }
    m.add(ls, v);
  }
  m.store(p.out + (int64_t)t * p.o_stride_t + (int64_t)h * D + lane * PER,
          p.lse && lane == 0 ? p.lse + row : nullptr);
}

// Rows of balanced decode whose item was cut between workgroups: combine the
// pieces' partial records (slot rule of balanced_decode); rows of sequences
// without keys get O = 0 and LSE = -inf; whole items were written already.
template <int D>
__global__ __launch_bounds__(256) void merge_balanced_kernel(BalancedMergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // b * Hq + h
  if (row >= (int64_t)p.num_seqs * p.num_q_heads) return;
  const int b = (int)(row / p.num_q_heads);
  const int h = (int)(row - (int64_t)b * p.num_q_heads);
  const int qn = p.cu_q_lens ? p.cu_q_lens[b + 1] - p.cu_q_lens[b] : 1;
  if (qn <= 0) return;
  const int t = p.cu_q_lens ? p.cu_q_lens[b] : b;
  if (t >= p.max_total_q) return;
  const int G = p.rows_per_item;
  const int g = h / G, r = h - g * G;
  const int U = p.sched[0];
  const int S = p.sched[4 + b];
  const int sb = p.sched[4 + b + 1] - S;
  constexpr int PER = D / 64;     // d values per lane
  constexpr int CH = kMergeChunk;
  uint16_t* dst = p.out + (int64_t)t * p.o_stride_t + (int64_t)h * D + lane * PER;
  if (sb == 0) {                  // no visible key
#pragma unroll
    for (int k = 0; k < PER; ++k) dst[k] = 0;
    if (p.lse && lane == 0) p.lse[(int64_t)t * p.num_q_heads + h] = neg_inf();
    return;
  }
  const int a0 = p.num_kv_heads * S + g * sb;
  const int w0 = a0 / U, w1 = (a0 + sb - 1) / U;
  if (w0 == w1) return;
  MergeRow<PER, CH> m;
  for (int c0 = w0; c0 <= w1; c0 += CH) {
    float ls[CH], v[CH][PER];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int wg = min(c0 + u, w1);                  // past the last piece: re-read it, unused
      const int64_t rec = (int64_t)(2 * wg + ((wg == w0 && a0 != w0 * U) ? 1 : 0)) * G + r;
      ls[u] = c0 + u <= w1 ? p.part_lse[rec] : neg_inf();
      const float* src = p.part_o + rec * D + lane * PER;
#pragma unroll
      for (int k = 0; k < PER; ++k) v[u][k] = src[k];
    }
    m.add(ls, v);
  }
  m.store(dst, p.lse && lane == 0 ? p.lse + (int64_t)t * p.num_q_heads + h : nullptr);
}

// ---------------------------------------------------------------------------
// KV-cache append: a workgroup per 16 new tokens, a thread per 8 elements
// ---------------------------------------------------------------------------

constexpr int kAppendTokens = 16;     // new tokens per workgroup, at most
__host__ __device__ inline int append_tokens_per_block(bool fp8) { return fp8 ? 4 : kAppendTokens; }
constexpr int kAppendBatch = 4;       // 16-byte groups a thread loads before it stores

// Division by a per-tensor descale d: q = x / d, correctly rounded.  For d in
// [2^-60, 2^60] (a wave-uniform test) the quotient of an x clamped to
// +-449 d comes from the exact reciprocal y = 1/d and one FMA correction:
// q0 = x y, r = x - q0 d (exact, one FMA), q = q0 + r y.  With y the
// correctly rounded reciprocal and no underflow in r this is the correctly
// rounded quotient (the FMA-based division correction of Markstein); a
// host check over every bf16 value against thousands of descales of that
// range finds every quotient of magnitude 2^-10 .. 448 equal to IEEE
// division and every E4M3 code equal.  Smaller quotients encode to zero either way (their
// sign is kept from q0), larger ones saturate, and the clamp keeps q0 finite.
// Outside that range of d the kernel divides.
struct DescaleDiv {
  float d, y, m;
  bool fast;
  __device__ explicit DescaleDiv(float d_) : d(d_), y(1.f / d_), m(449.f * d_),
                                            fast(d_ >= 0x1p-60f && d_ <= 0x1p60f) {}
  __device__ __forceinline__ float operator()(float x) const {
    if (!fast) return x / d;
    const float xc = __builtin_amdgcn_fmed3f(x, -m, m);
    const float q0 = xc * y;
    const float r = __builtin_fmaf(-q0, d, xc);
    return __builtin_copysignf(__builtin_fmaf(r, y, q0), q0);
  }
};

// 8 bf16 values (one 16-byte group) -> 8 OCP E4M3 codes of the binary32
// quotients value / d (correctly rounded, DescaleDiv); finite ones are
// clamped to +-448 (saturation, infinities included) and the hardware
// conversion rounds to nearest even.  The conversion gives every NaN the
// code 0xFF, so NaN codes are rewritten as 0x7F with the value's sign (a
// branch no lane takes unless its group holds a NaN).
__device__ __forceinline__ u32x2 e4m3_encode8(u32x4 v, const DescaleDiv& div) {
  float q[8];
  bool any_nan = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = (v[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
    const float x = __builtin_bit_cast(float, h << 16);
    const bool nan = (h & 0x7FFFu) > 0x7F80u;
    any_nan |= nan;
    q[i] = nan ? x : __builtin_amdgcn_fmed3f(div(x), 448.0f, -448.0f);
  }
  u32x2 out;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * j], q[4 * j + 1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * j + 2], q[4 * j + 3], w, true);
    out[j] = (uint32_t)w;
  }
  if (any_nan) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = __builtin_bit_cast(uint32_t, q[i]);
      if ((b & 0x7FFFFFFFu) > 0x7F800000u) {
        const uint32_t sh = (i & 3) * 8;
        out[i >> 2] = (out[i >> 2] & ~(0xFFu << sh)) | ((0x7Fu | ((b >> 24) & 0x80u)) << sh);
      }
    }
  }
  return out;
}

// One workgroup appends `tpb` (<= kAppendTokens) consecutive new tokens: 16
// for bf16 pools, 4 for fp8 pools, whose division and encoding keep the VALU
// busy enough that more resident waves are needed to cover the loads.  The first
// threads resolve each token's sequence (binary search over cu_new), position
// and page once and publish the row's byte offset in the pools through LDS;
// then every thread moves 16-byte groups of the tokens' K and V rows, issuing
// kAppendBatch loads before their stores so the loads overlap.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ int64_t row_off[kAppendTokens];     // byte offset of the row in a pool, -1 = skip
  const int total = min(p.cu_new[p.num_seqs], p.max_new);
  const int tpb = append_tokens_per_block(p.fp8);
  const int t0 = blockIdx.x * tpb;
  if (t0 >= total) return;
  const int esz = p.fp8 ? 1 : 2;
  if ((int)threadIdx.x < tpb) {
    const int t = t0 + (int)threadIdx.x;
    int64_t off = -1;
    if (t < total) {
      int lo = 0, hi = p.num_seqs - 1;             // last b with cu_new[b] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu_new[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      const int n = p.cu_new[lo + 1] - p.cu_new[lo];
      const int pos = p.seq_lens[lo] - n + (t - p.cu_new[lo]);
      if (pos >= 0 && pos < (p.pt_cols << p.page_shift)) {
        const int page = p.page_table[(int64_t)lo * p.pt_row_stride + (pos >> p.page_shift)];
        const int slot = pos & ((1 << p.page_shift) - 1);
        // a page id outside the pool is a contract violation: the row is skipped
        if (page >= 0 && page < p.num_pages)
          off = (int64_t)page * p.kv_page_bytes + (int64_t)slot * p.num_kv_heads * p.head_dim * esz;
      }
    }
    row_off[threadIdx.x] = off;
  }
  __syncthreads();
  const int per_kv = p.num_kv_heads * (p.head_dim / 8);      // 16-byte groups per K (or V) row
  const int per_token = 2 * per_kv;
  const int groups = min(tpb, total - t0) * per_token;
  const DescaleDiv kd(p.fp8 ? *p.k_descale : 1.f);
  const DescaleDiv vd(p.fp8 ? *p.v_descale : 1.f);
  for (int base = threadIdx.x; base < groups; base += kAppendBatch * 256) {
    u32x4 v[kAppendBatch];
    int64_t dst[kAppendBatch];
    bool is_v[kAppendBatch];
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {
      // every lane loads (a group past the end re-reads group 0, always valid)
      // so that no load sits in a branch and all kAppendBatch stay in flight
      const int e = base + u * 256;
      const int ec = e < groups ? e : 0;
      const int i = ec / per_token;
      int r = ec - i * per_token;
      is_v[u] = r >= per_kv;
      r -= is_v[u] ? per_kv : 0;                   // group r of the row: element 8 r
      const int64_t off = row_off[i];
      const uint16_t* src = (is_v[u] ? p.v_new : p.k_new) + (int64_t)(t0 + i) * p.new_stride_t + r * 8;
      v[u] = *reinterpret_cast<const u32x4*>(src);
      dst[u] = (e < groups && off >= 0) ? off + (int64_t)r * 8 * esz : -1;
    }
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {
      if (dst[u] < 0) continue;
      uint8_t* pool = (is_v[u] ? p.v_pool : p.k_pool) + dst[u];
      if (!p.fp8) *reinterpret_cast<u32x4*>(pool) = v[u];
      else *reinterpret_cast<u32x2*>(pool) = e4m3_encode8(v[u], is_v[u] ? vd : kd);
    }
  }
}

template <int D, bool FP8, int MODE>
hipError_t launch_one(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if constexpr (FP8 && MODE == kPrefill && Block<MODE, D>::stream) {
    if (p.q_fp8) {
      hipLaunchKernelGGL((attn_kernel<D, FP8, MODE, true>), grid, dim3(Block<MODE, D, true>::threads), 0, stream, p);
      return hipGetLastError();
    }
  }
  if (p.q_fp8) return hipErrorInvalidValue;
  if constexpr (MODE == kMixed) {
    if (p.queue) {
      hipLaunchKernelGGL((attn_kernel<D, FP8, MODE, false, true>), grid, dim3(Block<MODE, D>::threads), 0, stream, p);
      return hipGetLastError();
    }
  }
  if (p.queue) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_kernel<D, FP8, MODE>), grid, dim3(Shape<D, FP8, MODE>::threads), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_mode(Mode mode, const AttnParams& p, dim3 grid, hipStream_t stream) {
  switch (mode) {
    case kDecode: return launch_one<D, FP8, kDecode>(p, grid, stream);
    case kPrefill: return launch_one<D, FP8, kPrefill>(p, grid, stream);
    case kMixed: return launch_one<D, FP8, kMixed>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool FP8>
int lds_mode(Mode mode) {
  switch (mode) {
    case kDecode: return Lds<D, FP8, kDecode>::bytes;
    case kPrefill: return Lds<D, FP8, kPrefill>::bytes;
    case kMixed: return Lds<D, FP8, kMixed>::bytes;
  }
  return 0;
}

}  // namespace

hipError_t launch_attention(int head_dim, bool kv_fp8, Mode mode, const AttnParams& p, dim3 grid,
                            hipStream_t stream) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  switch (head_dim) {
    case 64: return kv_fp8 ? launch_mode<64, true>(mode, p, grid, stream) : launch_mode<64, false>(mode, p, grid, stream);
    case 128: return kv_fp8 ? launch_mode<128, true>(mode, p, grid, stream) : launch_mode<128, false>(mode, p, grid, stream);
    case 256: return kv_fp8 ? launch_mode<256, true>(mode, p, grid, stream) : launch_mode<256, false>(mode, p, grid, stream);
  }
  return hipErrorInvalidValue;
}

template <int D, bool FP8, int MODE>
constexpr int wgs_per_cu() {
  constexpr int by_lds = kLdsMax / Lds<D, FP8, MODE>::bytes;
  constexpr int by_waves = Shape<D, FP8, MODE>::waves_per_eu * 4 / Shape<D, FP8, MODE>::waves;   // 4 SIMDs per CU
  constexpr int n = by_lds < by_waves ? by_lds : by_waves;
  return n > 0 ? n : 1;
}

template <int D, bool FP8>
int wgs_mode(Mode mode) {
  switch (mode) {
    case kDecode: return wgs_per_cu<D, FP8, kDecode>();
    case kPrefill: return wgs_per_cu<D, FP8, kPrefill>();
    case kMixed: return wgs_per_cu<D, FP8, kMixed>();
  }
  return 1;
}

int workgroups_per_cu(int head_dim, bool kv_fp8, Mode mode) {
  switch (head_dim) {
    case 64: return kv_fp8 ? wgs_mode<64, true>(mode) : wgs_mode<64, false>(mode);
    case 128: return kv_fp8 ? wgs_mode<128, true>(mode) : wgs_mode<128, false>(mode);
    case 256: return kv_fp8 ? wgs_mode<256, true>(mode) : wgs_mode<256, false>(mode);
  }
  return 1;
}

int attention_lds_bytes(int head_dim, bool kv_fp8, Mode mode) {
  switch (head_dim) {
    case 64: return kv_fp8 ? lds_mode<64, true>(mode) : lds_mode<64, false>(mode);
    case 128: return kv_fp8 ? lds_mode<128, true>(mode) : lds_mode<128, false>(mode);
    case 256: return kv_fp8 ? lds_mode<256, true>(mode) : lds_mode<256, false>(mode);
  }
  return 0;
}

template <int D>
int block_rows_d(Mode mode, bool q_fp8) {
  switch (mode) {
    case kDecode: return Block<kDecode, D>::waves * Block<kDecode, D>::nct * kCols;
    case kPrefill:
      return q_fp8 ? Block<kPrefill, D, true>::waves * kCols : Block<kPrefill, D>::waves * Block<kPrefill, D>::nct * kCols;
    case kMixed: return Block<kMixed, D>::waves * Block<kMixed, D>::nct * kCols;
  }
  return 0;
}

int block_rows(int head_dim, Mode mode, bool q_fp8) {
  switch (head_dim) {
    case 64: return block_rows_d<64>(mode, q_fp8);
    case 128: return block_rows_d<128>(mode, q_fp8);
    case 256: return block_rows_d<256>(mode, q_fp8);
  }
  return 0;
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  if (p.max_new <= 0 || p.num_seqs <= 0) return hipSuccess;
  const int tpb = append_tokens_per_block(p.fp8);
  const dim3 grid((unsigned)((p.max_new + tpb - 1) / tpb));
  hipLaunchKernelGGL(append_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_mla(const AttnParams& p, dim3 grid, hipStream_t stream) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (p.num_q_heads > 128 || p.group > 64 || p.group < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_hs_kernel<kMlaHsWaves>, grid, dim3(kMlaHsWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge_balanced(int head_dim, const BalancedMergeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (grid.x == 0) return hipSuccess;
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(merge_balanced_kernel<64>, grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(merge_balanced_kernel<128>, grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL(merge_balanced_kernel<256>, grid, dim3(256), 0, stream, p); break;
    case 512: hipLaunchKernelGGL(merge_balanced_kernel<512>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Metadata check (pa_check_metadata): one thread per sequence; page ids
// are read as values only.  The mask is cleared by a one-thread launch
// before the check launch ORs into it.
__global__ void check_clear_kernel(int32_t* flags) { *flags = 0; }

__global__ __launch_bounds__(256) void check_kernel(CheckParams q) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= q.num_seqs) return;
  int bits = 0;
  const int L = q.seq_lens[b];
  const int64_t cap = (int64_t)q.pt_cols << q.page_shift;
  if (L < 0 || L > cap) bits |= 4;
  int qn = 1;
  if (q.cu_q_lens) {
    const int c0 = q.cu_q_lens[b], c1 = q.cu_q_lens[b + 1];
    qn = c1 - c0;
    if (qn < 0 || (b == 0 && c0 != 0) || (b == q.num_seqs - 1 && c1 > q.max_total_q)) bits |= 8;
  }
  if (L > 0 && qn > L) bits |= 2;
  const int64_t live = L > 0 ? min((int64_t)L, cap) : 0;
  const int np = (int)((live + (1 << q.page_shift) - 1) >> q.page_shift);
  const int32_t* row = q.page_table + (int64_t)b * q.pt_row_stride;
  for (int c = 0; c < np; ++c) {
    const int id = row[c];
    if (id < 0 || id >= q.num_pages) {
      bits |= 1;
      break;
    }
  }
  if (bits) atomicOr(q.flags, bits);
}

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, stream, p.flags);
  if (p.num_seqs > 0) hipLaunchKernelGGL(check_kernel, dim3((unsigned)((p.num_seqs + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_queue_setup(const QueueSetupParams& p, hipStream_t stream) {
  if (p.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(queue_setup_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge(int head_dim, const MergeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.max_total_q * p.num_q_heads;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (grid.x == 0) return hipSuccess;
  switch (head_dim) {
    case 64: hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(256), 0, stream, p); break;
    case 512: hipLaunchKernelGGL(merge_kernel<512>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
