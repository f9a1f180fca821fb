// pa_calib.hip -- measurement kernel: the dense bf16 (or E4M3) MFMA rate one
// MI355X sustains on random operands.
//
// The published dense bf16 peak (256 CUs x 4 SIMDs x 2.4 GHz x 1024 flop per
// SIMD clock) assumes every SIMD retires one v_mfma_f32_32x32x16_bf16 every
// 32 clocks at the full clock.  Under a long matrix-core load the chip lowers
// its clock, and how far depends on how much the operand bits toggle.  This
// kernel does nothing but MFMAs on caller-supplied (random) operands, so its
// rate is the practical ceiling against which an attention kernel's MFMA use
// can be read.  It is not part of the attention path.
#include <type_traits>

#include "pa_internal.h"

namespace {

typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef float f32x16c __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));
typedef int i32x8c __attribute__((ext_vector_type(8)));

constexpr int kWavesPerGroup = 4;
constexpr int kOps = 8;          // distinct A and B operands per lane
// Independent accumulators per wave: a bf16 32x32x16 product needs eight
// chains in flight to issue back to back (with four, a kernel of nothing but
// these products reaches 0.6 of the rate eight give); the E4M3 32x32x64
// product, twice as long, needs four.
template <bool F8>
struct Chains { static constexpr int value = F8 ? 4 : 8; };

// Each wave: 8 A and 8 B operands (16 bytes per lane each for bf16, 32 for
// E4M3) from `ops`, eight (bf16) or four (E4M3) accumulator chains; one loop
// iteration issues 64
// MFMAs, pairing A operand j with B operand (j + r) mod 8 in round r, so
// consecutive MFMAs never see the same pair of inputs.  The accumulators are
// summed into `sink` so that no MFMA is dead.
template <bool F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mfma_rate_kernel(
    const uint16_t* __restrict__ ops, float* __restrict__ sink, int iters) {
  using Op = typename std::conditional<F8, i32x8c, bf16x8c>::type;
  constexpr int kChains = Chains<F8>::value;
  constexpr int W = F8 ? 2 : 1;                // 16-byte words per operand and lane
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const u32x4c* src = reinterpret_cast<const u32x4c*>(ops) + (int64_t)gw * 2 * kOps * 64 * W + lane;
  Op a[kOps], b[kOps];
#pragma unroll
  for (int j = 0; j < kOps; ++j) {
    if constexpr (F8) {
      const u32x4c a0 = src[64 * j], a1 = src[64 * (kOps + j)];
      const u32x4c b0 = src[64 * (2 * kOps + j)], b1 = src[64 * (3 * kOps + j)];
      a[j] = i32x8c{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      b[j] = i32x8c{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    } else {
      a[j] = __builtin_bit_cast(bf16x8c, src[64 * j]);
      b[j] = __builtin_bit_cast(bf16x8c, src[64 * (kOps + j)]);
    }
  }
  f32x16c acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kOps; ++r)
#pragma unroll
      for (int j = 0; j < kOps; ++j) {
        if constexpr (F8)
          acc[j % kChains] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[(j + r) % kOps],
                                                                             acc[j % kChains], 0, 0, 0, 0, 0, 0);
        else
          acc[j % kChains] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + r) % kOps], acc[j % kChains], 0, 0, 0);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  sink[(int64_t)gw * 64 + lane] = s;
}

}  // namespace

extern "C" pa_status pa_calibrate_mfma(const uint16_t* operands, int64_t operand_words, float* sink,
                                       int64_t sink_floats, int32_t num_workgroups, int32_t iters, int32_t fp8,
                                       hipStream_t stream) {
  if (!operands || !sink || num_workgroups <= 0 || iters <= 0 || (fp8 != 0 && fp8 != 1)) return PA_ERR_INVALID;
  // every wave reads 2 * 8 operands of 64 lanes x 16 (bf16) or 32 (E4M3) bytes
  // and writes 64 floats
  if (operand_words < (int64_t)num_workgroups * (fp8 ? 65536 : 32768) ||
      sink_floats < (int64_t)num_workgroups * 64 * kWavesPerGroup)
    return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(operands) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3) != 0)
    return PA_ERR_INVALID;
  if (fp8)
    hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3(num_workgroups), dim3(64 * kWavesPerGroup), 0, stream, operands,
                       sink, iters);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3(num_workgroups), dim3(64 * kWavesPerGroup), 0, stream, operands,
                       sink, iters);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" double pa_calibrate_mfma_flops(int32_t num_workgroups, int32_t iters, int32_t fp8) {
  return (double)num_workgroups * kWavesPerGroup * iters * kOps * kOps * (2.0 * 32 * 32 * (fp8 ? 64 : 16));
}
