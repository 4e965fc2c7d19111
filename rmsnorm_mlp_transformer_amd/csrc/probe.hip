// MFMA issue-rate probe: the matrix instructions of the GEMMs' main loops
// with nothing else around them, to measure what the chip sustains on them
// (its clock under that load) apart from any GEMM's feeding. A measurement
// aid, not an operation of the method.
#include <hip/hip_runtime.h>

#include "probe.hpp"
#include "te_common.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

// Each wave runs four independent accumulation chains of `iters` MFMAs on
// fixed pseudo-random operands (a hash of the lane: operand bits move the
// power draw, and with it the clock), then stores one float per thread so the
// loop is not removed. Workgroup 0's first thread records the shader-clock
// and reference-clock ticks of its loop.
template <bool FP8>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int64_t iters, float* sink, uint64_t* ticks) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  auto hash = [](uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
  };
  f32x16_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  uint64_t t0 = 0, r0 = 0;
  if constexpr (FP8) {
    // E4M3 codes with the exponent field below 15 (no NaN), either sign
    i32x8_t a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = (int)(hash(id * 16u + k) & 0xF7F7F7F7u);
      b[k] = (int)(hash(id * 16u + 8u + k) & 0xF7F7F7F7u);
    }
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[c], 0, 0, 0, 0, 0, 0);
    }
  } else {
    // bf16 values of magnitude in [0.5, 2), either sign
    bf16x8_t a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t ha = hash(id * 16u + k), hb = hash(id * 16u + 8u + k);
      a[k] = __builtin_bit_cast(__bf16, (uint16_t)((ha & 0x807Fu) | 0x3F00u | ((ha >> 8) & 0x80u)));
      b[k] = __builtin_bit_cast(__bf16, (uint16_t)((hb & 0x807Fu) | 0x3F00u | ((hb >> 8) & 0x80u)));
    }
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[c], 0, 0, 0);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float v = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) v += acc[c][r];
  sink[id] = v;
  if (blockIdx.x == 0 && threadIdx.x == 0 && ticks != nullptr) {
    ticks[0] = t1 - t0;
    ticks[1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_probe(bool fp8, int64_t iters, int blocks, float* sink, uint64_t* ticks, hipStream_t s) {
  LaunchScope scope(fp8 ? "mfma_probe_fp8" : "mfma_probe_bf16", s);
  if (fp8) launch_kernel(mfma_probe_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, iters, sink, ticks);
  else launch_kernel(mfma_probe_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, iters, sink, ticks);
  return hipGetLastError();
}

}  // namespace te
