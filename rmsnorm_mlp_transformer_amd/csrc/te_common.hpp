// Device helpers shared by the gfx950 kernels: element conversions, the
// E4M3 encoder, the activation functions and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "te_kernels.hpp"

namespace te {

// ---------------------------------------------------------------- vector types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

// Streaming loads carry the non-temporal hint (the nt bit of gfx950 loads):
// data that one pass reads once is not kept in the caches ahead of lines
// other work reuses, and measured streaming kernels move 10-15% more bytes
// per second from HBM with it. TE_NT_LOADS=0 turns the hint off.
#ifndef TE_NT_LOADS
#define TE_NT_LOADS 1
#endif
constexpr int kBufAuxStream = TE_NT_LOADS ? 2 : 0;   // cache-policy operand of buffer loads: nt
__device__ __forceinline__ uint4 load_stream16(const void* p) {
#if TE_NT_LOADS
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round-to-nearest-even fp32 -> bf16 (gfx950 has a hardware convert for this).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
// Two values in one v_cvt_pk_bf16_f32 (round to nearest even), lo in bits 15:0.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

// OCP E4M3 encoding (the format's definition: saturate to +-448, then round
// to nearest even on the E4M3 grid, subnormals on the grid k * 2^-9): a med3
// clamp followed by gfx950's fp32 -> fp8 pair conversion, which rounds to
// nearest even on that grid. A probe of this build compared the pair with an
// integer implementation of the definition on every finite bf16 value, 4M
// random fp32 values over 2^-30..2^13 and the neighbours of every E4M3
// midpoint: no difference. A NaN input encodes as NaN (0x7F / 0xFF).
__device__ __forceinline__ float e4m3_clamp(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }
// codes of a, b in bits 7:0 and 15:8
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false) & 0xFFFFu;
}
// codes of a, b, c, d in bytes 0..3
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? (float)m * 0.001953125f
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// Current scaling from a (non-negative) amax: scale = 448 / amax, or 1.
__device__ __forceinline__ float fp8_scale_from_amax(float amax) {
  return amax > 0.0f ? 448.0f / amax : 1.0f;
}

// ---------------------------------------------------------------- activations
constexpr float kGeluK0 = 0.7978845608028654f;   // sqrt(2/pi)
constexpr float kGeluK1 = 0.044715f;
constexpr float kInvSqrt2 = 0.70710678118654752f;
// -2 K0 log2(e) and -2 K0 K1 log2(e): the exponent of the sigmoid form of GELU
constexpr float kGeluE0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
constexpr float kGeluE1 = -2.0f * 0.7978845608028654f * 0.044715f * 1.4426950408889634f;
constexpr float kInvSqrt2Pi = 0.39894228040143268f;
// 2 K0 and 6 K0 K1: the factor 2 u'(x) = 2 K0 (1 + 3 K1 x^2) of the GELU derivative
constexpr float kGeluD0 = 2.0f * 0.7978845608028654f;
constexpr float kGeluD1 = 6.0f * 0.7978845608028654f * 0.044715f;

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// GELU (tanh form) and its derivative from one sigmoid: with s = sigmoid(2u),
// u = K0 (x + K1 x^3), gelu = x s and
// gelu' = s + x s (1 - s) 2u' = s (1 + (x - x s) (2 K0 + 6 K0 K1 x^2)).
// Past |x| = 20 s is exactly 0 or 1 in fp32; the clamp (med3) keeps x^2
// finite (no 0 * inf), and the unclamped x still carries a NaN through.
__device__ __forceinline__ void gelu_fwd_bwd(float x, float& f, float& d) {
  const float xc = __builtin_amdgcn_fmed3f(x, -20.0f, 20.0f);
  const float x2 = xc * xc;
  const float s = fast_rcp(1.0f + __builtin_amdgcn_exp2f(xc * fmaf(kGeluE1, x2, kGeluE0)));
  f = x * s;
  d = s * fmaf(fmaf(-x, s, x), fmaf(kGeluD1, x2, kGeluD0), 1.0f);
}

template <int A>
__device__ __forceinline__ float act_fwd(float x) {
  if constexpr (A == kRelu) {
    return x > 0.0f ? x : 0.0f;
  } else if constexpr (A == kGelu) {
    // 0.5 x (1 + tanh(u)) = x * sigmoid(2u) = x / (1 + 2^(-2u log2 e)),
    // u = K0 (x + K1 x^3): one exp2 and one reciprocal
    const float t = x * fmaf(kGeluE1, x * x, kGeluE0);
    return x * fast_rcp(1.0f + __builtin_amdgcn_exp2f(t));
  } else if constexpr (A == kGeluErf) {
    return 0.5f * x * (1.0f + erff(x * kInvSqrt2));
  } else if constexpr (A == kSilu) {
    return x * fast_rcp(1.0f + __expf(-x));
  } else {
    return x;
  }
}

template <int A>
__device__ __forceinline__ float act_bwd(float x) {
  if constexpr (A == kRelu) {
    return x > 0.0f ? 1.0f : 0.0f;
  } else if constexpr (A == kGelu) {
    float f, d;
    gelu_fwd_bwd(x, f, d);
    return d;
  } else if constexpr (A == kGeluErf) {
    return 0.5f * (1.0f + erff(x * kInvSqrt2)) + x * __expf(-0.5f * x * x) * kInvSqrt2Pi;
  } else if constexpr (A == kSilu) {
    const float s = fast_rcp(1.0f + __expf(-x));
    return s * (1.0f + x * (1.0f - s));
  } else {
    return 1.0f;
  }
}

// Both the activation and its derivative at x (the gated backward needs the
// two), sharing the exponential where the forms allow.
template <int A>
__device__ __forceinline__ void act_fwd_bwd(float x, float& f, float& d) {
  if constexpr (A == kGelu) {
    gelu_fwd_bwd(x, f, d);
  } else if constexpr (A == kSilu) {
    const float s = fast_rcp(1.0f + __expf(-x));
    f = x * s;
    d = s * (1.0f + x * (1.0f - s));
  } else {
    f = act_fwd<A>(x);
    d = act_bwd<A>(x);
  }
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// amax accumulator: non-negative floats order like their bit patterns.
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// Workgroup-wide max of a non-negative value followed by a single atomic:
// thousands of waves hitting one address serialise in the L2, so each
// workgroup contributes one atomic. Must be reached by every thread of the
// workgroup (it synchronises); red must hold one float per wave.
// Most workgroups an amax pass launches: each adds one atomic on the same
// address at its end, and those serialise in the L2 at the kernel's tail. A
// sweep (256-2048) at the bench shapes put the norm amax pass best at 512
// and the plain amax (8 loads in flight per lane) at 256.
#ifndef TE_AMAX_BLOCKS
#define TE_AMAX_BLOCKS 512
#endif
constexpr unsigned kAmaxBlocks = TE_AMAX_BLOCKS;

__device__ __forceinline__ void block_max_atomic(float v, float* amax, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int i = 1; i < nw; ++i) m = fmaxf(m, red[i]);
    atomic_max_nonneg(amax, m);
  }
}

// Workgroup max of v (v >= 0) written to *out by thread 0: one partial per
// workgroup, reduced by a later launch (no atomics, no zeroed slot needed).
__device__ __forceinline__ void block_max_store(float v, float* out, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int i = 1; i < nw; ++i) m = fmaxf(m, red[i]);
    *out = m;
  }
}

}  // namespace te
