// Row-wise LayerNorm / RMSNorm forward for gfx950.
//
// One 64-lane wavefront owns one row at a time: the row is read once into
// registers with 16-byte loads (each load instruction of the wave covers
// 1 KiB of the row), the mean and the centred sum of squares are reduced
// across the wave in fp32, and the normalised row is written straight out in
// the layout and precision the following GEMM reads as its A operand (fp32,
// bf16 or E4M3), so no separate normalised tensor is produced. The grid is
// capped and each wave walks several rows with the next row's loads in
// flight while the current one is reduced; gamma and beta sit in LDS, read
// once per workgroup. Rows wider than the register budget fall back to a
// loop that re-reads the row from cache.
//
// Definitions ("NVIDIA TransformerEngine JAX LayerNorm MLP", Description step
// (1); "... LayerNorm Dense", Inputs: gamma, beta, norm_type,
// zero_centered_gamma, epsilon): LayerNorm y = (x - mean) / sqrt(var + eps)
// * g + beta with the biased variance; RMSNorm y = x / sqrt(mean(x^2) + eps)
// * g; g = 1 + gamma for a zero-centred gamma.
#include <type_traits>

#include "gemm_lds.hpp"
#include "te_common.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

// Workgroups of the norm forward's store and quantise passes (4 waves each;
// 768 = three per CU, the occupancy of the 8-chunk row at ~140 VGPRs, was the
// fastest of 512 / 768 / 1024 at 8192 x 4096).
#ifndef TE_NORM_BLOCKS
#define TE_NORM_BLOCKS 768
#endif
constexpr int kNormBlocks = TE_NORM_BLOCKS;
// Workgroups of the amax pass, each writing one partial maximum that the
// quantise pass reduces (no atomics). 512 / 1024 / 2048 measured 16.5 /
// 16.9 / 25 us for the pass at 8192 x 4096, and reading more partials costs
// the quantise pass about as much again.
#ifndef TE_NORM_AMAX_BLOCKS
#define TE_NORM_AMAX_BLOCKS 512
#endif
constexpr int kNormAmaxBlocks = TE_NORM_AMAX_BLOCKS;

template <bool BF16>
struct Io {
  static constexpr int VEC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  static __device__ __forceinline__ void unpack(const uint4& c, float* f) {
    if constexpr (BF16) {
      f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x); f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
      f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z); f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
    } else {
      f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
      f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
    }
  }
};

// The normalised value; the same operation sequence in every mode, so the
// amax pass and the quantise pass see bit-identical values.
__device__ __forceinline__ float norm_value(float v, float mean, float rs, float g, float b) {
#pragma clang fp contract(off)
  return __builtin_fmaf((v - mean) * rs, g, b);
}

// Store VEC output values of chunk `c` of row `row`: row-major, or (nks > 0,
// BF16 and E4M3 outputs) in the tiled GEMM operand layout with nks k stages
// per row tile. A chunk's 8 or 16 output bytes never straddle a 16-byte slot.
template <int OUT, int VEC>
__device__ __forceinline__ void store_chunk(void* y, int64_t row, int64_t hidden, int64_t c,
                                            const float* v, float qscale, int64_t nks) {
  constexpr int OB = OUT == kF32 ? 4 : OUT == kBF16 ? 2 : 1;   // output bytes per value
  const int64_t off = OUT != kF32 && nks > 0 ? tiled_offset(row, c * VEC * OB, nks, 0) : (row * hidden + c * VEC) * OB;
  uint8_t* p = reinterpret_cast<uint8_t*>(y) + off;
  if constexpr (OUT == kF32) {
#pragma unroll
    for (int i = 0; i < VEC; i += 4)
      *reinterpret_cast<float4*>(p + 4 * i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  } else if constexpr (OUT == kBF16) {
    if constexpr (VEC == 8) {
      *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  } else {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < VEC; i += 4)
      w[i / 4] = e4m3_pack4(v[i] * qscale, v[i + 1] * qscale, v[i + 2] * qscale, v[i + 3] * qscale);
    if constexpr (VEC == 8) *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint32_t*>(p) = w[0];
  }
}

// Tiled output staged through LDS: the workgroup's four rows r0 .. r0 + 3
// (one per wave, r0 a multiple of 4, so all in one 256-row tile) are written
// to LDS as the four 64-byte pieces of every k stage, stage s at 256 s with
// row w's piece in slot w ^ (s % 4) (the XOR keeps a wave's chunk writes on
// distinct banks), each piece already in the operand's chunk swizzle; the
// workgroup then stores each stage's 256 bytes as one contiguous run.
template <int OUT, int VEC>
__device__ __forceinline__ void stage_chunk(uint8_t* stg, int w, int64_t row, int64_t c, const float* v,
                                            float qscale) {
  constexpr int OB = OUT == kBF16 ? 2 : 1;
  static_assert(OUT != kF32 && VEC == 8, "bf16 or E4M3 output of 8-value chunks");
  const int kb = (int)c * VEC * OB;                   // byte of the chunk in its row
  const int s = kb >> 6;
  const int slot = ((kb >> 4) & 3) ^ (int)((row >> 2) & 3);
  uint8_t* p = stg + s * 256 + ((w ^ (s & 3)) << 6) + (slot << 4) + (kb & 15);
  if constexpr (OUT == kBF16) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(e4m3_pack4(v[0] * qscale, v[1] * qscale, v[2] * qscale, v[3] * qscale),
                                              e4m3_pack4(v[4] * qscale, v[5] * qscale, v[6] * qscale, v[7] * qscale));
  }
}

struct NormArgs {
  const void* x; const void* gamma; const void* beta;
  int64_t rows, hidden; float eps; int zcg;
  void* y; float* mu; float* rsigma; float* amax; float* scale_out; float* scale_inv_out;
  float* part; int nparts;   // the amax pass's per-workgroup maxima
  int64_t y_nks;             // > 0: y in the tiled GEMM operand layout with that many k stages
  ClearList clear;           // amax pass: floats workgroup 0 sets to zero
};

// Maximum of the amax pass's partial maxima, returned to every thread of the
// workgroup (each thread reads a strided share, then a wave and an LDS
// reduction). The partials are maxima of absolute values, so the result does
// not depend on the order.
__device__ __forceinline__ float block_max_of_parts(const float* part, int n, float* red) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, part[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
  return m;
}

// NCH > 0: NCH 16-byte chunks per lane kept in registers. NCH == 0: loop.
// STAGED (NCH > 0, bf16 or E4M3 output in the tiled GEMM operand layout): the
// output goes through LDS (stage_chunk()) and leaves in 256-byte runs.
template <bool BF16, int NCH, bool RMS, int MODE, int OUT, bool STAGED = false>
__global__ void __launch_bounds__(256) norm_fwd_kernel(NormArgs a) {
  using I = Io<BF16>;
  constexpr int VEC = I::VEC;
  static_assert(!STAGED || (NCH > 0 && MODE != kNormAmax && OUT != kF32), "staged: tiled bf16 / E4M3 rows");
  const int lane = threadIdx.x & 63;
  const int64_t nch = a.hidden / VEC;
  const uint4* gr = reinterpret_cast<const uint4*>(a.gamma);
  const uint4* br = reinterpret_cast<const uint4*>(a.beta);
  const float inv_h = 1.0f / (float)a.hidden;

  if constexpr (MODE == kNormAmax) {
    // the call's amax slots that later passes raise with atomics start at zero
    if (blockIdx.x == 0) {
      const int t = threadIdx.x;
      if (t < a.clear.n) a.clear.first[t] = 0.0f;
      if (t < 3 && a.clear.one[t] != nullptr) *a.clear.one[t] = 0.0f;
    }
  }
  float qscale = 1.0f;
  if constexpr (MODE == kNormQuant) {
    // the tensor's amax from the amax pass's partials; workgroup 0 publishes
    // amax, scale and scale_inv
    __shared__ float qred[4];
    const float amax = block_max_of_parts(a.part, a.nparts, qred);
    qscale = fp8_scale_from_amax(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *a.amax = amax;
      *a.scale_out = qscale;
      *a.scale_inv_out = 1.0f / qscale;
    }
  }
  float lmax = 0.0f;
  // byte-range descriptors: chunks past the row (lane + 64 j >= nch) read as zero
  const uint32_t row_bytes = (uint32_t)(nch * 16);
  const __amdgpu_buffer_rsrc_t rgam = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.gamma), (short)0,
                                                                        (int)row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rbet = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(RMS ? a.gamma : a.beta),
                                                                        (short)0, (int)row_bytes, 0x00020000);
  auto load16 = [&](__amdgpu_buffer_rsrc_t r, int64_t c, auto stream) {
    const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)c * 16, 0, decltype(stream)::value ? kBufAuxStream : 0);
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
  };
  using Stream = std::true_type;
  using Cached = std::false_type;
  // gamma and beta, read once per workgroup into LDS (rows of up to NCH * 64
  // chunks use the register path below)
  __shared__ uint4 sg[NCH > 0 ? NCH * 64 : 1], sb[NCH > 0 && !RMS ? NCH * 64 : 1];
  // STAGED: four rows of output (NCH * 64 chunks of 8 values each)
  __shared__ __attribute__((aligned(16))) uint8_t stg[STAGED ? 4 * NCH * 64 * 8 * (OUT == kBF16 ? 2 : 1) : 16];
  if constexpr (NCH > 0) {
    for (int64_t c = threadIdx.x; c < nch; c += blockDim.x) {
      sg[c] = load16(rgam, c, Cached{});
      if constexpr (!RMS) sb[c] = load16(rbet, c, Cached{});
    }
    __syncthreads();
  }
  // one wave per row; a wave loops over rows wave, wave + 4 G, ... of a grid
  // of G workgroups
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * 4;
  int64_t row = (int64_t)blockIdx.x * 4 + wave;
  // the output of one row from its 16-byte chunks (x, gamma, beta in registers)
  auto finish_row = [&](int64_t row, const uint4* xw) {
    float mean = 0.0f, rs;
    float v[NCH > 0 ? NCH : 1][VEC];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      I::unpack(xw[j], v[j]);
      if constexpr (!RMS) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) s += v[j][i];
      }
    }
    if constexpr (!RMS) mean = wave_sum(s) * inv_h;
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (lane + 64 * j < nch) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float d = v[j][i] - mean;
          ss += d * d;
        }
      }
    }
    rs = rsqrtf(wave_sum(ss) * inv_h + a.eps);
    if constexpr (MODE != kNormQuant) {
      if (lane == 0) {
        if (a.mu != nullptr && !RMS) a.mu[row] = mean;
        if (a.rsigma != nullptr) a.rsigma[row] = rs;
      }
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int64_t c = lane + 64 * j;
      if (c < nch) {
        float g[VEC], b[VEC], y[VEC];
        I::unpack(sg[c], g);
        if constexpr (!RMS) I::unpack(sb[c], b);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float gi = a.zcg ? 1.0f + g[i] : g[i];
          y[i] = norm_value(v[j][i], mean, rs, gi, RMS ? 0.0f : b[i]);
          lmax = fmaxf(lmax, fabsf(y[i]));
        }
        if constexpr (STAGED) stage_chunk<OUT, VEC>(stg, wave, row, c, y, qscale);
        else if constexpr (MODE != kNormAmax) store_chunk<OUT, VEC>(a.y, row, a.hidden, c, y, qscale, a.y_nks);
      }
    }
  };
  if constexpr (STAGED) {
    // every wave of the workgroup walks the same row groups (rows 4 g .. 4 g
    // + 3 of groups g = blockIdx.x, + gridDim.x, ...), so all reach the
    // barriers; a row past the end is neither loaded nor staged
    auto load_row = [&](int64_t r, uint4* xw) {
      const bool ok = r < a.rows;
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint4*>(reinterpret_cast<const uint4*>(a.x) + (ok ? r : 0) * nch), (short)0,
          ok ? (int)row_bytes : 0, 0x00020000);
#pragma unroll
      for (int j = 0; j < NCH; ++j) xw[j] = load16(rx, lane + 64 * j, Stream{});
    };
    constexpr int OB = OUT == kBF16 ? 2 : 1;
    const int64_t groups = (a.rows + 3) / 4;
    const int64_t nks = a.y_nks;
    const int64_t rb = a.hidden * OB;   // output bytes per row
    uint8_t* ybase = reinterpret_cast<uint8_t*>(a.y);
    // the staged group leaves as 256-byte runs: 16-byte unit u = 16 s + q of
    // stage s is slot q % 4 of the piece in LDS slot q / 4
    auto store_group = [&](int64_t g) {
      const int64_t r0 = 4 * g;
      for (int64_t u = threadIdx.x; u < nks * 16; u += blockDim.x) {
        const int64_t st = u >> 4;
        const int q = (int)(u & 15), p = q & 3;
        const int64_t r = r0 + ((q >> 2) ^ (int)(st & 3));
        const int cs = p ^ (int)((r >> 2) & 3);   // the chunk the slot holds
        if (r < a.rows && st * 64 + cs * 16 < rb) {
          const uint4 v = *reinterpret_cast<const uint4*>(stg + st * 256 + q * 16);
          *reinterpret_cast<uint4*>(ybase + (((r0 >> 8) * nks + st) << kTiledBlockShift) + ((r & 255) << 6) + p * 16) = v;
        }
      }
    };
    // LDS-only barrier: the prefetched rows' loads stay in flight across it
    auto lds_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS accesses are done (lgkmcnt 0)
      block_barrier();
    };
    int64_t g = blockIdx.x;
    if (g < groups) {
      uint4 xa[NCH], xb[NCH];
      load_row(row, xa);
      while (true) {
        load_row(row + step, xb);
        __builtin_amdgcn_sched_barrier(0);
        if (row < a.rows) finish_row(row, xa);
        lds_barrier();
        store_group(g);
        lds_barrier();
        row += step;
        g += gridDim.x;
        if (g >= groups) break;
        load_row(row + step, xa);
        __builtin_amdgcn_sched_barrier(0);
        if (row < a.rows) finish_row(row, xb);
        lds_barrier();
        store_group(g);
        lds_barrier();
        row += step;
        g += gridDim.x;
        if (g >= groups) break;
      }
    }
  } else if (row < a.rows) {
    if constexpr (NCH > 0) {
      // the next row's x is in flight while the current one is reduced and
      // written (two register sets used
      // alternately, so no load result is copied before it arrives). Rows past
      // the end get an empty buffer range: their loads return zero and touch
      // no memory, so every load is unconditional.
      auto load_row = [&](int64_t r, uint4* xw) {
        const bool ok = r < a.rows;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint4*>(reinterpret_cast<const uint4*>(a.x) + (ok ? r : 0) * nch), (short)0,
            ok ? (int)row_bytes : 0, 0x00020000);
#pragma unroll
        for (int j = 0; j < NCH; ++j) xw[j] = load16(rx, lane + 64 * j, Stream{});
      };
      uint4 xa[NCH], xb[NCH];
      load_row(row, xa);
      while (true) {
        load_row(row + step, xb);
        __builtin_amdgcn_sched_barrier(0);
        finish_row(row, xa);
        row += step;
        if (row >= a.rows) break;
        load_row(row + step, xa);
        __builtin_amdgcn_sched_barrier(0);
        finish_row(row, xb);
        row += step;
        if (row >= a.rows) break;
      }
    }
  }
  if constexpr (NCH == 0) {
    for (; row < a.rows; row += step) {
      const uint4* xr = reinterpret_cast<const uint4*>(a.x) + row * nch;
      float mean = 0.0f, rs;
      float s = 0.0f, v[VEC];
      // a lane's terms are summed in blocks of kSumBlock chunks, and the
      // blocks' sums into the total: a row of 2^22 features is 2^16 terms
      // per lane, whose plain running sum drifted 5e-5 (relative) from the
      // exact one for bf16 inputs; blocked, the longest chain is 512 terms
      constexpr int64_t kSumBlock = 64 * 64;
      if constexpr (!RMS) {
        for (int64_t c0 = lane; c0 < nch; c0 += kSumBlock) {
          float p = 0.0f;
          for (int64_t c = c0; c < nch && c < c0 + kSumBlock; c += 64) {
            I::unpack(xr[c], v);
#pragma unroll
            for (int i = 0; i < VEC; ++i) p += v[i];
          }
          s += p;
        }
        mean = wave_sum(s) * inv_h;
      }
      float ss = 0.0f;
      for (int64_t c0 = lane; c0 < nch; c0 += kSumBlock) {
        float p = 0.0f;
        for (int64_t c = c0; c < nch && c < c0 + kSumBlock; c += 64) {
          I::unpack(xr[c], v);
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const float d = v[i] - mean;
            p += d * d;
          }
        }
        ss += p;
      }
      rs = rsqrtf(wave_sum(ss) * inv_h + a.eps);
      if constexpr (MODE != kNormQuant) {
        if (lane == 0) {
          if (a.mu != nullptr && !RMS) a.mu[row] = mean;
          if (a.rsigma != nullptr) a.rsigma[row] = rs;
        }
      }
      for (int64_t c = lane; c < nch; c += 64) {
        float g[VEC], b[VEC], y[VEC];
        I::unpack(xr[c], v);
        I::unpack(gr[c], g);
        if constexpr (!RMS) I::unpack(br[c], b);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float gi = a.zcg ? 1.0f + g[i] : g[i];
          y[i] = norm_value(v[i], mean, rs, gi, RMS ? 0.0f : b[i]);
          lmax = fmaxf(lmax, fabsf(y[i]));
        }
        if constexpr (MODE != kNormAmax) store_chunk<OUT, VEC>(a.y, row, a.hidden, c, y, qscale, a.y_nks);
      }
    }
  }
  if constexpr (MODE == kNormAmax) {
    __shared__ float red[4];
    block_max_store(lmax, a.part + blockIdx.x, red);
  }
}

template <bool BF16, int NCH, bool RMS>
hipError_t dispatch_mode(const NormArgs& a, int mode, int y_dtype, hipStream_t s) {
  // one row per wave at a time; the grid is capped and the waves loop over
  // rows (the next row loads while one is reduced). The amax pass has its own
  // cap, and its grid size is the number of partials the quantise pass reads.
  const int64_t blocks = (a.rows + 3) / 4;
  const int64_t cap = mode == kNormAmax ? (int64_t)kNormAmaxBlocks : (int64_t)kNormBlocks;
  const dim3 grid((unsigned)(blocks > cap ? cap : blocks)), block(256);
  // tiled output of the register path goes through LDS
  constexpr bool kStage = NCH > 0 && BF16;
  const bool staged = kStage && a.y_nks > 0;
  if (mode == kNormAmax) {
    launch_kernel(norm_fwd_kernel<BF16, NCH, RMS, kNormAmax, kF32>, grid, block, 0, s, a);
  } else if (mode == kNormQuant) {
    if (staged) launch_kernel(norm_fwd_kernel<BF16, NCH, RMS, kNormQuant, kE4M3, kStage>, grid, block, 0, s, a);
    else launch_kernel(norm_fwd_kernel<BF16, NCH, RMS, kNormQuant, kE4M3>, grid, block, 0, s, a);
  } else if (y_dtype == kF32) {
    launch_kernel(norm_fwd_kernel<BF16, NCH, RMS, kNormStore, kF32>, grid, block, 0, s, a);
  } else if (staged) {
    launch_kernel(norm_fwd_kernel<BF16, NCH, RMS, kNormStore, kBF16, kStage>, grid, block, 0, s, a);
  } else {
    launch_kernel(norm_fwd_kernel<BF16, NCH, RMS, kNormStore, kBF16>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <bool BF16, bool RMS>
hipError_t dispatch_nch(const NormArgs& a, int mode, int y_dtype, hipStream_t s) {
  const int64_t nch = a.hidden / Io<BF16>::VEC;
  const int64_t per_lane = (nch + 63) / 64;
  if (per_lane <= 1) return dispatch_mode<BF16, 1, RMS>(a, mode, y_dtype, s);
  if (per_lane <= 2) return dispatch_mode<BF16, 2, RMS>(a, mode, y_dtype, s);
  if (per_lane <= 4) return dispatch_mode<BF16, 4, RMS>(a, mode, y_dtype, s);
  if (per_lane <= 8) return dispatch_mode<BF16, 8, RMS>(a, mode, y_dtype, s);
  return dispatch_mode<BF16, 0, RMS>(a, mode, y_dtype, s);
}

}  // namespace

int64_t norm_amax_parts(int64_t rows) {
  const int64_t blocks = (rows + 3) / 4;
  return blocks < kNormAmaxBlocks ? blocks : (int64_t)kNormAmaxBlocks;
}

hipError_t launch_norm(const void* x, const void* gamma, const void* beta, int64_t rows,
                       int64_t hidden, int x_dtype, bool rms, bool zcg, float eps, int mode,
                       int y_dtype, void* y, float* mu, float* rsigma, float* amax,
                       float* scale_out, float* scale_inv_out, float* part, hipStream_t s, bool y_tiled,
                       const ClearList* clear) {
  static const char* names[3] = {"norm_fwd", "norm_amax", "norm_quant"};
  LaunchScope scope(names[mode], s);
  if (mode != kNormStore && part == nullptr) return hipErrorInvalidValue;
  const int64_t out_bytes = mode == kNormQuant ? 1 : y_dtype == kBF16 ? 2 : 4;
  if (y_tiled && (out_bytes == 4 || hidden * out_bytes > kTiledMaxRowBytes)) return hipErrorInvalidValue;
  NormArgs a{x, gamma, beta, rows, hidden, eps, zcg ? 1 : 0, y, mu, rsigma, amax, scale_out,
             scale_inv_out, part, (int)norm_amax_parts(rows), y_tiled ? tiled_stages(hidden * out_bytes) : 0,
             clear != nullptr ? *clear : ClearList{}};
  if (a.clear.n > 256 || (a.clear.n > 0 && a.clear.first == nullptr) || (clear != nullptr && mode != kNormAmax))
    return hipErrorInvalidValue;
  if (x_dtype == kBF16) {
    return rms ? dispatch_nch<true, true>(a, mode, y_dtype, s)
               : dispatch_nch<true, false>(a, mode, y_dtype, s);
  }
  return rms ? dispatch_nch<false, true>(a, mode, y_dtype, s)
             : dispatch_nch<false, false>(a, mode, y_dtype, s);
}

}  // namespace te
