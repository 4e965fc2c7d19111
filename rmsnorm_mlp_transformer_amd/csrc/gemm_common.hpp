// Tile geometry and the fused epilogue shared by the bf16 and fp8 MFMA GEMMs.
//
// Work split: a workgroup of 2 x WN waves computes a 256 x 256 tile of
// h = A * B. Wave w = (wm, wn) = (w % 2, w / 2) owns 128 rows x (256 / WN)
// columns as 4 x NJ blocks of 32 x 32 (NJ = 8 / WN). The GEMMs issue the MFMA with the B fragment as
// the first operand, so each accumulator block holds the transposed tile:
// lane l owns row m = 32 i + (l % 32) and, for register group g = 0..3, the
// four consecutive columns 32 j + 8 g + 4 (l / 32) + {0,1,2,3} in
// registers 4 g .. 4 g + 3. Every epilogue store is therefore an 8-byte
// vector of four bf16 values.
//
// Gated activations ((f, linear) pairs, "NVIDIA TransformerEngine JAX
// Activation", Inputs: activation_type ("silu", "linear")): the tile's 256 B
// columns are the 128 first-half columns [j0, j0 + 128) followed by the
// matching second-half columns [F + j0, F + j0 + 128); wave wn owns the
// first-half blocks j < NJ / 2 at [j0 + 16 NJ wn, +16 NJ) and their partners
// j + NJ / 2, so the gate product f(a) * b happens in registers.
#pragma once

#include "te_common.hpp"

namespace te {

// Waves per GEMM workgroup (4: one per SIMD, 128 x 128 each; 8: two per SIMD,
// 128 x 64 each).
#ifndef TE_GEMM_WAVES
#define TE_GEMM_WAVES 8
#endif
// bf16 pipeline: k depth per LDS stage and number of stages (STAGES * BK * 1 KiB of LDS).
#ifndef TE_GEMM_BK
#define TE_GEMM_BK 32
#endif
#ifndef TE_GEMM_STAGES
#define TE_GEMM_STAGES 4
#endif
// fp8 pipeline: k bytes per LDS stage and number of stages.
#ifndef TE_GEMM_FP8_BK
#define TE_GEMM_FP8_BK 64
#endif
#ifndef TE_GEMM_FP8_STAGES
#define TE_GEMM_FP8_STAGES 4
#endif

constexpr int kTileM = 256;
constexpr int kTileN = 256;

struct EpiArgs {
  const uint16_t* bias;   // bf16 [n_b] or NULL
  uint16_t* out;          // bf16 [M, n_out] or NULL
  uint16_t* h_out;        // bf16 [M, n_b] or NULL
  float* amax;            // or NULL
  int M, n_b, F;          // F = n_b / 2 when gated, else n_b
};

// LDS row (0..255) of B-fragment block j (of NJ) for wave column wn.
template <bool GATED, int NJ>
__device__ __forceinline__ int b_block_row(int wn, int j) {
  if constexpr (GATED) {
    constexpr int H = NJ / 2;
    return j < H ? wn * 32 * H + j * 32 : 128 + wn * 32 * H + (j - H) * 32;
  } else {
    return wn * 32 * NJ + j * 32;
  }
}

// Maps the linear workgroup index to a (tile_m, tile_n) pair. Workgroups are
// dealt round-robin to the 8 XCDs (each with its own L2), so the index is
// first regrouped so that consecutive logical tiles land on one XCD; the
// logical order then walks groups of 8 row-tiles across all column-tiles, so
// the tiles resident on an XCD at one time share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
  constexpr int kGroup = 8;
  const int per_group = kGroup * tiles_n;
  const int group = b / per_group;
  const int first_m = group * kGroup;
  const int gsz = min(tiles_m - first_m, kGroup);
  const int in_group = b - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

__device__ __forceinline__ void load_bias4(const uint16_t* bias, int col, float* b) {
  if (bias == nullptr) {
    b[0] = b[1] = b[2] = b[3] = 0.0f;
    return;
  }
  const uint2 w = *reinterpret_cast<const uint2*>(bias + col);
  b[0] = bf16_lo(w.x); b[1] = bf16_hi(w.x); b[2] = bf16_lo(w.y); b[3] = bf16_hi(w.y);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

__device__ __forceinline__ void round_bf16x4(float* v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = bf16_to_f32(f32_to_bf16(v[r]));
}

// h = acc * scale + bias; then the stores / amax selected by the flags.
// AMAX evaluates the activation from h rounded to bf16, exactly as a later
// pass reading the stored h would.
template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX, int NJ>
__device__ __forceinline__ void gemm_epilogue(const f32x16_t (&acc)[4][NJ], const EpiArgs& ep,
                                              int m0, int n0, int wm, int wn, int lane,
                                              float scale) {
  const int lm = lane & 31, lh = lane >> 5;
  float lmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + lm;
    if (m < ep.M) {
      if constexpr (!GATED) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = n0 + wn * 32 * NJ + j * 32 + g * 8 + lh * 4;
            if (col < ep.n_b) {
              float h[4], b[4];
              load_bias4(ep.bias, col, b);
#pragma unroll
              for (int r = 0; r < 4; ++r) h[r] = acc[i][j][4 * g + r] * scale + b[r];
              if constexpr (STORE_H) store_bf16x4(ep.h_out + (int64_t)m * ep.n_b + col, h);
              if constexpr (AMAX) round_bf16x4(h);
              float o[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) o[r] = act_fwd<ACT>(h[r]);
              if constexpr (STORE_OUT) store_bf16x4(ep.out + (int64_t)m * ep.n_b + col, o);
              if constexpr (AMAX) {
#pragma unroll
                for (int r = 0; r < 4; ++r) lmax = fmaxf(lmax, fabsf(o[r]));
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = n0 + wn * 16 * NJ + j * 32 + g * 8 + lh * 4;   // first-half column
            if (col < ep.F) {
              float ha[4], hb[4], ba[4], bb[4];
              load_bias4(ep.bias, col, ba);
              load_bias4(ep.bias, ep.F + col, bb);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                ha[r] = acc[i][j][4 * g + r] * scale + ba[r];
                hb[r] = acc[i][j + NJ / 2][4 * g + r] * scale + bb[r];
              }
              if constexpr (STORE_H) {
                store_bf16x4(ep.h_out + (int64_t)m * ep.n_b + col, ha);
                store_bf16x4(ep.h_out + (int64_t)m * ep.n_b + ep.F + col, hb);
              }
              if constexpr (AMAX) {
                round_bf16x4(ha);
                round_bf16x4(hb);
              }
              float o[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) o[r] = act_fwd<ACT>(ha[r]) * hb[r];
              if constexpr (STORE_OUT) store_bf16x4(ep.out + (int64_t)m * ep.F + col, o);
              if constexpr (AMAX) {
#pragma unroll
                for (int r = 0; r < 4; ++r) lmax = fmaxf(lmax, fabsf(o[r]));
              }
            }
          }
        }
      }
    }
  }
  if constexpr (AMAX) {
    lmax = wave_max(lmax);
    if (lane == 0) atomic_max_nonneg(ep.amax, lmax);
  }
}

}  // namespace te
