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

// The four LDS stage arrays of a GEMM (32 KiB each) are reused after the main
// loop as a 256 x C bf16 staging tile: rows [64 a, 64 a + 64) live in array a,
// which the callable st(a) returns.

// Staging layout: row r holds C bf16 as C / 4 units of 8 bytes; unit u sits at
// u ^ (r % 32). A wave's 8-byte writes (32 rows, one unit each) and its
// 16-byte reads (16 chunks of one row) then touch 64 distinct banks.
template <int C, typename St>
__device__ __forceinline__ uint8_t* stage_unit(St st, int r, int u) {
  return st(r >> 6) + (r & 63) * (C * 2) + 8 * (u ^ (r & 31));
}

// Copies the staged tile to global memory: every lane moves 16 bytes, a wave
// covers whole rows (fully coalesced). dst(r, c) returns the destination of
// tile row r, columns [c, c + 8), or nullptr when it is outside the matrix.
template <int C, int NT, typename St, typename Dst>
__device__ __forceinline__ void stage_copy_out(St st, int tid, int rows_valid, Dst dst) {
  constexpr int CH = C / 8;                        // 16-byte chunks per row
#pragma unroll 4
  for (int idx = tid; idx < kTileM * CH; idx += NT) {
    const int r = idx / CH, q = idx % CH;
    if (r >= rows_valid) break;                    // rows only grow with idx
    uint16_t* d = dst(r, 8 * q);
    if (d == nullptr) continue;
    const uint8_t* src = st(r >> 6) + (r & 63) * (C * 2) + 16 * (q ^ ((r & 31) >> 1));
    uint4 v = *reinterpret_cast<const uint4*>(src);
    if (r & 1) v = make_uint4(v.z, v.w, v.x, v.y);  // odd rows swap the two 8-byte units
    *reinterpret_cast<uint4*>(d) = v;
  }
}

// h = acc * scale + bias; then the stores / amax selected by the flags. Both
// stores go through the LDS staging tile (the main loop's LDS is free here).
// AMAX evaluates the activation from h rounded to bf16, exactly as a later
// pass reading the stored h would.
template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX, int NJ, int NT, typename St>
__device__ __forceinline__ void gemm_epilogue(const f32x16_t (&acc)[4][NJ], const EpiArgs& ep,
                                              int m0, int n0, int wm, int wn, int lane, int tid,
                                              float scale, St st) {
  const int lm = lane & 31, lh = lane >> 5;
  const int rows_valid = min(ep.M - m0, kTileM);
  float lmax = 0.0f;
  // every wave's LDS reads of the main loop are done before the staging writes
  __syncthreads();

  // ---- pre-activation h: tile columns follow the B tile (gated: first half, then second half)
  if constexpr (STORE_H || AMAX) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + lm;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int tc0 = b_block_row<GATED, NJ>(wn, j);       // tile column of the block
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int tc = tc0 + g * 8 + lh * 4;
          int col;
          if constexpr (GATED) col = tc < 128 ? n0 + tc : ep.F + n0 + tc - 128;
          else col = n0 + tc;
          float h[4], b[4];
          const bool in_range = GATED ? (n0 + (tc & 127) < ep.F) : (col < ep.n_b);
          if (in_range) load_bias4(ep.bias, col, b);
          else b[0] = b[1] = b[2] = b[3] = 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = acc[i][j][4 * g + q] * scale + b[q];
          if constexpr (STORE_H) {
            *reinterpret_cast<uint2*>(stage_unit<256>(st, r, tc >> 2)) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
          if constexpr (AMAX && !GATED) {
            if (in_range && m0 + r < ep.M) {
              round_bf16x4(h);
#pragma unroll
              for (int q = 0; q < 4; ++q) lmax = fmaxf(lmax, fabsf(act_fwd<ACT>(h[q])));
            }
          }
        }
      }
      if constexpr (AMAX && GATED) {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = n0 + wn * 16 * NJ + j * 32 + g * 8 + lh * 4;   // first-half column
            if (col < ep.F && m0 + r < ep.M) {
              float ha[4], hb[4], ba[4], bb[4];
              load_bias4(ep.bias, col, ba);
              load_bias4(ep.bias, ep.F + col, bb);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                ha[q] = acc[i][j][4 * g + q] * scale + ba[q];
                hb[q] = acc[i][j + NJ / 2][4 * g + q] * scale + bb[q];
              }
              round_bf16x4(ha);
              round_bf16x4(hb);
#pragma unroll
              for (int q = 0; q < 4; ++q) lmax = fmaxf(lmax, fabsf(act_fwd<ACT>(ha[q]) * hb[q]));
            }
          }
        }
      }
    }
    if constexpr (STORE_H) {
      __syncthreads();
      stage_copy_out<256, NT>(st, tid, rows_valid, [&](int r, int c) -> uint16_t* {
        int col;
        bool ok;
        if constexpr (GATED) {
          ok = n0 + (c & 127) < ep.F;
          col = c < 128 ? n0 + c : ep.F + n0 + c - 128;
        } else {
          col = n0 + c;
          ok = col < ep.n_b;
        }
        return ok ? ep.h_out + (int64_t)(m0 + r) * ep.n_b + col : nullptr;
      });
      if constexpr (STORE_OUT) __syncthreads();      // the staging tile is reused below
    }
  }

  // ---- activation output
  if constexpr (STORE_OUT) {
    constexpr int C = GATED ? 128 : 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + lm;
      if constexpr (!GATED) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int tc = wn * 32 * NJ + j * 32 + g * 8 + lh * 4;
            const int col = n0 + tc;
            float h[4], b[4];
            if (col < ep.n_b) load_bias4(ep.bias, col, b);
            else b[0] = b[1] = b[2] = b[3] = 0.0f;
            float o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              h[q] = acc[i][j][4 * g + q] * scale + b[q];
              o[q] = act_fwd<ACT>(h[q]);
            }
            *reinterpret_cast<uint2*>(stage_unit<C>(st, r, tc >> 2)) =
                make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int tc = wn * 16 * NJ + j * 32 + g * 8 + lh * 4;        // first-half tile column
            const int col = n0 + tc;
            float ba[4], bb[4];
            if (col < ep.F) {
              load_bias4(ep.bias, col, ba);
              load_bias4(ep.bias, ep.F + col, bb);
            } else {
              ba[0] = ba[1] = ba[2] = ba[3] = bb[0] = bb[1] = bb[2] = bb[3] = 0.0f;
            }
            float o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              o[q] = act_fwd<ACT>(acc[i][j][4 * g + q] * scale + ba[q]) * (acc[i][j + NJ / 2][4 * g + q] * scale + bb[q]);
            *reinterpret_cast<uint2*>(stage_unit<C>(st, r, tc >> 2)) =
                make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          }
        }
      }
    }
    __syncthreads();
    const int n_out = GATED ? ep.F : ep.n_b;
    stage_copy_out<C, NT>(st, tid, rows_valid, [&](int r, int c) -> uint16_t* {
      return n0 + c < n_out ? ep.out + (int64_t)(m0 + r) * n_out + n0 + c : nullptr;
    });
  }

  if constexpr (AMAX) {
    __shared__ float red[NT / 64];
    block_max_atomic(lmax, ep.amax, red);
  }
}

}  // namespace te
