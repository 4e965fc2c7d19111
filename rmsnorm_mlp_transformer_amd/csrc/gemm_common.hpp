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

#include <type_traits>

#include "gemm_lds.hpp"
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
// bf16 schedule: 1 = ping-pong (the two waves of a SIMD alternate between
// MFMA and memory phases), 0 = every wave interleaves reads and MFMAs.
#ifndef TE_GEMM_PINGPONG
#define TE_GEMM_PINGPONG 1
#endif

constexpr int kTileM = 256;
constexpr int kTileN = 256;

struct EpiArgs {
  const uint16_t* bias;   // bf16 [n_b] or NULL
  uint16_t* out;          // bf16 [M, n_out] or NULL (fp32 [M, n_out] with OUT_F32)
  uint16_t* h_out;        // bf16 [M, n_b] or NULL
  float* amax;            // or NULL
  int M, n_b, F;          // F = n_b / 2 when gated, else n_b
  int group;              // row-tiles per group of the tile walk (tile_group())
  int out_nks;            // > 0: out is a tiled operand with that many k stages per row tile
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
// logical order then walks groups of `group` row-tiles across all
// column-tiles, so the tiles resident on an XCD at one time share A and B
// panels in its L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int group, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int b = blockIdx.x;
  if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
  const int per_group = group * tiles_n;
  const int grp = b / per_group;
  const int first_m = grp * group;
  const int gsz = min(tiles_m - first_m, group);
  const int in_group = b - grp * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// Row-tiles per group of the walk above. The XCD's ~32 resident tiles cover
// group x (32 / group) tiles; 4 and 8 minimise the panels they read. A sweep
// at the workloads' shapes (2, 4, 8, 16; interleaved runs on one box) picked,
// for 64 or more column-tiles, 4 for the bf16 GEMM and 2 for the fp8 GEMM
// (0.5% and 1-3% faster than 8), and for fewer column-tiles 8 and 4; the
// gated GEMM1 keeps 8 (4 was 0.4% slower); 16 was up to 30% slower.
inline int tile_group(int64_t tiles_n, bool fp8, bool gated) {
  if (gated) return 8;
  if (fp8) return tiles_n >= 64 ? 2 : 4;
  return tiles_n >= 64 ? 4 : 8;
}

// Global column of tile column tc (gated tiles hold [n0, n0 + 128) of the
// first half and the same columns of the second half); in_range is false
// for columns outside the matrix.
template <bool GATED>
__device__ __forceinline__ int tile_col(const EpiArgs& ep, int n0, int tc, bool& in_range) {
  if constexpr (GATED) {
    in_range = n0 + (tc & 127) < ep.F;
    return tc < 128 ? n0 + tc : ep.F + n0 + tc - 128;
  } else {
    in_range = n0 + tc < ep.n_b;
    return n0 + tc;
  }
}

// The bias values of the columns a lane owns in the epilogue (block j of NJ,
// group g of 4: tile columns b_block_row(wn, j) + 8 g + 4 (lane / 32) + 0..3)
// as packed bf16 pairs; zero without a bias or outside the matrix. Loaded
// before the main loop, so the epilogue never waits for them.
template <bool GATED, int NJ>
__device__ __forceinline__ void load_bias_frag(const EpiArgs& ep, int n0, int wn, int lane, uint2 (&bv)[NJ][4]) {
  const int lh = (lane & 63) >> 5;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bool ok;
      const int col = tile_col<GATED>(ep, n0, b_block_row<GATED, NJ>(wn, j) + g * 8 + lh * 4, ok);
      bv[j][g] = ep.bias != nullptr && ok ? *reinterpret_cast<const uint2*>(ep.bias + col) : make_uint2(0u, 0u);
    }
}

// h from an accumulator: acc * scale + bias, or acc * scale when the bias
// started the accumulation (the bf16 GEMMs, whose scale is 1)
template <bool IN_ACC>
__device__ __forceinline__ float hval(float acc, float scale, float b) {
  return IN_ACC ? acc * scale : acc * scale + b;
}

__device__ __forceinline__ void unpack_bias4(const uint2& w, float* b) {
  b[0] = bf16_lo(w.x); b[1] = bf16_hi(w.x); b[2] = bf16_lo(w.y); b[3] = bf16_hi(w.y);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// x, as a value the compiler cannot see through (it stops the reuse of
// values computed from x earlier in the epilogue).
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
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
// covers whole rows (fully coalesced). The LDS reads of a batch of BATCH
// chunks per thread are issued before its stores. dst(r, c) returns the
// destination of tile row r, columns [c, c + 8), or nullptr when it is
// outside the matrix.
template <int C, int NT, int BATCH, typename St, typename Dst>
__device__ __forceinline__ void stage_copy_out(St st, int tid, int rows_valid, Dst dst) {
  constexpr int CH = C / 8;                        // 16-byte chunks per row
  constexpr int N = kTileM * CH / NT;              // chunks per thread
  static_assert(kTileM * CH % NT == 0 && NT % CH == 0, "whole rows per pass");
  static_assert(N % BATCH == 0, "whole batches");
#pragma unroll
  for (int k0 = 0; k0 < N; k0 += BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int r = (tid + (k0 + k) * NT) / CH, q = (tid + (k0 + k) * NT) % CH;
      v[k] = *reinterpret_cast<const uint4*>(st(r >> 6) + (r & 63) * (C * 2) + 16 * (q ^ ((r & 31) >> 1)));
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int r = (tid + (k0 + k) * NT) / CH, q = (tid + (k0 + k) * NT) % CH;
      if (r < rows_valid) {
        uint16_t* d = dst(r, 8 * q);
        if (d != nullptr) {
          const uint4 w = (r & 1) ? make_uint4(v[k].z, v[k].w, v[k].x, v[k].y) : v[k];  // odd rows swap 8-byte units
          *reinterpret_cast<uint4*>(d) = w;
        }
      }
    }
  }
}

// Tiled staging (an output in the tiled GEMM operand layout): the tile is
// staged as its own tiled image, block s (tile columns [32 s, 32 s + 32))
// of rows [64 a, 64 a + 64) at st(a) + 4 KiB s, row r at 64 (r % 64), its
// 16-byte chunk c at slot c ^ chunk_swizzle<4>(r) as in global memory, and
// the two 8-byte halves of the slot exchanged in rows with bit 4 set. A
// staging write (8 bytes: four columns of one row, 32 consecutive rows per
// half-wave) then touches 32 distinct 8-byte bank pairs, and the copy-out
// moves each wave's 16 rows x 64 bytes of a block as one contiguous KiB,
// from LDS and to memory alike.
template <typename St>
__device__ __forceinline__ uint8_t* stage_tiled(St st, int r, int tc) {
  const int s = tc >> 5, c = (tc >> 3) & 3, h = ((tc >> 2) & 1) ^ ((r >> 4) & 1);
  return st(r >> 6) + s * 4096 + (r & 63) * 64 + ((c ^ chunk_swizzle<4>(r)) << 4) + h * 8;
}

// Copies a tile staged by stage_tiled() (C bf16 columns) to the tiled
// operand whose block 0 for this tile starts at dst (block s at dst + s * 16
// KiB). Rows past rows_valid and columns past cols_valid are not written.
template <int C, int NT, int BATCH, typename St>
__device__ __forceinline__ void stage_copy_out_tiled(St st, int tid, int rows_valid, int cols_valid, uint8_t* dst) {
  constexpr int N = kTileM * (C / 8) / NT;   // 16-byte chunks per thread
  static_assert(kTileM * (C / 8) % NT == 0 && C % 32 == 0, "whole blocks");
  static_assert(N % BATCH == 0, "whole batches");
#pragma unroll
  for (int k0 = 0; k0 < N; k0 += BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = tid + (k0 + k) * NT, p = u & 3, r = (u >> 2) & 255, s = u >> 10;   // slot p of row r, block s
      v[k] = *reinterpret_cast<const uint4*>(st(r >> 6) + s * 4096 + (r & 63) * 64 + p * 16);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int u = tid + (k0 + k) * NT, p = u & 3, r = (u >> 2) & 255, s = u >> 10;
      const int col = 32 * s + 8 * (p ^ chunk_swizzle<4>(r));   // first of the slot's 8 columns
      if (r < rows_valid && col < cols_valid) {
        const uint4 w = (r & 16) ? make_uint4(v[k].z, v[k].w, v[k].x, v[k].y) : v[k];
        *reinterpret_cast<uint4*>(dst + ((int64_t)s << kTiledBlockShift) + r * 64 + p * 16) = w;
      }
    }
  }
}

// max |act(h)| over values whose range is [hmin, hmax]. Each supported
// activation is increasing for h >= 0 and bounded in magnitude by a small
// constant for h < 0 (GELU: 0.170 near h = -0.75, SiLU: 0.279 near h = -1.28,
// ReLU: 0), so once |act(hmax)| reaches amax_exact_from() the negative side
// cannot exceed it and the max is act(hmax). Linear: max(|hmax|, |hmin|).
// No values (hmax < hmin): 0.
template <int ACT>
__device__ __forceinline__ float amax_from_range(float hmax, float hmin) {
  if (!(hmax >= hmin)) return 0.0f;
  if constexpr (ACT == kLinear) return fmaxf(fabsf(hmax), fabsf(hmin));
  else if constexpr (ACT == kRelu) return fmaxf(hmax, 0.0f);
  else return hmax > 0.0f ? fabsf(act_fwd<ACT>(hmax)) : 0.0f;
}
template <int ACT>
constexpr float amax_exact_from() {
  return ACT == kGelu || ACT == kGeluErf ? 0.2f : ACT == kSilu ? 0.3f : 0.0f;
}

// h = acc * scale + bias (BIAS_IN_ACC: acc * scale, the accumulators having
// started from the bias); then the stores / amax selected by the flags. Both
// bf16 stores go through the LDS staging tile (the main loop's LDS is free
// here). AMAX evaluates the activation from h rounded to bf16, exactly as a
// later pass reading the stored h would. bv: load_bias_frag() of the same
// lane. OUT_F32 (plain, ungated output only) writes the output as fp32 with
// direct 16-byte stores: a lane's four consecutive columns of one row; the
// four register groups of a block cover 128 contiguous bytes of each row.
template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX, int NJ, int NT, bool OUT_F32 = false,
          bool BIAS_IN_ACC = false, typename St>
__device__ __forceinline__ void gemm_epilogue(const f32x16_t (&acc)[4][NJ], const uint2 (&bv)[NJ][4],
                                              const EpiArgs& ep, int m0, int n0, int wm, int wn, int lane,
                                              int tid, float scale, St st) {
  const int lm = lane & 31, lh = lane >> 5;
  const int rows_valid = min(ep.M - m0, kTileM);
  if constexpr (OUT_F32) {
    static_assert(STORE_OUT && !STORE_H && !AMAX && !GATED, "fp32 output: plain epilogue only");
    float* out = reinterpret_cast<float*>(ep.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + lm;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int tc = b_block_row<false, NJ>(wn, j) + g * 8 + lh * 4;
          float b[4];
          unpack_bias4(bv[j][g], b);
          float4 o;
          o.x = act_fwd<ACT>(hval<BIAS_IN_ACC>(acc[i][j][4 * g + 0], scale, b[0]));
          o.y = act_fwd<ACT>(hval<BIAS_IN_ACC>(acc[i][j][4 * g + 1], scale, b[1]));
          o.z = act_fwd<ACT>(hval<BIAS_IN_ACC>(acc[i][j][4 * g + 2], scale, b[2]));
          o.w = act_fwd<ACT>(hval<BIAS_IN_ACC>(acc[i][j][4 * g + 3], scale, b[3]));
          // n_b is a multiple of 16 and tc of 4: the four columns are all in or all out
          if (r < rows_valid && n0 + tc < ep.n_b)
            *reinterpret_cast<float4*>(out + (int64_t)(m0 + r) * ep.n_b + n0 + tc) = o;
        }
      }
    }
    return;
  }
  float lmax = 0.0f;
  // range of the lane's h (plain amax), rounded to bf16 at the end: rounding
  // to nearest is monotonic, so the rounded maximum is the maximum of the
  // rounded values (and likewise the minimum)
  float hmax = -INFINITY, hmin = INFINITY;
  // every wave's LDS reads of the main loop are done before the staging writes
  __syncthreads();

  // ---- pre-activation h: tile columns follow the B tile (gated: first half, then second half)
  if constexpr (STORE_H || AMAX) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + lm;
      float hmax_i = -INFINITY, hmin_i = INFINITY;   // this row's part of the range
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int tc = b_block_row<GATED, NJ>(wn, j) + g * 8 + lh * 4;
          float h[4], b[4];
          unpack_bias4(bv[j][g], b);
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = hval<BIAS_IN_ACC>(acc[i][j][4 * g + q], scale, b[q]);
          if constexpr (STORE_H) {
            *reinterpret_cast<uint2*>(stage_unit<256>(st, r, tc >> 2)) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
          if constexpr (AMAX && !GATED) {
            // no column check: a column past the matrix holds h = 0 exactly
            // (its B values and its bias read as zero), and a 0 added to the
            // range changes no result of amax_from_range() (nor the exact
            // evaluation it falls back to)
            hmax_i = fmaxf(fmaxf(hmax_i, h[0]), fmaxf(h[1], fmaxf(h[2], h[3])));
            hmin_i = fminf(fminf(hmin_i, h[0]), fminf(h[1], fminf(h[2], h[3])));
          }
        }
      }
      if constexpr (AMAX && !GATED) {
        // rows past the matrix hold h = bias: left out, one check per row
        if (m0 + r < ep.M) {
          hmax = fmaxf(hmax, hmax_i);
          hmin = fminf(hmin, hmin_i);
        }
      }
      if constexpr (AMAX && GATED) {
        // block j (first half) pairs with block j + NJ / 2 (the same columns of the second half)
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = n0 + b_block_row<GATED, NJ>(wn, j) + g * 8 + lh * 4;   // first-half column
            if (col < ep.F && m0 + r < ep.M) {
              float ha[4], hb[4], ba[4], bb[4];
              unpack_bias4(bv[j][g], ba);
              unpack_bias4(bv[j + NJ / 2][g], bb);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                ha[q] = hval<BIAS_IN_ACC>(acc[i][j][4 * g + q], scale, ba[q]);
                hb[q] = hval<BIAS_IN_ACC>(acc[i][j + NJ / 2][4 * g + q], scale, bb[q]);
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
      // while the accumulators are still live (STORE_OUT follows), smaller batches
      constexpr int kHChunks = kTileM * 32 / NT;
      stage_copy_out<256, NT, STORE_OUT ? 4 : kHChunks>(st, tid, rows_valid, [&](int r, int c) -> uint16_t* {
        bool ok;
        const int col = tile_col<GATED>(ep, n0, c, ok);
        return ok ? ep.h_out + (int64_t)(m0 + r) * ep.n_b + col : nullptr;
      });
      if constexpr (STORE_OUT) __syncthreads();      // the staging tile is reused below
    }
  }

  // ---- activation output
  if constexpr (STORE_OUT) {
    constexpr int C = GATED ? 128 : 256;
    // the staging layout is chosen once, outside the loops (a per-store
    // choice costs a branch and both address computations per store); with
    // the h store before it, the per-store choice keeps fewer registers live
    auto stage_act = [&](auto tiled) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + lm;
        auto dst = [&](int tc) -> uint2* {
          return reinterpret_cast<uint2*>(static_cast<bool>(tiled) ? stage_tiled(st, r, tc) : stage_unit<C>(st, r, tc >> 2));
        };
        if constexpr (!GATED) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int tc = b_block_row<GATED, NJ>(wn, j) + g * 8 + lh * 4;
              float b[4], o[4];
              unpack_bias4(bv[j][g], b);
#pragma unroll
              for (int q = 0; q < 4; ++q) o[q] = act_fwd<ACT>(hval<BIAS_IN_ACC>(acc[i][j][4 * g + q], scale, b[q]));
              *dst(tc) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NJ / 2; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int tc = b_block_row<GATED, NJ>(wn, j) + g * 8 + lh * 4;   // first-half tile column
              float ba[4], bb[4], o[4];
              unpack_bias4(bv[j][g], ba);
              unpack_bias4(bv[j + NJ / 2][g], bb);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                o[q] = act_fwd<ACT>(hval<BIAS_IN_ACC>(acc[i][j][4 * g + q], scale, ba[q])) * (hval<BIAS_IN_ACC>(acc[i][j + NJ / 2][4 * g + q], scale, bb[q]));
              *dst(tc) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            }
          }
        }
      }
    };
    if constexpr (STORE_H) stage_act(ep.out_nks > 0);
    else if (ep.out_nks > 0) stage_act(std::true_type{});
    else stage_act(std::false_type{});
    __syncthreads();
    const int n_out = GATED ? ep.F : ep.n_b;
    if (ep.out_nks > 0) {
      // m0 / 256 is the row tile; n0 is a multiple of 128 columns (256 bytes), i.e. of 4 k stages
      uint8_t* dst = reinterpret_cast<uint8_t*>(ep.out) +
                     (((int64_t)(m0 / kTileM) * ep.out_nks + n0 / 32) << kTiledBlockShift);
      stage_copy_out_tiled<C, NT, 8>(st, tid, rows_valid, n_out - n0, dst);
    } else {
      stage_copy_out<C, NT, kTileM * (C / 8) / NT>(st, tid, rows_valid, [&](int r, int c) -> uint16_t* {
        return n0 + c < n_out ? ep.out + (int64_t)(m0 + r) * n_out + n0 + c : nullptr;
      });
    }
  }

  if constexpr (AMAX && !GATED) {
    // max |act(h)| from the range of h: exact whenever it reaches the
    // activation's threshold; otherwise (a lane whose values are all small)
    // every value is evaluated.
    lmax = amax_from_range<ACT>(bf16_to_f32(f32_to_bf16(hmax)), bf16_to_f32(f32_to_bf16(hmin)));
    if (lmax < amax_exact_from<ACT>()) {
      lmax = 0.0f;
      // an opaque copy of the scale: recomputing h here from the
      // accumulators keeps the compiler from holding the first pass's h
      // values (128 registers) live until this rarely taken branch
      const float scale_a = opaque(scale);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + lm;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int tc = b_block_row<GATED, NJ>(wn, j) + g * 8 + lh * 4;
            bool in_range;
            tile_col<GATED>(ep, n0, tc, in_range);
            if (in_range && m0 + r < ep.M) {
              float h[4], b[4];
              unpack_bias4(bv[j][g], b);
#pragma unroll
              for (int q = 0; q < 4; ++q) h[q] = hval<BIAS_IN_ACC>(acc[i][j][4 * g + q], scale_a, b[q]);
              round_bf16x4(h);
#pragma unroll
              for (int q = 0; q < 4; ++q) lmax = fmaxf(lmax, fabsf(act_fwd<ACT>(h[q])));
            }
          }
        }
      }
    }
  }
  if constexpr (AMAX) {
    __shared__ float red[NT / 64];
    block_max_atomic(lmax, ep.amax, red);
  }
}

}  // namespace te
