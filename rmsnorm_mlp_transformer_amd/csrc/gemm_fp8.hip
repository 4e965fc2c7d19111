// fp8 (E4M3 x E4M3) MFMA GEMM for gfx950 with fp32 accumulation and the
// fused epilogue. Used when the quantizer set enables per-tensor current
// scaling: "NVIDIA TransformerEngine JAX LayerNorm Dense" (Description: the
// normalised output and the kernel are quantised, then the GEMM runs) and
// "... LayerNorm MLP" (Description: the same for GEMM1 and GEMM2).
//
// Both operands arrive K-contiguous: A codes [M, K] and B^T codes [n_b, K]
// (the weight quantiser writes the kernel transposed). One
// v_mfma_scale_f32_32x32x64_f8f6f4 (format E4M3 for both operands, unit
// block scales) consumes 32 consecutive k bytes per lane and operand. LDS
// tiles are [256][128 + 16] bytes per operand and stage (row stride 36
// dwords: conflict-free 16-byte reads), two stages of BK = 128.
//
// The accumulator is multiplied by scale_inv(A) * scale_inv(B), which the
// kernel derives from the two amax values exactly as the quantisers did.
#include "gemm_common.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int BK = 128;                    // bytes (= k values) per stage
constexpr int LDS_LD = BK + 16;            // bytes per LDS row
constexpr int STAGE_BYTES = kTileM * LDS_LD;

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* Bt;
  int K;
  const float* amax_a;
  const float* amax_b;
  EpiArgs ep;
};

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX>
__global__ void __launch_bounds__(256, 1) gemm_fp8_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int M = a.ep.M, K = a.K, NB = a.ep.n_b, F = a.ep.F;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = GATED ? (F + 127) / 128 : (NB + kTileN - 1) / kTileN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTileM;
  const int n0 = GATED ? tn * 128 : tn * kTileN;

  // loader: 16-byte chunk c of 8 per row, rows r + 32 p (same for A and B)
  const int lc = tid & 7, lr = tid >> 3;
  int brow[8];
  bool bval[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = lr + 32 * p;             // LDS row of the B tile
    if constexpr (GATED) {
      const int c = n0 + (r & 127);
      bval[p] = c < F;
      brow[p] = r < 128 ? c : F + c;
    } else {
      brow[p] = n0 + r;
      bval[p] = brow[p] < NB;
    }
  }

  uint4 ga[8], gb[8];
  auto load_stage = [&](int k0) {
    const int k = k0 + lc * 16;
    const bool kv = k < K;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int m = m0 + lr + 32 * p;
      ga[p] = (m < M && kv) ? ldg16(a.A + (int64_t)m * K + k) : make_uint4(0, 0, 0, 0);
      gb[p] = (bval[p] && kv) ? ldg16(a.Bt + (int64_t)brow[p] * K + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int s) {
    uint8_t* As = smem[s][0];
    uint8_t* Bs = smem[s][1];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      *reinterpret_cast<uint4*>(As + (lr + 32 * p) * LDS_LD + lc * 16) = ga[p];
      *reinterpret_cast<uint4*>(Bs + (lr + 32 * p) * LDS_LD + lc * 16) = gb[p];
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int lm = lane & 31, lk = (lane >> 5) * 32;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * BK);
    const uint8_t* As = smem[cur][0];
    const uint8_t* Bs = smem[cur][1];
#pragma unroll
    for (int kk = 0; kk < BK / 64; ++kk) {
      i32x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* p = As + (wm * 128 + i * 32 + lm) * LDS_LD + kk * 64 + lk;
        const uint4 lo = *reinterpret_cast<const uint4*>(p), hi = *reinterpret_cast<const uint4*>(p + 16);
        af[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* p = Bs + (b_block_row<GATED>(wn, j) + lm) * LDS_LD + kk * 64 + lk;
        const uint4 lo = *reinterpret_cast<const uint4*>(p), hi = *reinterpret_cast<const uint4*>(p + 16);
        bfr[j] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          // cbsz/blgp = 0: both operands E4M3; scales 127 = 2^0 (no block scaling)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0,
                                                                       0, 127, 0, 127);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  const float sa = fp8_scale_from_amax(*a.amax_a), sb = fp8_scale_from_amax(*a.amax_b);
  const float scale = (1.0f / sa) * (1.0f / sb);
  gemm_epilogue<ACT, GATED, STORE_OUT, STORE_H, AMAX>(acc, a.ep, m0, n0, wm, wn, lane, scale);
}

template <int ACT, bool GATED>
hipError_t launch_flags(const GemmArgs& a, unsigned grid, hipStream_t s) {
  const bool out = a.ep.out != nullptr, h = a.ep.h_out != nullptr, amax = a.ep.amax != nullptr;
  if (amax) {
    if (h) gemm_fp8_kernel<ACT, GATED, false, true, true><<<grid, 256, 0, s>>>(a);
    else gemm_fp8_kernel<ACT, GATED, false, false, true><<<grid, 256, 0, s>>>(a);
  } else if (h) {
    if (out) gemm_fp8_kernel<ACT, GATED, true, true, false><<<grid, 256, 0, s>>>(a);
    else gemm_fp8_kernel<ACT, GATED, false, true, false><<<grid, 256, 0, s>>>(a);
  } else {
    gemm_fp8_kernel<ACT, GATED, true, false, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* Bt, int64_t M, int64_t n_b, int64_t K,
                           const float* amax_a, const float* amax_b, const Epilogue& e,
                           hipStream_t s) {
  LaunchScope scope(e.amax != nullptr ? "gemm_fp8_h_amax" : "gemm_fp8", s);
  GemmArgs a;
  a.A = A;
  a.Bt = Bt;
  a.K = (int)K;
  a.amax_a = amax_a;
  a.amax_b = amax_b;
  a.ep.bias = reinterpret_cast<const uint16_t*>(e.bias);
  a.ep.out = reinterpret_cast<uint16_t*>(e.out);
  a.ep.h_out = reinterpret_cast<uint16_t*>(e.h_out);
  a.ep.amax = e.amax;
  a.ep.M = (int)M;
  a.ep.n_b = (int)n_b;
  a.ep.F = e.gated ? (int)(n_b / 2) : (int)n_b;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM;
  const int64_t tiles_n = e.gated ? (n_b / 2 + 127) / 128 : (n_b + kTileN - 1) / kTileN;
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
#define TE_G(A_) return e.gated ? launch_flags<A_, true>(a, grid, s) : launch_flags<A_, false>(a, grid, s)
  switch (e.act) {
    case kRelu: TE_G(kRelu);
    case kGelu: TE_G(kGelu);
    case kGeluErf: TE_G(kGeluErf);
    case kSilu: TE_G(kSilu);
    default: TE_G(kLinear);
  }
#undef TE_G
}

}  // namespace te
