// fp32 GEMM with the fused bias / activation / gate epilogue, for the
// full-precision path (fp32 inputs, fp32 products and accumulation). A
// 256-thread workgroup computes a 64 x 64 output tile (for gated
// activations, 64 first-half and the matching 64 second-half columns) with
// LDS-staged 16-deep k slices; each thread owns a 4 x 4 block.
//
// Source: "NVIDIA TransformerEngine JAX LayerNorm MLP", Description steps
// (2)-(4); "... LayerNorm Dense", Outputs (x @ kernel + bias).
#include "te_common.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int T = 64, TK = 16;

struct F32Args {
  const float* A;
  const float* B;
  const float* bias;
  float* out;
  float* h_out;
  int M, NB, K, F;
};

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H>
__global__ void __launch_bounds__(256) gemm_f32_kernel(F32Args a) {
  constexpr int G = GATED ? 2 : 1;
  __shared__ float As[TK][T + 4];
  __shared__ float Bs[G][TK][T + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * T, j0 = blockIdx.x * T;
  const int ncols = GATED ? a.F : a.NB;
  float acc[G][4][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[h][r][c] = 0.0f;

  for (int k0 = 0; k0 < a.K; k0 += TK) {
    {  // A: 64 rows x 16 k, one float4 per thread
      const int r = tid >> 2, k = (tid & 3) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m0 + r < a.M && k0 + k < a.K) v = *reinterpret_cast<const float4*>(a.A + (int64_t)(m0 + r) * a.K + k0 + k);
      As[k][r] = v.x; As[k + 1][r] = v.y; As[k + 2][r] = v.z; As[k + 3][r] = v.w;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {  // B: 16 k x 64 columns, one float4 per thread
      const int k = tid >> 4, c = (tid & 15) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + c < ncols && k0 + k < a.K)
        v = *reinterpret_cast<const float4*>(a.B + (int64_t)(k0 + k) * a.NB + h * a.F + j0 + c);
      *reinterpret_cast<float4*>(&Bs[h][k][c]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = As[kk][ty * 4 + r];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 bv = *reinterpret_cast<const float4*>(&Bs[h][kk][tx * 4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[h][r][0] = fmaf(av[r], bv.x, acc[h][r][0]);
          acc[h][r][1] = fmaf(av[r], bv.y, acc[h][r][1]);
          acc[h][r][2] = fmaf(av[r], bv.z, acc[h][r][2]);
          acc[h][r][3] = fmaf(av[r], bv.w, acc[h][r][3]);
        }
      }
    }
    __syncthreads();
  }

  const int col = j0 + tx * 4;
  if (col >= ncols) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + ty * 4 + r;
    if (m >= a.M) continue;
    float hv[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        hv[h][c] = acc[h][r][c] + (a.bias != nullptr ? a.bias[h * a.F + col + c] : 0.0f);
    if constexpr (STORE_H) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        *reinterpret_cast<float4*>(a.h_out + (int64_t)m * a.NB + h * a.F + col) =
            make_float4(hv[h][0], hv[h][1], hv[h][2], hv[h][3]);
    }
    if constexpr (STORE_OUT) {
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = GATED ? act_fwd<ACT>(hv[0][c]) * hv[G - 1][c] : act_fwd<ACT>(hv[0][c]);
      *reinterpret_cast<float4*>(a.out + (int64_t)m * ncols + col) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <int ACT, bool GATED>
hipError_t launch_flags(const F32Args& a, dim3 grid, hipStream_t s) {
  if (a.h_out != nullptr) {
    if (a.out != nullptr) launch_kernel(gemm_f32_kernel<ACT, GATED, true, true>, grid, 256, 0, s, a);
    else launch_kernel(gemm_f32_kernel<ACT, GATED, false, true>, grid, 256, 0, s, a);
  } else {
    launch_kernel(gemm_f32_kernel<ACT, GATED, true, false>, grid, 256, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(const float* A, const float* B, int64_t M, int64_t n_b, int64_t K,
                           const Epilogue& e, hipStream_t s) {
  LaunchScope scope("gemm_f32", s);
  F32Args a{A, B, reinterpret_cast<const float*>(e.bias), reinterpret_cast<float*>(e.out),
            reinterpret_cast<float*>(e.h_out), (int)M, (int)n_b, (int)K,
            e.gated ? (int)(n_b / 2) : (int)n_b};
  const int ncols = a.F;
  const dim3 grid((unsigned)((ncols + T - 1) / T), (unsigned)((M + T - 1) / T));
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
