// bf16 MFMA GEMM for gfx950 with the fused bias / activation / gate epilogue:
// GEMM1 + bias1 + activation and GEMM2 + bias2 of the feed-forward sublayer
// ("NVIDIA TransformerEngine JAX LayerNorm MLP", Description steps (2)-(4))
// and the dense layer of "... LayerNorm Dense" (Outputs: x @ kernel + bias).
//
// A is [M, K] row-major (K contiguous); B is the page's kernel layout
// [K, N] row-major (N contiguous). The MFMA (v_mfma_f32_32x32x16_bf16) wants
// 8 consecutive k values per lane for both operands, so B is transposed on
// its way into LDS: each thread loads an 8 (k) x 8 (n) block with eight
// 16-byte loads, transposes it in registers and writes eight 16-byte rows of
// a k-contiguous LDS tile. Both LDS tiles are [256][64 + 8] bf16: the 16-byte
// pad makes the row stride 36 dwords, so the 16 lanes served together by
// ds_read_b128 fall on distinct banks.
//
// Pipeline: two LDS stages of BK = 64; the global loads for stage k+1 are in
// flight while the MFMAs of stage k run, and one barrier per stage separates
// the LDS writes from the reads.
#include "gemm_common.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int BK = 64;
constexpr int LDS_LD = BK + 8;                       // bf16 elements per LDS row
constexpr int STAGE_ELEMS = kTileM * LDS_LD;         // one operand tile

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int K;
  EpiArgs ep;
};

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX>
__global__ void __launch_bounds__(256, 1) gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][STAGE_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int M = a.ep.M, K = a.K, NB = a.ep.n_b, F = a.ep.F;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = GATED ? (F + 127) / 128 : (NB + kTileN - 1) / kTileN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTileM;
  const int n0 = GATED ? tn * 128 : tn * kTileN;

  // A loader: chunk column ac (8 k), rows ar + 32 p
  const int ac = tid & 7, ar = tid >> 3;
  // B loader: k-block bk (8 k), n-block bn (8 n)
  const int bk = tid & 7, bn = tid >> 3;
  int bcol;
  bool bvalid;
  if constexpr (GATED) {
    const int c = n0 + (bn & 15) * 8;
    bvalid = c < F;
    bcol = (bn < 16) ? c : F + c;
  } else {
    bcol = n0 + bn * 8;
    bvalid = bcol < NB;
  }

  uint4 ga[8], gb[8];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int m = m0 + ar + 32 * p, k = k0 + ac * 8;
      ga[p] = (m < M && k < K) ? ldg16(a.A + (int64_t)m * K + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + bk * 8 + i;
      gb[i] = (bvalid && k < K) ? ldg16(a.B + (int64_t)k * NB + bcol) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int s) {
    uint16_t* As = smem[s][0];
    uint16_t* Bs = smem[s][1];
#pragma unroll
    for (int p = 0; p < 8; ++p)
      *reinterpret_cast<uint4*>(As + (ar + 32 * p) * LDS_LD + ac * 8) = ga[p];
    // transpose the 8x8 block: row j of the output = column j of the input
    const uint32_t* g = reinterpret_cast<const uint32_t*>(gb);   // g[i*4 + w] = word w of k-row i
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t x = g[(2 * p) * 4 + j / 2], y = g[(2 * p + 1) * 4 + j / 2];
        w[p] = (j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
      }
      *reinterpret_cast<uint4*>(Bs + (bn * 8 + j) * LDS_LD + bk * 8) = make_uint4(w[0], w[1], w[2], w[3]);
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

  const int lm = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage((kt + 1) * BK);
    const uint16_t* As = smem[cur][0];
    const uint16_t* Bs = smem[cur][1];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 128 + i * 32 + lm) * LDS_LD + kk * 16 + lk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (b_block_row<GATED>(wn, j) + lm) * LDS_LD + kk * 16 + lk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  gemm_epilogue<ACT, GATED, STORE_OUT, STORE_H, AMAX>(acc, a.ep, m0, n0, wm, wn, lane, 1.0f);
}

template <int ACT, bool GATED>
hipError_t launch_flags(const GemmArgs& a, unsigned grid, hipStream_t s) {
  const bool out = a.ep.out != nullptr, h = a.ep.h_out != nullptr, amax = a.ep.amax != nullptr;
  if (amax) {
    if (h) gemm_bf16_kernel<ACT, GATED, false, true, true><<<grid, 256, 0, s>>>(a);
    else gemm_bf16_kernel<ACT, GATED, false, false, true><<<grid, 256, 0, s>>>(a);
  } else if (h) {
    if (out) gemm_bf16_kernel<ACT, GATED, true, true, false><<<grid, 256, 0, s>>>(a);
    else gemm_bf16_kernel<ACT, GATED, false, true, false><<<grid, 256, 0, s>>>(a);
  } else {
    gemm_bf16_kernel<ACT, GATED, true, false, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const void* A, const void* B, int64_t M, int64_t n_b, int64_t K,
                            const Epilogue& e, hipStream_t s) {
  LaunchScope scope(e.gated ? "gemm_bf16_gated" : (e.act == kLinear ? "gemm_bf16" : "gemm_bf16_act"), s);
  GemmArgs a;
  a.A = reinterpret_cast<const uint16_t*>(A);
  a.B = reinterpret_cast<const uint16_t*>(B);
  a.K = (int)K;
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
