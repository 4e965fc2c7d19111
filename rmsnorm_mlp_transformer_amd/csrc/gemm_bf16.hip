// bf16 MFMA GEMM for gfx950 with the fused bias / activation / gate epilogue:
// GEMM1 + bias1 + activation and GEMM2 + bias2 of the feed-forward sublayer
// ("NVIDIA TransformerEngine JAX LayerNorm MLP", Description steps (2)-(4))
// and the dense layer of "... LayerNorm Dense" (Outputs: x @ kernel + bias).
//
// A is [M, K] row-major (K contiguous); B is the page's kernel layout
// [K, N] row-major (N contiguous). Both tiles of a 64-deep k stage move from
// memory to LDS with buffer_load ... lds (no register staging): the A tile
// as 256 rows of 128 bytes, the B tile as 64 k-rows of 512 bytes, each with
// its 16-byte chunks XOR-swizzled per row so that the reads below hit
// distinct banks. The MFMA (v_mfma_f32_32x32x16_bf16) wants 8 consecutive k
// per lane for both operands: A fragments are plain ds_read_b128 of a row,
// B fragments are two ds_read_b64_tr_b16 (4 k each) that transpose the
// N-contiguous tile on the way out of LDS. Two LDS stages (128 KiB): the
// loads of stage k+1 are in flight while the MFMAs of stage k run; one
// barrier per stage.
#include "gemm_common.hpp"
#include "gemm_lds.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int BK = 64;                          // k per stage
constexpr int A_BYTES = kTileM * BK * 2;        // 256 rows x 128 B
constexpr int B_BYTES = BK * kTileN * 2;        // 64 k-rows x 512 B
constexpr int STAGE = A_BYTES + B_BYTES;        // 64 KiB

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int K;
  EpiArgs ep;
};

// A row r keeps its 8 chunks (8 k each) at slots c ^ swz_a(r).
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }
// B k-row kr keeps its 32 chunks (8 n each) at slots q ^ swz_b(kr).
__device__ __forceinline__ int swz_b(int kr) { return (kr & 3) << 1; }

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX>
__global__ void __launch_bounds__(256, 1) gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int M = a.ep.M, K = a.K, NB = a.ep.n_b, F = a.ep.F;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = GATED ? (F + 127) / 128 : (NB + kTileN - 1) / kTileN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTileM;
  const int n0 = GATED ? tn * 128 : tn * kTileN;

  // ---- loaders: wave w fills A rows [64w, 64w + 64) and B k-rows [16w, 16w + 16),
  // 1 KiB (8 A rows / 2 B rows) per instruction j
  const int rows_a = min(M - m0, kTileM);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(a.A + (int64_t)m0 * K, (uint32_t)rows_a * K * 2);
  uint32_t off_a[8];
  int kc_a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_a(r);
    off_a[j] = (uint32_t)r * K * 2 + c * 16;
    kc_a[j] = c * 8;
  }
  uint32_t off_b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kr = wave * 16 + j * 2 + (lane >> 5);
    const int q = (lane & 31) ^ swz_b(kr);
    int n;
    if constexpr (GATED) n = q < 16 ? n0 + 8 * q : F + n0 + 8 * (q - 16);
    else n = n0 + 8 * q;
    off_b[j] = (uint32_t)kr * NB * 2 + n * 2;
  }
  auto issue_stage = [&](int kt, int s) {
    const int k0 = kt * BK;
    uint8_t* As = smem + s * STAGE;
    uint8_t* Bs = As + A_BYTES;
    const bool tail = k0 + BK > K;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = (tail && k0 + kc_a[j] >= K) ? kOffNone : off_a[j];
      load_lds16(rsrc_a, As + wave * 8192 + j * 1024, v, (uint32_t)k0 * 2);
    }
    const int krows = min(K - k0, BK);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(a.B + (int64_t)k0 * NB, (uint32_t)krows * NB * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) load_lds16(rsrc_b, Bs + wave * 8192 + j * 1024, off_b[j], 0);
  };

  // ---- fragment addresses (byte offsets inside a stage)
  const int lr = lane & 31, lh = lane >> 5;
  int a_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    a_off[kk] = (wm * 128 + lr) * 128 + 16 * ((2 * kk + lh) ^ swz_a(lr));
  const int g = lane >> 4, i4 = (lane >> 2) & 3, c4 = lane & 3;
  int b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n_local = b_block_row<GATED>(wn, j) + 16 * (g & 1) + 4 * c4;
    b_off[j] = A_BYTES + (8 * (g >> 1) + i4) * 512 + 16 * ((n_local >> 3) ^ (2 * i4)) + 8 * (c4 & 1);
  }

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  issue_stage(0, 0);
  wait_loads_and_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue_stage(kt + 1, cur ^ 1);
    const uint8_t* S = smem + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(S + a_off[kk] + i * 32 * 128);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const i16x4_t lo = lds_read_tr16(S + b_off[j] + (16 * kk) * 512);
        const i16x4_t hi = lds_read_tr16(S + b_off[j] + (16 * kk + 4) * 512);
        bfr[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    wait_loads_and_barrier();
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
