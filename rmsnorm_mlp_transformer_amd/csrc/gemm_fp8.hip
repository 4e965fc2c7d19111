// fp8 (E4M3 x E4M3) MFMA GEMM for gfx950 with fp32 accumulation and the
// fused epilogue. Used when the quantizer set enables per-tensor current
// scaling: "NVIDIA TransformerEngine JAX LayerNorm Dense" (Description: the
// normalised output and the kernel are quantised, then the GEMM runs) and
// "... LayerNorm MLP" (Description: the same for GEMM1 and GEMM2).
//
// Both operands arrive K-contiguous: A codes [M, K] and B^T codes [n_b, K]
// (the weight quantiser writes the kernel transposed). A 128-deep k stage of
// each operand (256 rows x 128 bytes) moves to LDS with buffer_load ... lds,
// 16-byte chunks XOR-swizzled per row; each lane then reads its 32
// consecutive k bytes per operand with two ds_read_b128 and issues
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 for both operands, unit block
// scales). Two LDS stages (128 KiB), one barrier per stage.
//
// The accumulator is multiplied by scale_inv(A) * scale_inv(B), which the
// kernel derives from the two amax values exactly as the quantisers did.
#include "gemm_common.hpp"
#include "gemm_lds.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int BK = 128;                         // k bytes per stage
constexpr int OP_BYTES = kTileM * BK;           // 256 rows x 128 B per operand
constexpr int STAGE = 2 * OP_BYTES;             // 64 KiB

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* Bt;
  int K;
  const float* amax_a;
  const float* amax_b;
  EpiArgs ep;
};

// Row r keeps its 8 chunks (16 k each) at slots c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX>
__global__ void __launch_bounds__(256, 1) gemm_fp8_kernel(GemmArgs a) {
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

  // ---- loaders: wave w fills rows [64w, 64w + 64) of both tiles, 8 rows per instruction
  const int rows_a = min(M - m0, kTileM);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(a.A + (int64_t)m0 * K, (uint32_t)rows_a * K);
  // B^T rows of this tile: [n0, n0 + 256), or for gated the first-half rows
  // [n0, n0 + 128) (waves 0, 1) and the second-half rows [F + n0, F + n0 + 128) (waves 2, 3)
  int b_row0, b_rows;
  if constexpr (GATED) {
    b_row0 = (wave < 2 ? 0 : F) + n0;
    b_rows = min(F - n0, 128);
  } else {
    b_row0 = n0;
    b_rows = min(NB - n0, kTileN);
  }
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(a.Bt + (int64_t)b_row0 * K, (uint32_t)b_rows * K);
  const int b_first = GATED ? (wave & 1) * 64 : wave * 64;   // first row of this wave inside its part
  uint32_t off_a[8], off_b[8];
  int kc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + j * 8 + (lane >> 3);            // row inside the LDS tile
    const int c = (lane & 7) ^ swz(r);
    off_a[j] = (uint32_t)r * K + c * 16;
    off_b[j] = (uint32_t)(b_first + j * 8 + (lane >> 3)) * K + c * 16;
    kc[j] = c * 16;
  }
  auto issue_stage = [&](int kt, int s) {
    const int k0 = kt * BK;
    uint8_t* As = smem + s * STAGE;
    uint8_t* Bs = As + OP_BYTES;
    const bool tail = k0 + BK > K;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool out = tail && k0 + kc[j] >= K;
      load_lds16(rsrc_a, As + wave * 8192 + j * 1024, out ? kOffNone : off_a[j], (uint32_t)k0);
      load_lds16(rsrc_b, Bs + wave * 8192 + j * 1024, out ? kOffNone : off_b[j], (uint32_t)k0);
    }
  };

  // ---- fragment addresses: 32 k bytes = logical chunks 4 kk + 2 h and + 1
  const int lr = lane & 31, lh = lane >> 5;
  int a_lo[2], a_hi[2], b_lo[4][2], b_hi[4][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = 4 * kk + 2 * lh;
    a_lo[kk] = (wm * 128 + lr) * 128 + 16 * (c ^ swz(lr));
    a_hi[kk] = (wm * 128 + lr) * 128 + 16 * ((c + 1) ^ swz(lr));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = b_block_row<GATED>(wn, j) + lr;
      b_lo[j][kk] = OP_BYTES + row * 128 + 16 * (c ^ swz(lr));
      b_hi[j][kk] = OP_BYTES + row * 128 + 16 * ((c + 1) ^ swz(lr));
    }
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
    for (int kk = 0; kk < 2; ++kk) {
      i32x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(S + a_lo[kk] + i * 32 * 128);
        const uint4 hi = *reinterpret_cast<const uint4*>(S + a_hi[kk] + i * 32 * 128);
        af[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 lo = *reinterpret_cast<const uint4*>(S + b_lo[j][kk]);
        const uint4 hi = *reinterpret_cast<const uint4*>(S + b_hi[j][kk]);
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
    wait_loads_and_barrier();
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
