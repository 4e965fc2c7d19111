// fp8 MFMA GEMM for gfx950 with both operands K-contiguous (E4M3 x E4M3),
// fp32 accumulation and the fused bias / activation / gate / amax epilogue,
// used when the quantizer set enables per-tensor current scaling:
// "NVIDIA TransformerEngine JAX LayerNorm Dense" (Description: the
// normalised output and the kernel are quantised, then the GEMM runs) and
// "... LayerNorm MLP" (Description: the same for GEMM1 and GEMM2). The
// weight quantiser writes the kernel transposed; the accumulator is
// multiplied by scale_inv(A) * scale_inv(B), derived from the two amax
// values exactly as the quantisers did.
//
// A is [M, K] and B^T is [n_b, K], both K-contiguous. Each k stage holds 64
// bytes (64 values) of every tile row for 256 rows of each operand; both
// tiles move HBM -> LDS with buffer_load ... lds (16 bytes per lane, no
// register staging), 16-byte chunks XOR-swizzled per row, and come back with
// conflict-free ds_read_b128: an MFMA (v_mfma_f32_32x32x64_f8f6f4, E4M3 for
// both operands, no block scaling) takes two 16-byte chunks per lane and
// operand.
//
// Either operand may be tiled (the tiled GEMM operand layout of
// te_kernels.hpp, written by the library's own quantisers): a stage's tile
// of that operand is then one 16 KiB block in its LDS image, and each wave's
// loads read one contiguous KiB each.
//
// 256 x 256 output tile per workgroup, 8 waves of 128 x 64, 4 LDS stages
// (128 KiB). Ping-pong schedule: waves 0-3 and 4-7 hold one wave per SIMD
// each and alternate, one phase apart, between a memory phase (all fragment
// reads of the current stage, then their share of the DMA three stages
// ahead) and a compute phase (the stage's MFMAs), so each SIMD's matrix core is fed
// by one wave while the other loads.
#include "gemm_common.hpp"
#include "gemm_lds.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int kWaves = 8;
constexpr int kRowBytes = 64;              // bytes of one tile row per k stage
constexpr int kStages = 4;
constexpr int kCpr = kRowBytes / 16;       // 16-byte chunks per tile row
constexpr int kOpBytes = kTileM * kRowBytes;
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kNJ = 2;                     // 32-column blocks per wave
constexpr int kRowsPerWave = kTileM / kWaves;
constexpr int kLJ = kRowsPerWave * kRowBytes / 1024;   // 1 KiB loads per wave, operand and stage
constexpr int kLoads = 2 * kLJ;                        // per wave and stage

struct FpArgs {
  const uint8_t* A;
  const uint8_t* Bt;
  int K;
  int a_tiled, b_tiled;     // operand in the tiled layout (B^T gated: split F)
  const float* amax_a;      // amaxes of the two quantised operands
  const float* amax_b;
  EpiArgs ep;
};

struct Frags {        // one 64-k step: [row block] / [column block]
  i32x8_t a[4];
  i32x8_t b[kNJ];
};

__device__ __forceinline__ i32x8_t join16x2(const uint4& lo, const uint4& hi) {
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX, bool OUT_F32 = false>
__global__ void __launch_bounds__(64 * kWaves, 1) gemm_bt_kernel(FpArgs a) {
  constexpr int E = 1;                     // bytes per element
  constexpr int KE = kRowBytes / E;        // k values per stage
  // one array per stage: distinct objects let the compiler see that the
  // LDS-DMA of a later stage cannot alias the reads of the current one
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sm2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sm3[kStageBytes];
  auto stage_ptr = [&](int s) -> uint8_t* { return s == 0 ? sm0 : s == 1 ? sm1 : s == 2 ? sm2 : sm3; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wm = wave & 1, wn = wave >> 1;
  const int M = a.ep.M, K = a.K, NB = a.ep.n_b, F = a.ep.F;
  const int tiles_m = (M + kTileM - 1) / kTileM;
  const int tiles_n = GATED ? (F + 127) / 128 : (NB + kTileN - 1) / kTileN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, a.ep.group, tm, tn);
  const int m0 = tm * kTileM;
  const int n0 = GATED ? tn * 128 : tn * kTileN;
  const uint32_t pitch = (uint32_t)K * E;  // bytes per operand row (< 2^31, checked by the caller)

  // ---- loaders: wave w fills tile rows [w R, (w + 1) R) of both operands
  static_assert(kRowBytes == 64, "the tiled layout's stages are 64 bytes per row");
  const int rows_a = min(M - m0, kTileM);
  const uint32_t nks = (uint32_t)(K * E + kRowBytes - 1) / kRowBytes;   // k stages per tiled row tile
  const __amdgpu_buffer_rsrc_t rsrc_a =
      a.a_tiled ? make_rsrc(a.A + ((int64_t)tm * nks << kTiledBlockShift), nks << kTiledBlockShift)
                : make_rsrc(a.A + (int64_t)m0 * pitch, (uint32_t)rows_a * pitch);
  // B^T rows of this tile: [n0, n0 + 256), or for gated the first-half rows
  // [n0, n0 + 128) (waves 0-3) and the second-half rows [F + n0, F + n0 + 128) (waves 4-7)
  int b_row0, b_rows;
  if constexpr (GATED) {
    b_row0 = (wave < kWaves / 2 ? 0 : F) + n0;
    b_rows = min(F - n0, 128);
  } else {
    b_row0 = n0;
    b_rows = min(NB - n0, kTileN);
  }
  // tiled B^T: block tn holds this tile's rows (gated: the split layout's 128 + 128 rows)
  const __amdgpu_buffer_rsrc_t rsrc_b =
      a.b_tiled ? make_rsrc(a.Bt + ((int64_t)tn * nks << kTiledBlockShift), nks << kTiledBlockShift)
                : make_rsrc(a.Bt + (int64_t)b_row0 * pitch, (uint32_t)b_rows * pitch);
  // soffset bytes per k value: a whole block per stage when tiled
  const uint32_t kstride_a = a.a_tiled ? (uint32_t)kTileM : (uint32_t)E;
  const uint32_t kstride_b = a.b_tiled ? (uint32_t)kTileM : (uint32_t)E;
  const int b_first = GATED ? (wave % (kWaves / 2)) * kRowsPerWave : wave * kRowsPerWave;
  uint32_t off_a[kLJ], off_b[kLJ];
  int kc[kLJ];
#pragma unroll
  for (int j = 0; j < kLJ; ++j) {
    const int r = wave * kRowsPerWave + j * (64 / kCpr) + lane / kCpr;   // row inside the LDS tile
    const int c = (lane % kCpr) ^ chunk_swizzle<kCpr>(r);
    const int rb = b_first + j * (64 / kCpr) + lane / kCpr;              // row of B^T (of its half when gated)
    // tiled: LDS row r's slot lane % kCpr sits at 64 r + 16 (lane % kCpr) of the block; rows
    // past the operand read zero
    const uint32_t tile_off = (uint32_t)(r * kRowBytes + (lane % kCpr) * 16);
    off_a[j] = a.a_tiled ? (r < rows_a ? tile_off : kOffNone) : (uint32_t)r * pitch + c * 16;
    off_b[j] = a.b_tiled ? (rb < b_rows ? tile_off : kOffNone) : (uint32_t)rb * pitch + c * 16;
    kc[j] = c * (16 / E);
  }
  auto issue_stage = [&](int kt, int s) {
    const int k0 = kt * KE;
    uint8_t* As = stage_ptr(s);
    uint8_t* Bs = As + kOpBytes;
    // chunks at or past K (including whole stages past the end) read as zero
#pragma unroll
    for (int j = 0; j < kLJ; ++j) {
      const bool out = k0 + kc[j] >= K;
      load_lds16(rsrc_a, As + wave * kRowsPerWave * kRowBytes + j * 1024, out ? kOffNone : off_a[j],
                 (uint32_t)k0 * kstride_a);
      load_lds16(rsrc_b, Bs + wave * kRowsPerWave * kRowBytes + j * 1024, out ? kOffNone : off_b[j],
                 (uint32_t)k0 * kstride_b);
    }
  };

  // ---- fragment addresses. Lane l reads row l % 32 of its 32-row block; the
  // chunk swizzle of every such row is that of row l % 32.
  const int lr = lane & 31, lh = lane >> 5;
  const int sw = chunk_swizzle<kCpr>(lr);
  int a_off[2], b_off[kNJ][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // the lane's 32 k bytes are chunks 2 lh and 2 lh + 1
    const int c = 2 * lh + h;
    a_off[h] = (wm * 128 + lr) * kRowBytes + 16 * (c ^ sw);
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
      b_off[j][h] = kOpBytes + (b_block_row<GATED, kNJ>(wn, j) + lr) * kRowBytes + 16 * (c ^ sw);
  }

  uint2 bv[kNJ][4];   // the epilogue's bias values, loaded while the main loop runs

  f32x16_t acc[4][kNJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Frags f;
  auto read_frags = [&](int s) {
    const uint8_t* S = stage_ptr(s);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = join16x2(*reinterpret_cast<const uint4*>(S + a_off[0] + i * 32 * kRowBytes),
                        *reinterpret_cast<const uint4*>(S + a_off[1] + i * 32 * kRowBytes));
#pragma unroll
    for (int j = 0; j < kNJ; ++j)
      f.b[j] = join16x2(*reinterpret_cast<const uint4*>(S + b_off[j][0]),
                        *reinterpret_cast<const uint4*>(S + b_off[j][1]));
  };
  // B fragment first: each lane then holds 4 consecutive output columns
  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
        // cbsz/blgp = 0: both operands E4M3. With constant zero scale operands
        // the compiler emits the plain v_mfma_f32_32x32x64_f8f6f4 (no block
        // scaling, checked in the generated code); with unit E8M0 scales (127)
        // it emits the scaled form, whose scale operands cost a register and
        // measured 0.4% slower in GEMM2 (same results).
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
  };

  // ---- ping-pong pipeline.
  //   phase 2t:   group 0 memory M(t),  group 1 compute C(t-1)
  //   phase 2t+1: group 0 compute C(t), group 1 memory M(t)
  // M(t): fragment reads of stage t, DMA of the wave's share of stage t+3
  // into the buffer of stage t-1, then wait for those reads and for the
  // wave's share of stage t+1 (two newer stages stay in flight); barrier.
  // C(t): the stage's MFMAs; barrier.
  // The buffer of stage t-1 was last read by group 1 in phase 2t-1 and those
  // reads completed before that phase's barrier; both groups' shares of stage
  // t+1 are complete before phase 2t+2, where it is first read. Every step
  // issues exactly one stage (past K it reads nothing), so the vmcnt budget is
  // the same in every step, and both groups pass the same number of barriers.
  const bool late = wave >= kWaves / 2;
  const int nk = (K + KE - 1) / KE;
  // the bias loads go out right after the first stage's DMA, which they
  // would otherwise hold back
  issue_stage(0, 0);
  load_bias_frag<GATED, kNJ>(a.ep, n0, wn, lane, bv);
#pragma unroll
  for (int s = 1; s < kStages - 1; ++s) issue_stage(s, s);
  wait_vmcnt<(kStages - 2) * kLoads>();
  block_barrier();
  if (late) block_barrier();
  auto step = [&](int kt, int s) {
    // the fragment reads go out before the DMA (issuing the LDS-DMA first
    // held the reads and the phase's MFMAs back)
    read_frags(s);
    __builtin_amdgcn_sched_barrier(0);
    issue_stage(kt + kStages - 1, (s + kStages - 1) % kStages);
    wait_vmcnt_lgkm0<(kStages - 2) * kLoads>();
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    mfmas();
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    block_barrier();
  };
  int kb = 0;
  for (; kb + kStages <= nk; kb += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) step(kb + s, s);
  }
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (kb + s < nk) step(kb + s, s);
  if (!late) block_barrier();
  wait_vmcnt<0>();   // no LDS-DMA may still be writing when the epilogue reuses the LDS

  const float sa = fp8_scale_from_amax(*a.amax_a), sb = fp8_scale_from_amax(*a.amax_b);
  const float scale = (1.0f / sa) * (1.0f / sb);
  gemm_epilogue<ACT, GATED, STORE_OUT, STORE_H, AMAX, kNJ, 64 * kWaves, OUT_F32>(acc, bv, a.ep, m0, n0, wm, wn, lane,
                                                                                tid, scale, stage_ptr);
}

template <int ACT, bool GATED>
hipError_t launch_flags(const FpArgs& a, unsigned grid, hipStream_t s) {
  const bool out = a.ep.out != nullptr, h = a.ep.h_out != nullptr, amax = a.ep.amax != nullptr;
  constexpr int T = 64 * kWaves;
  if (amax) {
    if (h) launch_kernel(gemm_bt_kernel<ACT, GATED, false, true, true>, grid, T, 0, s, a);
    else launch_kernel(gemm_bt_kernel<ACT, GATED, false, false, true>, grid, T, 0, s, a);
  } else if (h) {
    if (out) launch_kernel(gemm_bt_kernel<ACT, GATED, true, true, false>, grid, T, 0, s, a);
    else launch_kernel(gemm_bt_kernel<ACT, GATED, false, true, false>, grid, T, 0, s, a);
  } else {
    launch_kernel(gemm_bt_kernel<ACT, GATED, true, false, false>, grid, T, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_bt(const void* A, const void* Bt, int64_t M, int64_t n_b, int64_t K, const float* amax_a,
                     const float* amax_b, const Epilogue& e, hipStream_t s, bool a_tiled, bool b_tiled) {
  if (e.out_tiled) return hipErrorInvalidValue;
  if ((a_tiled || b_tiled) && K > kTiledMaxRowBytes) return hipErrorInvalidValue;
  FpArgs a;
  a.A = static_cast<const uint8_t*>(A);
  a.Bt = static_cast<const uint8_t*>(Bt);
  a.K = (int)K;
  a.a_tiled = a_tiled ? 1 : 0;
  a.b_tiled = b_tiled ? 1 : 0;
  a.amax_a = amax_a;
  a.amax_b = amax_b;
  a.ep.bias = static_cast<const uint16_t*>(e.bias);
  a.ep.out = static_cast<uint16_t*>(e.out);
  a.ep.h_out = static_cast<uint16_t*>(e.h_out);
  a.ep.amax = e.amax;
  a.ep.M = (int)M;
  a.ep.n_b = (int)n_b;
  a.ep.F = e.gated ? (int)(n_b / 2) : (int)n_b;
  a.ep.out_nks = 0;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM;
  const int64_t tiles_n = e.gated ? (n_b / 2 + 127) / 128 : (n_b + kTileN - 1) / kTileN;
  a.ep.group = tile_group(tiles_n, true, e.gated);
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  if (e.out_f32) {
    if (e.act != kLinear || e.gated || e.h_out != nullptr || e.amax != nullptr || e.out == nullptr)
      return hipErrorInvalidValue;
    launch_kernel(gemm_bt_kernel<kLinear, false, true, false, false, true>, grid, 64 * kWaves, 0, s, a);
    return hipGetLastError();
  }
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

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* Bt, int64_t M, int64_t n_b, int64_t K,
                           const float* amax_a, const float* amax_b, const Epilogue& e, hipStream_t s,
                           bool a_tiled, bool b_tiled) {
  LaunchScope scope(e.amax != nullptr ? "gemm_fp8_h_amax" : "gemm_fp8", s);
  return launch_bt(A, Bt, M, n_b, K, amax_a, amax_b, e, s, a_tiled, b_tiled);
}

}  // namespace te
