// bf16 MFMA GEMM for gfx950 with the fused bias / activation / gate epilogue:
// GEMM1 + bias1 + activation and GEMM2 + bias2 of the feed-forward sublayer
// ("NVIDIA TransformerEngine JAX LayerNorm MLP", Description steps (2)-(4))
// and the dense layer of "... LayerNorm Dense" (Outputs: x @ kernel + bias).
//
// A is [M, K] row-major (K contiguous); B is the page's kernel layout
// [K, N] row-major (N contiguous). Both tiles of a BK-deep k stage move from
// memory to LDS with buffer_load ... lds (no register staging): the A tile
// as 256 rows of 2 BK bytes, the B tile as BK k-rows of 512 bytes, each with
// its 16-byte chunks XOR-swizzled per row so that the reads below hit
// distinct banks. The MFMA (v_mfma_f32_32x32x16_bf16) wants 8 consecutive k
// per lane for both operands: A fragments are plain ds_read_b128 of a row,
// B fragments are two ds_read_b64_tr_b16 (4 k each) that transpose the
// N-contiguous tile on the way out of LDS. STAGES LDS stages (128 KiB in
// all): the loads of the next STAGES - 1 stages are in flight while the
// MFMAs of the current one run; one barrier per stage.
//
// With AT, A is given transposed, A^T [K, M] row-major (M contiguous): the
// weight-gradient GEMMs of the backward, x^T @ dY, whose operands are both
// stored token-major. The A tile is then loaded and read exactly like the B
// tile (k-rows of 256 values, transposing reads).
//
// A tiled A (the tiled GEMM operand layout of te_kernels.hpp, written by the
// library's own normalisation or the previous GEMM's epilogue) holds every
// stage's A tile as one 16 KiB block in its LDS image: each wave's loads of
// a stage read one contiguous KiB each, at the block's offset.
#include "gemm_common.hpp"
#include "gemm_lds.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int K;
  int a_tiled;     // A in the tiled operand layout (not with AT)
  EpiArgs ep;
};

// Tile sizes of one pipeline stage of depth BK: A is 256 rows of BK bf16
// (CPR 16-byte chunks per row), B is BK k-rows of 256 bf16 (32 chunks per row).
template <int BK>
struct Stage {
  static constexpr int CPR = BK / 8;
  static constexpr int A_BYTES = kTileM * BK * 2;
  static constexpr int B_BYTES = BK * kTileN * 2;
  static constexpr int BYTES = A_BYTES + B_BYTES;
};

// B k-row kr keeps its 32 chunks (8 n each) at slots q ^ swz_b(kr). A
// ds_read_b64_tr_b16 served 32 lanes at a time reads 4 consecutive k-rows x
// 4 chunks; XOR with 4 (kr & 3) puts the four rows' chunks in four disjoint
// quarters of the 64 banks.
__device__ __forceinline__ int swz_b(int kr) { return (kr & 3) << 2; }

template <int ACT, bool GATED, bool STORE_OUT, bool STORE_H, bool AMAX, int WAVES, int BK, int STAGES, bool PP,
          bool AT, bool OUT_F32 = false>
__global__ void __launch_bounds__(64 * WAVES, 1) gemm_bf16_kernel(GemmArgs a) {
  using St = Stage<BK>;
  constexpr int NJ = 16 / WAVES;                      // 32-column blocks per wave
  constexpr int RA = kTileM / WAVES;                  // A rows loaded per wave
  constexpr int LA = RA * St::CPR * 16 / 1024;        // 1 KiB A loads per wave and stage
  constexpr int RB = BK / WAVES;                      // B k-rows loaded per wave
  constexpr int LB = RB / 2;                          // 1 KiB B loads per wave and stage
  static_assert(LA >= 1 && LB >= 1, "tile too small for the wave count");
  static_assert(!AT || LA == LB, "a transposed A tile is loaded like the B tile");
  // one array per stage: distinct objects let the compiler see that the LDS-DMA
  // of a later stage cannot alias the reads of the current one (no vmcnt wait)
  __shared__ __attribute__((aligned(1024))) uint8_t sm0[St::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sm1[St::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t sm2[STAGES > 2 ? St::BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sm3[STAGES > 3 ? St::BYTES : 16];
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 stages");
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

  // ---- loaders: wave w fills A rows [w RA, (w + 1) RA) (AT: A k-rows [w RB,
  // (w + 1) RB)) and B k-rows [w RB, (w + 1) RB)
  const int rows_a = min(M - m0, kTileM);
  // tiled A: the tile's blocks, one per k stage (a stage is one block: 256 rows of 2 BK = 64 bytes)
  static_assert(AT || BK * 2 == 64, "the tiled layout's stages are 64 bytes per row");
  const bool a_tiled = !AT && a.a_tiled != 0;
  const uint32_t nks_a = (uint32_t)(K + BK - 1) / BK;
  const __amdgpu_buffer_rsrc_t rsrc_a =
      AT ? make_rsrc(a.A, (uint32_t)K * M * 2)
         : a_tiled ? make_rsrc(reinterpret_cast<const uint8_t*>(a.A) + ((int64_t)tm * nks_a << kTiledBlockShift),
                               nks_a << kTiledBlockShift)
                   : make_rsrc(a.A + (int64_t)m0 * K, (uint32_t)rows_a * K * 2);
  // soffset bytes per k value: a whole block per stage when tiled
  const uint32_t kstride_a = a_tiled ? (uint32_t)kTileM * 2 : 2u;
  uint32_t off_a[LA];
  int kc_a[LA];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    if constexpr (AT) {
      // columns past M read the next k-row (finite data; those output rows are not stored)
      const int kr = wave * RB + j * 2 + (lane >> 5);
      const int q = (lane & 31) ^ swz_b(kr);
      off_a[j] = (uint32_t)kr * M * 2 + (uint32_t)(m0 + 8 * q) * 2;
      kc_a[j] = kr;
    } else {
      const int r = wave * RA + j * (64 / St::CPR) + lane / St::CPR;
      const int c = (lane % St::CPR) ^ chunk_swizzle<St::CPR>(r);
      // tiled: the block holds slot lane % CPR of row r at 64 r + 16 (lane % CPR) (rows past M read zero)
      off_a[j] = a_tiled ? (r < rows_a ? (uint32_t)(r * 64 + (lane % St::CPR) * 16) : kOffNone)
                         : (uint32_t)r * K * 2 + c * 16;
      kc_a[j] = c * 8;
    }
  }
  // the whole B operand (K * NB * 2 < 2^31 bytes, checked by the launcher)
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(a.B, (uint32_t)K * NB * 2);
  uint32_t off_b[LB];
  int kr_b[LB];
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int kr = wave * RB + j * 2 + (lane >> 5);
    kr_b[j] = kr;
    const int q = (lane & 31) ^ swz_b(kr);
    int n;
    if constexpr (GATED) n = q < 16 ? n0 + 8 * q : F + n0 + 8 * (q - 16);
    else n = n0 + 8 * q;
    off_b[j] = (uint32_t)kr * NB * 2 + n * 2;
  }
  auto issue_stage = [&](int kt, int s) {
    const int k0 = kt * BK;
    uint8_t* As = stage_ptr(s);
    uint8_t* Bs = As + St::A_BYTES;
    const bool tail = k0 + BK > K;
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      if constexpr (AT) {
        const uint32_t v = k0 + kc_a[j] >= K ? kOffNone : off_a[j];
        load_lds16(rsrc_a, As + wave * RB * 512 + j * 1024, v, (uint32_t)k0 * M * 2);
      } else {
        const uint32_t v = (tail && k0 + kc_a[j] >= K) ? kOffNone : off_a[j];
        load_lds16(rsrc_a, As + wave * RA * BK * 2 + j * 1024, v, (uint32_t)k0 * kstride_a);
      }
    }
    // k-rows at or past K (including whole stages past the end) read as zero:
    // their lanes take an offset beyond the range, so the check fails on the
    // per-lane offset alone
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const uint32_t v = k0 + kr_b[j] >= K ? kOffNone : off_b[j];
      load_lds16(rsrc_b, Bs + wave * RB * 512 + j * 1024, v, (uint32_t)k0 * NB * 2);
    }
  };

  // ---- fragment addresses (byte offsets inside a stage)
  const int lr = lane & 31, lh = lane >> 5;
  int a_off[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk)
    a_off[kk] = (wm * 128 + lr) * BK * 2 + 16 * ((2 * kk + lh) ^ chunk_swizzle<St::CPR>(lr));
  const int g = lane >> 4, i4 = (lane >> 2) & 3, c4 = lane & 3;
  // transposing-read offset of the 32-value block starting at column `base`
  // of a k-row tile (B, and A with AT)
  auto tr_off = [&](int base) {
    const int v = base + 16 * (g & 1) + 4 * c4;
    return (8 * (g >> 1) + i4) * 512 + 16 * ((v >> 3) ^ swz_b(i4)) + 8 * (c4 & 1);
  };
  int at_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) at_off[i] = tr_off(wm * 128 + i * 32);
  int b_off[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n_local = b_block_row<GATED, NJ>(wn, j) + 16 * (g & 1) + 4 * c4;
    b_off[j] = St::A_BYTES + (8 * (g >> 1) + i4) * 512 + 16 * ((n_local >> 3) ^ swz_b(i4)) + 8 * (c4 & 1);
  }

  // the bias starts the accumulation (h = bias + the products, in fp32), so
  // no bias registers stay live through the main loop and the epilogue has
  // no add per value. Its loads go out right after the first stage's DMA
  // (which they would otherwise hold back), and the wait for that stage
  // covers them.
  uint2 bv[NJ][4];
  f32x16_t acc[4][NJ];
  auto start_from_bias = [&]() {
    load_bias_frag<GATED, NJ>(a.ep, n0, wn, lane, bv);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float b[4];
        unpack_bias4(bv[j][g], b);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][4 * g + q] = b[q];
      }
  };

  // ---- one k-substep: fragment reads and the MFMAs that consume them
  constexpr int KS = BK / 16;                         // substeps per stage
  static_assert(KS == 2, "the step schedule below splits a stage into two substeps");
  struct Frags {
    bf16x8_t a[4];
    bf16x8_t b[NJ];
  };
  auto read_frags = [&](int s, int kk, Frags& f) {
    const uint8_t* S = stage_ptr(s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (AT) {
        const i16x4_t lo = lds_read_tr16(S + at_off[i] + (16 * kk) * 512);
        const i16x4_t hi = lds_read_tr16(S + at_off[i] + (16 * kk + 4) * 512);
        f.a[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        f.a[i] = *reinterpret_cast<const bf16x8_t*>(S + a_off[kk] + i * 32 * BK * 2);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const i16x4_t lo = lds_read_tr16(S + b_off[j] + (16 * kk) * 512);
      const i16x4_t hi = lds_read_tr16(S + b_off[j] + (16 * kk + 4) * 512);
      f.b[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  // interleave one fragment read after each MFMA (4 A + 2 NJ B reads, 4 NJ MFMAs)
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < 4 + 2 * NJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
  };

  const int nk = (K + BK - 1) / BK;
  static_assert(STAGES == 4, "three stages ahead of the one being consumed");
  if constexpr (PP) {
    // ---- ping-pong pipeline. Waves 0-3 and 4-7 form two groups with one
    // wave of each on every SIMD. Each wave alternates a memory phase M(t)
    // (all fragment reads of stage t, its share of the DMA of stage t+3, then
    // waits) and a compute phase C(t) (the stage's 16 MFMAs), with a barrier
    // after each. Group 1 starts one phase late, so on every SIMD one wave
    // issues MFMAs while the other feeds LDS and registers.
    //   phase 2t:   group 0 M(t),  group 1 C(t-1)
    //   phase 2t+1: group 0 C(t),  group 1 M(t)
    // The DMA of M(t) refills the buffer of stage t-1, last read by group 1 in
    // phase 2t-1 and waited for (lgkmcnt 0) before that phase's barrier. The
    // wait at the end of M(t) completes the wave's share of stage t+1 (two
    // newer stages stay in flight); both groups' shares of stage t+1 are then
    // complete before phase 2t+2, where it is first read.
    const bool late = wave >= WAVES / 2;
    Frags fa, fb;
    issue_stage(0, 0);
    start_from_bias();
#pragma unroll
    for (int s = 1; s < STAGES - 1; ++s) issue_stage(s, s);
    wait_vmcnt<(STAGES - 2) * (LA + LB)>();
    block_barrier();
    if (late) block_barrier();
    auto pp_step = [&](int kt, int s) {
      // the fragment reads go out before the DMA: issuing the LDS-DMA first
      // held the reads back (and the phase's MFMAs with them) by ~100 clocks
      // per stage
      read_frags(s, 0, fa);
      read_frags(s, 1, fb);
      __builtin_amdgcn_sched_barrier(0);
      issue_stage(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
      wait_vmcnt_lgkm0<(STAGES - 2) * (LA + LB)>();
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      mfmas(fa);
      mfmas(fb);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      block_barrier();
    };
    int kb = 0;
    for (; kb + STAGES <= nk; kb += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) pp_step(kb + s, s);
    }
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (kb + s < nk) pp_step(kb + s, s);
    if (!late) block_barrier();   // the same number of barriers in both groups
  } else {
    // ---- interleaved pipeline. Step kt, with stage kt's first-substep fragments in f0:
    //   MFMAs(f0) || reads of f1 (stage kt, second substep)
    //   wait: own LDS reads and the DMA of stage kt+1; barrier (all waves)
    //   DMA of stage kt+3 into the buffer of stage kt-1 (no longer read)
    //   MFMAs(f1) || reads of f0 for stage kt+1
    // Every step issues exactly one stage (past K it reads nothing), so the
    // wait before the barrier always leaves the newest STAGES - 3 stages in flight.
    Frags f0, f1;
    auto step = [&](int kt, int s) {
      read_frags(s, 1, f1);
      mfmas(f0);
      interleave();
      wait_vmcnt_lgkm0<(STAGES - 3) * (LA + LB)>();
      block_barrier();
      issue_stage(kt + STAGES - 1, (s + STAGES - 1) % STAGES);
      __builtin_amdgcn_sched_group_barrier(0x020, LA + LB, 0);   // the DMA goes out first
      read_frags((s + 1) % STAGES, 0, f0);
      mfmas(f1);
      interleave();
    };
    issue_stage(0, 0);
    start_from_bias();
#pragma unroll
    for (int s = 1; s < STAGES - 1; ++s) issue_stage(s, s);
    wait_vmcnt<(STAGES - 2) * (LA + LB)>();
    block_barrier();
    read_frags(0, 0, f0);
    int kb = 0;
    for (; kb + STAGES <= nk; kb += STAGES) {
#pragma unroll
      for (int s = 0; s < STAGES; ++s) step(kb + s, s);
    }
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (kb + s < nk) step(kb + s, s);
  }
  wait_vmcnt<0>();   // no LDS-DMA may still be writing when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);

  gemm_epilogue<ACT, GATED, STORE_OUT, STORE_H, AMAX, NJ, 64 * WAVES, OUT_F32, true>(acc, bv, a.ep, m0, n0, wm, wn, lane,
                                                                                   tid, 1.0f, stage_ptr);
}

constexpr int kWaves = TE_GEMM_WAVES;
constexpr int kBK = TE_GEMM_BK;
constexpr int kStages = TE_GEMM_STAGES;
constexpr bool kPingPong = TE_GEMM_PINGPONG != 0;

template <int ACT, bool GATED>
hipError_t launch_flags(const GemmArgs& a, unsigned grid, hipStream_t s) {
  const bool out = a.ep.out != nullptr, h = a.ep.h_out != nullptr, amax = a.ep.amax != nullptr;
  constexpr int T = 64 * kWaves;
  if (amax) {
    if (h) launch_kernel(gemm_bf16_kernel<ACT, GATED, false, true, true, kWaves, kBK, kStages, kPingPong, false>, grid, T, 0, s, a);
    else launch_kernel(gemm_bf16_kernel<ACT, GATED, false, false, true, kWaves, kBK, kStages, kPingPong, false>, grid, T, 0, s, a);
  } else if (h) {
    if (out) launch_kernel(gemm_bf16_kernel<ACT, GATED, true, true, false, kWaves, kBK, kStages, kPingPong, false>, grid, T, 0, s, a);
    else launch_kernel(gemm_bf16_kernel<ACT, GATED, false, true, false, kWaves, kBK, kStages, kPingPong, false>, grid, T, 0, s, a);
  } else {
    launch_kernel(gemm_bf16_kernel<ACT, GATED, true, false, false, kWaves, kBK, kStages, kPingPong, false>, grid, T, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_at(const void* At, const void* B, int64_t M, int64_t n_b, int64_t K, const Epilogue& e,
                               hipStream_t s) {
  if (e.act != kLinear || e.gated || e.h_out != nullptr || e.amax != nullptr) return hipErrorInvalidValue;
  LaunchScope scope("gemm_bf16_wgrad", s);
  GemmArgs a;
  a.A = reinterpret_cast<const uint16_t*>(At);
  a.B = reinterpret_cast<const uint16_t*>(B);
  a.K = (int)K;
  a.a_tiled = 0;
  a.ep.bias = reinterpret_cast<const uint16_t*>(e.bias);
  a.ep.out = reinterpret_cast<uint16_t*>(e.out);
  a.ep.h_out = nullptr;
  a.ep.amax = nullptr;
  a.ep.M = (int)M;
  a.ep.n_b = (int)n_b;
  a.ep.F = (int)n_b;
  a.ep.group = 8;
  a.ep.out_nks = 0;
  const unsigned grid = (unsigned)(((M + kTileM - 1) / kTileM) * ((n_b + kTileN - 1) / kTileN));
  launch_kernel(gemm_bf16_kernel<kLinear, false, true, false, false, kWaves, kBK, kStages, kPingPong, true>, grid, 64 * kWaves, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const void* A, const void* B, int64_t M, int64_t n_b, int64_t K,
                            const Epilogue& e, hipStream_t s, bool a_tiled) {
  LaunchScope scope(e.name != nullptr ? e.name
                                      : e.gated ? "gemm_bf16_gated" : (e.act == kLinear ? "gemm_bf16" : "gemm_bf16_act"),
                    s);
  GemmArgs a;
  a.A = reinterpret_cast<const uint16_t*>(A);
  a.B = reinterpret_cast<const uint16_t*>(B);
  a.K = (int)K;
  a.a_tiled = a_tiled ? 1 : 0;
  a.ep.bias = reinterpret_cast<const uint16_t*>(e.bias);
  a.ep.out = reinterpret_cast<uint16_t*>(e.out);
  a.ep.h_out = reinterpret_cast<uint16_t*>(e.h_out);
  a.ep.amax = e.amax;
  a.ep.M = (int)M;
  a.ep.n_b = (int)n_b;
  a.ep.F = e.gated ? (int)(n_b / 2) : (int)n_b;
  a.ep.out_nks = e.out_tiled ? (int)tiled_stages((int64_t)a.ep.F * 2) : 0;
  if (e.out_tiled && (e.out_f32 || e.out == nullptr || (int64_t)a.ep.F * 2 > kTiledMaxRowBytes))
    return hipErrorInvalidValue;
  if (a_tiled && K * 2 > kTiledMaxRowBytes) return hipErrorInvalidValue;
  const int64_t tiles_m = (M + kTileM - 1) / kTileM;
  const int64_t tiles_n = e.gated ? (n_b / 2 + 127) / 128 : (n_b + kTileN - 1) / kTileN;
  a.ep.group = tile_group(tiles_n, false, e.gated);
  const unsigned grid = (unsigned)(tiles_m * tiles_n);
  if (e.out_f32) {
    if (e.act != kLinear || e.gated || e.h_out != nullptr || e.amax != nullptr || e.out == nullptr)
      return hipErrorInvalidValue;
    launch_kernel(gemm_bf16_kernel<kLinear, false, true, false, false, kWaves, kBK, kStages, kPingPong, false, true>,
                  grid, 64 * kWaves, 0, s, a);
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

}  // namespace te
