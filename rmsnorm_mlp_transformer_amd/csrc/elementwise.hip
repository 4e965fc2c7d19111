// HBM-bound kernels for gfx950: per-tensor amax and E4M3 quantisation
// (current scaling), dequantisation, the activation forward (act_lu) and the
// activation backward with the fused bias-gradient reduction (dact + dbias).
//
// Every kernel moves 16 bytes per lane per access so that one wave touches
// 1 KiB of contiguous memory per load instruction.
//
// Sources: "NVIDIA TransformerEngine JAX Activation" (Description: forward
// activation with optional quantisation, backward activation gradient;
// Outputs: dequantised result); "... LayerNorm MLP" (Description: the fused
// backward gives the activation gradient with the bias reduction);
// "... LayerNorm Dense" (Description: the normalised input and the kernel
// are quantised before the GEMM).
#include "gemm_lds.hpp"
#include "te_common.hpp"
#include "te_kernels.hpp"

namespace te {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void unpack8_bf16(const uint4& c, float* f) {
  f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x); f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
  f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z); f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
}
__device__ __forceinline__ uint4 pack8_bf16(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t e, const float* f) {
  if constexpr (BF16) {
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + e) = pack8_bf16(f);
  } else {
    float* p = reinterpret_cast<float*>(base) + e;
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
}
__device__ __forceinline__ uint2 encode8(const float* f, float scale) {
  return make_uint2(e4m3_pack4(f[0] * scale, f[1] * scale, f[2] * scale, f[3] * scale),
                    e4m3_pack4(f[4] * scale, f[5] * scale, f[6] * scale, f[7] * scale));
}

// Products and sums that must round the same way in every kernel that forms
// them (the dact variants must give bitwise equal bias gradients): no fusion
// into an fma.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Raw buffer access (32-bit byte offsets inside one descriptor): a lane's
// offset plus a wave-uniform soffset, so that the unrolled row loop costs no
// 64-bit address arithmetic. Accesses at or past the descriptor's size read
// zeros and are dropped when storing.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc buf_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 8 elements as raw 16-byte words (bf16: one, fp32: two), unpacked later so
// that a wave can keep all of its loads in flight before the first use.
template <bool BF16>
struct Raw8 {
  i32x4_t w[BF16 ? 1 : 2];
};
template <bool BF16>
__device__ __forceinline__ void load8_raw(Rsrc r, uint32_t voff, uint32_t soff, Raw8<BF16>& d) {
  d.w[0] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kBufAuxStream);
  if constexpr (!BF16) d.w[1] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, kBufAuxStream);
}
template <bool BF16>
__device__ __forceinline__ void unpack8_raw(const Raw8<BF16>& d, float* f) {
  if constexpr (BF16) {
    unpack8_bf16(make_uint4((uint32_t)d.w[0][0], (uint32_t)d.w[0][1], (uint32_t)d.w[0][2], (uint32_t)d.w[0][3]), f);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = __int_as_float(d.w[0][i]); f[4 + i] = __int_as_float(d.w[1][i]); }
  }
}
// The same from a plain pointer (element offset e).
template <bool BF16>
__device__ __forceinline__ void load8_raw_ptr(const void* base, int64_t e, Raw8<BF16>& d) {
  const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + e * (BF16 ? 2 : 4);
  const uint4 a = load_stream16(p);
  d.w[0] = i32x4_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  if constexpr (!BF16) {
    const uint4 b = load_stream16(p + 16);
    d.w[1] = i32x4_t{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
}
// Stores fold the row offset into the lane offset and pass a zero soffset:
// a 16-byte store whose data registers a VALU instruction rewrites right
// after it needs one wait state, and the compiler only inserts it for stores
// without a register soffset (with one, lanes 12-15 of each 16 were seen to
// store the rewritten values).
// AUX is the store's cache-policy operand (0, or kStoreAuxNt: the nt hint).
constexpr int kStoreAuxNt = 2;
template <bool BF16, int AUX = 0>
__device__ __forceinline__ void store8_buf(Rsrc r, uint32_t voff, uint32_t soff, const float* f) {
  const uint32_t o = voff + soff;
  if constexpr (BF16) {
    const uint4 v = pack8_bf16(f);
    const i32x4_t w = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, o, 0, AUX);
  } else {
    const i32x4_t a = {__float_as_int(f[0]), __float_as_int(f[1]), __float_as_int(f[2]), __float_as_int(f[3])};
    const i32x4_t b = {__float_as_int(f[4]), __float_as_int(f[5]), __float_as_int(f[6]), __float_as_int(f[7])};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, o, 0, AUX);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, o + 16, 0, AUX);
  }
}
__device__ __forceinline__ void store8_codes_buf(Rsrc r, uint32_t voff, uint32_t soff, uint2 c) {
  typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;
  const i32x2_t w = {(int)c.x, (int)c.y};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, voff + soff, 0, 0);
}

unsigned grid_for(int64_t work_items, int per_thread) {
  int64_t blocks = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
  if (blocks < 1) blocks = 1;
  if (blocks > 65535LL * 16) blocks = 65535LL * 16;
  return (unsigned)blocks;
}

// ------------------------------------------------------------------ fill / meta
__global__ void fill_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

__global__ void fill_zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Metadata of an empty tensor: amax 0, scale 1, scale_inv 1.
__global__ void empty_meta_kernel(float* amax, float* scale, float* scale_inv) {
  if (threadIdx.x == 0) {
    *amax = 0.0f;
    *scale = 1.0f;
    *scale_inv = 1.0f;
  }
}

// ------------------------------------------------------------------ amax
// n is a multiple of 8 (every tensor size here is a multiple of 16). Each
// lane keeps kUnroll 16-byte loads in flight per iteration.
constexpr int kUnroll = 8;

// One tensor of an amax pass: n8 chunks of 8 elements, its own amax slot.
struct AmaxJob {
  const void* x;
  int64_t n8;
  float* amax;
};

// Workgroups [0, blocks0) reduce job 0, the rest job 1 (two weights in one
// launch), each set looping over its tensor.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) amax_kernel(AmaxJob j0, AmaxJob j1, unsigned blocks0) {
  const bool second = blockIdx.x >= blocks0;
  const AmaxJob& j = second ? j1 : j0;
  const int64_t blk = second ? blockIdx.x - blocks0 : blockIdx.x;
  const int64_t nblk = second ? gridDim.x - blocks0 : blocks0;
  const void* x = j.x;
  const int64_t n8 = j.n8;
  float m = 0.0f;
  const int64_t stride = nblk * kThreads;
  for (int64_t c0 = blk * kThreads + threadIdx.x; c0 < n8; c0 += stride * kUnroll) {
    // chunks past the end re-read the last one (no change to the max), so
    // every load is unconditional and all are in flight before the first use
    Raw8<BF16> w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load8_raw_ptr<BF16>(x, min(c0 + u * stride, n8 - 1) * 8, w[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float f[8];
      unpack8_raw<BF16>(w[u], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    }
  }
  __shared__ float red[kThreads / 64];
  block_max_atomic(m, j.amax, red);
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) quantize_kernel(const void* x, int64_t n8, uint8_t* codes,
                                                            const float* amax, float* scale_out,
                                                            float* scale_inv_out) {
  const float scale = fp8_scale_from_amax(*amax);
  if (blockIdx.x == 0 && threadIdx.x == 0 && scale_out != nullptr) {
    *scale_out = scale;
    *scale_inv_out = 1.0f / scale;
  }
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < n8; c0 += stride * U) {
    // unconditional loads (past the end: the last chunk again), all in flight
    // before the first use; only the stores are guarded
    Raw8<BF16> w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load8_raw_ptr<BF16>(x, min(c0 + u * stride, n8 - 1) * 8, w[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * stride;
      float f[8];
      unpack8_raw<BF16>(w[u], f);
      if (c < n8) *reinterpret_cast<uint2*>(codes + c * 8) = encode8(f, scale);
    }
  }
}

// Quantise x [rows, cols] into codes_t [cols, rows]. A workgroup takes a
// 128-row x kQtCols-column tile: for each 64-column half, each thread loads 4
// consecutive rows x 8 columns (all 16-byte loads of the tile in flight
// before the first use), encodes them, transposes the 4 x 4 code blocks in
// registers (v_perm_b32) and writes one 4-byte word per column into an LDS
// tile [kQtCols columns][128 rows]; the tile then leaves as kQtCols output
// rows of 128 codes (full 128-byte lines), 16-byte stores.
// 256 columns (four halves, 16 loads per thread in flight): a sweep of
// 64 / 128 / 256 at the 4096 x 16384 and 16384 x 4096 weights took the
// pass over both from 0.0715 to 0.066 ms.
#ifndef TE_QT_COLS
#define TE_QT_COLS 256
#endif
constexpr int kQtRows = 128, kQtCols = TE_QT_COLS;
constexpr int kQtHalves = kQtCols / 64;
static_assert(kQtCols % 64 == 0, "whole 64-column halves");
constexpr int kQtPitch = kQtRows + 4;   // bytes per LDS row: 33 words, odd, spreads the word writes over the banks
// One matrix of a quantise-transpose pass.
struct QtJob {
  const void* x;
  int64_t rows, cols;
  uint8_t* codes_t;
  const float* amax;
  float* scale_out;        // nullable
  float* scale_inv_out;
  int64_t nks, split;      // nks > 0: codes_t in the tiled GEMM operand layout (k stages, split row)
};

// Workgroups [0, tiles0) take the tiles of job 0, the rest those of job 1.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) quantize_transpose_kernel(QtJob j0, QtJob j1, unsigned tiles0) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kQtCols * kQtPitch];
  const bool second = blockIdx.x >= tiles0;
  const QtJob& job = second ? j1 : j0;
  const int64_t blk = second ? blockIdx.x - tiles0 : blockIdx.x;
  const void* x = job.x;
  const int64_t rows = job.rows, cols = job.cols;
  uint8_t* codes_t = job.codes_t;
  const float scale = fp8_scale_from_amax(*job.amax);
  if (blk == 0 && threadIdx.x == 0 && job.scale_out != nullptr) {
    *job.scale_out = scale;
    *job.scale_inv_out = 1.0f / scale;
  }
  const int64_t tiles_c = (cols + kQtCols - 1) / kQtCols;
  const int64_t r0 = (blk / tiles_c) * kQtRows, c0 = (blk % tiles_c) * kQtCols;
  const int t = threadIdx.x;
  // rows 4 rg .. 4 rg + 3, columns cc .. cc + 7 of the tile. Rows or columns
  // outside the matrix re-read a clamped in-range chunk: their codes land in
  // tile cells that are never stored.
  const int rg = t >> 3;
  Raw8<BF16> w[kQtHalves][4];
#pragma unroll
  for (int h = 0; h < kQtHalves; ++h) {
    const int cc = (t & 7) * 8 + 64 * h;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      load8_raw_ptr<BF16>(x, min(r0 + 4 * rg + k, rows - 1) * cols + min(c0 + cc, cols - 8), w[h][k]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // column j of a 4 x 4 block: byte j of rows 0..3 -> one word (row 0 in byte 0)
  auto column = [](const uint32_t (&v)[4], int j) {
    const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 8);
    const uint32_t r01 = __builtin_amdgcn_perm(v[1], v[0], sel);   // bytes: v0.j, v1.j
    const uint32_t r23 = __builtin_amdgcn_perm(v[3], v[2], sel);   // bytes: v2.j, v3.j
    return __builtin_amdgcn_perm(r23, r01, 0x05040100u);
  };
#pragma unroll
  for (int h = 0; h < kQtHalves; ++h) {
    const int cc = (t & 7) * 8 + 64 * h;
    uint32_t lo[4], hi[4];   // row k: codes of columns cc..cc+3 and cc+4..cc+7
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float f[8];
      unpack8_raw<BF16>(w[h][k], f);
      lo[k] = e4m3_pack4(f[0] * scale, f[1] * scale, f[2] * scale, f[3] * scale);
      hi[k] = e4m3_pack4(f[4] * scale, f[5] * scale, f[6] * scale, f[7] * scale);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint32_t*>(tile + (cc + j) * kQtPitch + 4 * rg) = column(lo, j);
      *reinterpret_cast<uint32_t*>(tile + (cc + 4 + j) * kQtPitch + 4 * rg) = column(hi, j);
    }
  }
  __syncthreads();
  // write: kQtCols output rows (= input columns) x 8 chunks of 16 codes
#pragma unroll
  for (int p = 0; p < 2 * kQtHalves; ++p) {
    const int idx = t + p * kThreads;
    const int oc = idx >> 3, orr = (idx & 7) * 16;
    if (c0 + oc < cols && r0 + orr < rows) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + oc * kQtPitch + orr);
      const int64_t off = job.nks > 0 ? tiled_offset(c0 + oc, r0 + orr, job.nks, job.split) : (c0 + oc) * rows + r0 + orr;
      *reinterpret_cast<uint4*>(codes_t + off) = make_uint4(src[0], src[1], src[2], src[3]);
    }
  }
}

// y [cols, rows] = x [rows, cols]^T for bf16 (the weights of the backward's
// data-gradient GEMMs, so that they run on the N-contiguous kernel). A
// workgroup takes a 64 x 64 tile: each thread loads two 16-byte row chunks
// (rows and columns past the matrix re-read a clamped in-range chunk whose
// values are never stored), writes them into an LDS tile with an odd word
// pitch, and gathers 8 consecutive rows of one column into a 16-byte output
// chunk; a wave stores 8 output rows of 128 bytes.
constexpr int kTrTile = 64;
constexpr int kTrPitch = kTrTile * 2 + 4;   // bytes per LDS row: 33 words
__global__ void __launch_bounds__(kThreads) transpose_bf16_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                                  uint16_t* y) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTrTile * kTrPitch];
  const int64_t tiles_c = (cols + kTrTile - 1) / kTrTile;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * kTrTile, c0 = (int64_t)(blockIdx.x % tiles_c) * kTrTile;
  const int t = threadIdx.x, q = t & 7, rr = t >> 3;
  uint4 v[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int64_t r = min(r0 + rr + 32 * k, rows - 1), c = min(c0 + 8 * q, cols - 8);
    v[k] = load_stream16(x + r * cols + c);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t* d = reinterpret_cast<uint32_t*>(tile + (rr + 32 * k) * kTrPitch + 16 * q);
    d[0] = v[k].x; d[1] = v[k].y; d[2] = v[k].z; d[3] = v[k].w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = t + k * kThreads;
    const int oc = idx >> 3, p = idx & 7;   // output row (input column), 8-row chunk
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = *reinterpret_cast<const uint16_t*>(tile + (8 * p + i) * kTrPitch + 2 * oc);
    if (c0 + oc < cols && r0 + 8 * p < rows) {
      const uint4 w = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                                 e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16));
      *reinterpret_cast<uint4*>(y + (c0 + oc) * rows + r0 + 8 * p) = w;
    }
  }
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) dequantize_kernel(const uint8_t* codes, int64_t n8,
                                                              const float* scale_inv, void* y) {
  const float si = *scale_inv;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < n8; c += stride) {
    const uint2 w = *reinterpret_cast<const uint2*>(codes + c * 8);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = e4m3_decode((w.x >> (8 * i)) & 0xFF) * si;
      f[i + 4] = e4m3_decode((w.y >> (8 * i)) & 0xFF) * si;
    }
    store8<BF16>(y, c * 8, f);
  }
}

// ------------------------------------------------------------------ act_lu
// Thread (x) = 8 output columns; blocks in y walk the rows with a stride.
// MODE 0: store; 1: amax only; 2: E4M3 codes.

// ------------------------------------------------------------------ dact + dbias
// Block = W waves over one strip of 512 output columns (8 per lane) and one
// short chunk of rows (about 32: many small blocks balance well over the
// CUs); wave w takes rows w, w+W, ... of the chunk, 4 rows per iteration so
// that each lane has 8 (gated 12) 16-byte streaming loads in flight. Each
// lane keeps fp32 column sums in registers; the W waves are combined in LDS
// in a fixed order and every block writes one row of fp32 partials, which
// dbias_finalize sums in a fixed order (bitwise reproducible).
// MODE kDactStore writes dx; kDactAmax writes no dx but the block's max |dx|
// (fp32, before any rounding) to amax_part[block]; kDactQuant writes the E4M3
// codes of dx * scale, the scale coming from the finished amax; kDactSum
// writes nothing but the column partials (with the linear activation this is
// the bias gradient sum over rows of grad); kDactStoreAct writes dx and, from
// the same read of x, the activation output act(x) (gated: act(a) * b) in the
// input dtype, the value the forward's activation pass stores, so that a
// backward that needs both reads x once.
// 8 waves per block: a sweep of 4 / 8 / 16 waves (with 2 or 4 rows per
// iteration and 4096 / 8192 / 16384 blocks) at 8192 x 16384 (GELU) and
// 8192 x 2 x 14336 (SwiGLU) found 8 waves, 4 rows, 8192 blocks fastest:
// dact + dbias kernel 0.131 -> 0.128 ms and 0.214 -> 0.201 ms against 4 waves.
#ifndef TE_DACT_WAVES
#define TE_DACT_WAVES 8
#endif
#ifndef TE_DACT_UNROLL
#define TE_DACT_UNROLL 4
#endif
#ifndef TE_DACT_TARGET_BLOCKS
#define TE_DACT_TARGET_BLOCKS 8192
#endif
#ifndef TE_DACT_RESIDENT_BLOCKS
#define TE_DACT_RESIDENT_BLOCKS 8192
#endif
constexpr int kDactStrip = 512;
constexpr int kDactWaves = TE_DACT_WAVES;
constexpr int kDactUnroll = TE_DACT_UNROLL;
// The forward activation pass (act_lu, its amax and quantise modes) uses the
// same strip layout with its own shape: 4 waves of 8 rows per iteration (one
// input stream, so twice the rows of dact for the same loads in flight) were
// the fastest of 4 x 4, 4 x 8, 8 x 4 and 8 x 8 for the fp8 forward's act
// quantise pass at 8192 x 16384 (0.0703 -> 0.0673 ms against 8 x 4).
#ifndef TE_ACT_WAVES
#define TE_ACT_WAVES 4
#endif
#ifndef TE_ACT_UNROLL
#define TE_ACT_UNROLL 8
#endif
constexpr int kActWaves = TE_ACT_WAVES;
constexpr int kActUnroll = TE_ACT_UNROLL;
enum DactMode { kDactStore = 0, kDactAmax = 1, kDactQuant = 2, kDactSum = 3, kDactStoreAct = 4 };

template <bool BF16, int ACT, bool GATED, int MODE>
__global__ void __launch_bounds__(64 * kDactWaves) dact_kernel(const void* grad, const void* x, int64_t rows,
                                                               int64_t cols, int64_t rows_per_chunk,
                                                               void* dx, float* partials, float* amax_part,
                                                               const float* amax, void* act_out) {
  constexpr int G = GATED ? 2 : 1;
  constexpr int W = kDactWaves, U = kDactUnroll;
  constexpr int64_t ES = BF16 ? 2 : 4;                    // bytes per input / dx element
  constexpr int64_t OS = MODE == kDactQuant ? 1 : ES;     // bytes per output element
  __shared__ float red[W][G][kDactStrip];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int64_t col = (int64_t)blockIdx.x * kDactStrip + lane * 8;
  const int64_t xcols = G * cols;
  const int64_t nchunks = (rows + rows_per_chunk - 1) / rows_per_chunk;
  const bool writes = MODE == kDactStore || MODE == kDactQuant || MODE == kDactStoreAct;
  constexpr bool kAct = MODE == kDactStoreAct;
  // the lane's offsets in row w of a chunk; row w + k is k row pitches further (soffset)
  const uint32_t vg = (uint32_t)((w * cols + col) * ES);
  const uint32_t vx = (uint32_t)((w * xcols + col) * ES);
  const uint32_t vd = (uint32_t)((w * xcols + col) * OS);
  float qscale = 1.0f;
  if constexpr (MODE == kDactQuant) qscale = fp8_scale_from_amax(*amax);
  float sa[8], sb[8], m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) { sa[i] = 0.0f; sb[i] = 0.0f; }
  if (col < cols) {
    // chunks blockIdx.y, blockIdx.y + gridDim.y, ...: the sums run over all of them
    for (int64_t ch = blockIdx.y; ch < nchunks; ch += gridDim.y) {
      const int64_t r_begin = ch * rows_per_chunk;
      const int64_t nr = min(rows_per_chunk, rows - r_begin);   // rows of this chunk, >= 1
      // descriptors over the chunk's rows (below 2 GiB: the host sizes the chunks)
      const Rsrc rg = buf_rsrc(reinterpret_cast<const uint8_t*>(grad) + r_begin * cols * ES, nr * cols * ES);
      const Rsrc rx = buf_rsrc(reinterpret_cast<const uint8_t*>(x) + r_begin * xcols * ES, nr * xcols * ES);
      const Rsrc rd = buf_rsrc(writes ? reinterpret_cast<const uint8_t*>(dx) + r_begin * xcols * OS : nullptr,
                               writes ? nr * xcols * OS : 0);
      // act(x): [rows, cols] like grad, so it takes grad's offsets
      const Rsrc ra = buf_rsrc(kAct ? reinterpret_cast<const uint8_t*>(act_out) + r_begin * cols * ES : nullptr,
                               kAct ? nr * cols * ES : 0);
      // one output chunk of 8 values at byte offset voff (+ soff) of the chunk's dx
      auto emit = [&](uint32_t voff, uint32_t soff, const float* d) {
        if constexpr (MODE == kDactStore || MODE == kDactStoreAct) {
          // the gated dx (two outputs per grad element) is written with the nt
          // hint: 0.2014 -> 0.1918 ms at 8192 x 2 x 14336, while the same hint
          // made the one-output kernel slower (0.124 -> 0.1285 ms at 8192 x 16384)
          store8_buf<BF16, GATED ? kStoreAuxNt : 0>(rd, voff, soff, d);
        } else if constexpr (MODE == kDactAmax) {
#pragma unroll
          for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(d[i]));
        } else if constexpr (MODE == kDactQuant) {
          store8_codes_buf(rd, voff, soff, encode8(d, qscale));
        }
      };
      // rows past the chunk (the last iteration's tail) load as zero, which adds
      // nothing to the sums or the amax, and their stores are dropped
      for (int64_t r0 = 0; r0 < nr; r0 += W * U) {
        Raw8<BF16> gw[U], aw[U], bw[GATED ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t rr = r0 + (int64_t)u * W;
          load8_raw<BF16>(rg, vg, (uint32_t)(rr * cols * ES), gw[u]);
          load8_raw<BF16>(rx, vx, (uint32_t)(rr * xcols * ES), aw[u]);
          if constexpr (GATED) load8_raw<BF16>(rx, vx + (uint32_t)(cols * ES), (uint32_t)(rr * xcols * ES), bw[u]);
        }
        // every load of the step is issued before the first use (left to itself the
        // scheduler interleaves load, wait and unpack, one load in flight at a time)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t rr = r0 + (int64_t)u * W;
          const uint32_t so = (uint32_t)(rr * xcols * OS);
          float g[1][8], a[1][8], b[1][8];
          unpack8_raw<BF16>(gw[u], g[0]);
          unpack8_raw<BF16>(aw[u], a[0]);
          if constexpr (GATED) unpack8_raw<BF16>(bw[u], b[0]);
          float d[8];
          float y[8];   // act(x), kept by kDactStoreAct only
          if constexpr (GATED) {
            float db[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              float f, df;
              act_fwd_bwd<ACT>(a[0][i], f, df);
              d[i] = mul_rn(mul_rn(g[0][i], b[0][i]), df);
              db[i] = mul_rn(g[0][i], f);
              y[i] = mul_rn(f, b[0][i]);
              sa[i] = add_rn(sa[i], d[i]);
              sb[i] = add_rn(sb[i], db[i]);
            }
            emit(vd, so, d);
            emit(vd + (uint32_t)(cols * OS), so, db);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              // act_fwd_bwd's pair equals act_fwd and act_bwd bit for bit
              float df;
              if constexpr (kAct) act_fwd_bwd<ACT>(a[0][i], y[i], df);
              else df = act_bwd<ACT>(a[0][i]);
              d[i] = mul_rn(g[0][i], df);
              sa[i] = add_rn(sa[i], d[i]);
            }
            emit(vd, so, d);
          }
          if constexpr (kAct) store8_buf<BF16>(ra, vg, (uint32_t)(rr * cols * ES), y);
        }
      }
    }
  }
  if constexpr (MODE == kDactAmax) {
    __shared__ float mred[W];
    m = wave_max(m);
    if (lane == 0) mred[w] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float bm = mred[0];
#pragma unroll
      for (int k = 1; k < W; ++k) bm = fmaxf(bm, mred[k]);
      amax_part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = bm;
    }
  }
  if (MODE == kDactQuant || partials == nullptr) return;   // no dbias (uniform across the block)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[w][0][lane * 8 + i] = sa[i];
    if constexpr (GATED) red[w][G - 1][lane * 8 + i] = sb[i];
  }
  __syncthreads();
  // the block's threads finalise G*512 columns: fixed order w = 0..W-1
  for (int idx = threadIdx.x; idx < G * kDactStrip; idx += 64 * W) {
    const int h = idx / kDactStrip, cl = idx % kDactStrip;
    const int64_t c = (int64_t)blockIdx.x * kDactStrip + cl;
    if (c < cols) {
      float s = red[0][h][cl];
#pragma unroll
      for (int k = 1; k < W; ++k) s += red[k][h][cl];
      partials[(int64_t)blockIdx.y * xcols + h * cols + c] = s;
    }
  }
}

// Max over the per-block partial amaxes; writes amax, scale, scale_inv. One
// workgroup of 1024 threads, 8 loads in flight per lane.
constexpr int kFinThreads = 1024;
__global__ void __launch_bounds__(kFinThreads) amax_finalize_kernel(const float* part, int64_t n, float* amax,
                                                                     float* scale, float* scale_inv) {
  float m = 0.0f;
  constexpr int U = 8;
  for (int64_t i0 = threadIdx.x; i0 < n; i0 += (int64_t)kFinThreads * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = part[min(i0 + (int64_t)u * kFinThreads, n - 1)];   // past the end: the last again
#pragma unroll
    for (int u = 0; u < U; ++u) m = fmaxf(m, v[u]);
  }
  __shared__ float red[kFinThreads / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int k = 1; k < kFinThreads / 64; ++k) r = fmaxf(r, red[k]);
    const float sc = fp8_scale_from_amax(r);
    *amax = r;
    *scale = sc;
    *scale_inv = 1.0f / sc;
  }
}

// Column sums of the per-chunk partials. A block owns 64 columns (one per
// lane, 256-byte rows of partials) and its 8 waves sum disjoint, contiguous
// ranges of chunks, 8 loads in flight per lane; the wave sums are then added
// in wave order, so the result does not depend on timing.
constexpr int kFinWaves = 8;
template <int OUT>
__global__ void __launch_bounds__(64 * kFinWaves) dbias_finalize_kernel(const float* partials, int64_t chunks,
                                                                        int64_t n, void* dbias) {
  __shared__ float red[kFinWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const int64_t per = (chunks + kFinWaves - 1) / kFinWaves;
  const int64_t k1 = min((w + 1) * per, chunks);
  float s = 0.0f;
  if (c < n) {
    constexpr int U = 8;
    int64_t k = w * per;
    for (; k + U <= k1; k += U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = partials[(k + u) * n + c];
#pragma unroll
      for (int u = 0; u < U; ++u) s += v[u];
    }
    for (; k < k1; ++k) s += partials[k * n + c];
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < n) {
    float t = red[0][lane];
#pragma unroll
    for (int q = 1; q < kFinWaves; ++q) t += red[q][lane];
    if constexpr (OUT == kBF16) reinterpret_cast<uint16_t*>(dbias)[c] = f32_to_bf16(t);
    else reinterpret_cast<float*>(dbias)[c] = t;
  }
}

// Rows per work chunk of the strip kernels (dact, act): about TE_DACT_TARGET_BLOCKS chunks in all, at
// least 16 rows each, and a chunk's rows of x (fp32, gated: 2 cols) below
// 2 GiB so that one buffer descriptor with 32-bit offsets covers them.
int64_t dact_rows_per_chunk(int64_t rows, int64_t cols, bool gated) {
  const int64_t strips = (cols + kDactStrip - 1) / kDactStrip;
  int64_t chunks = (TE_DACT_TARGET_BLOCKS + strips - 1) / strips;
  const int64_t max_chunks = (rows + 15) / 16;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  int64_t rpc = (rows + chunks - 1) / chunks;
  const int64_t row_bytes = (gated ? 2 : 1) * cols * 4;
  const int64_t max_rpc = (((int64_t)1 << 31) - 1) / row_bytes;
  if (rpc > max_rpc) rpc = max_rpc;
  return rpc < 1 ? 1 : rpc;
}

// Activation forward (act_lu): y = act(x), gated y = act(a) * b for x = [a | b].
// The same layout as dact: 512-column strips, W waves over short row chunks
// read through per-chunk buffer descriptors, U rows per step with all loads
// in flight before the first use. MODE 0 stores y (OUT bf16 / fp32), 1 the
// amax of y only (one partial maximum per workgroup into amax[block index];
// the grid is capped and a workgroup loops over chunks), 2 the E4M3 codes of
// y * scale with the scale from the finished amax.
template <bool BF16, int ACT, bool GATED, int MODE, int OUT>
__global__ void __launch_bounds__(64 * kActWaves) act_kernel(const void* x, int64_t rows, int64_t cols,
                                                              int64_t rows_per_chunk, void* y, float* amax,
                                                              float* scale_out, float* scale_inv_out,
                                                              int64_t y_nks) {
  constexpr int G = GATED ? 2 : 1;
  constexpr int W = kActWaves, U = kActUnroll;
  constexpr int64_t ES = BF16 ? 2 : 4;
  constexpr int64_t OS = MODE == 2 ? 1 : (OUT == kBF16 ? 2 : 4);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int64_t col = (int64_t)blockIdx.x * kDactStrip + lane * 8;
  const int64_t xcols = G * cols;
  const int64_t nchunks = (rows + rows_per_chunk - 1) / rows_per_chunk;
  float qscale = 1.0f;
  if constexpr (MODE == 2) {
    qscale = fp8_scale_from_amax(*amax);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
      *scale_out = qscale;
      *scale_inv_out = 1.0f / qscale;
    }
  }
  const uint32_t vx = (uint32_t)((w * xcols + col) * ES);
  const uint32_t vy = (uint32_t)((w * cols + col) * OS);
  float m = 0.0f;
  if (col < cols) {
    for (int64_t ch0 = blockIdx.y; ch0 < nchunks; ch0 += gridDim.y) {
      // the quantise mode takes the last rows first: the ones its producer,
      // GEMM1's epilogue, wrote last (0.0714 -> 0.0697 ms at 8192 x 16384)
      const int64_t ch = MODE == 2 ? nchunks - 1 - ch0 : ch0;
      const int64_t r_begin = ch * rows_per_chunk;
      const int64_t nr = min(rows_per_chunk, rows - r_begin);
      const Rsrc rx = buf_rsrc(reinterpret_cast<const uint8_t*>(x) + r_begin * xcols * ES, nr * xcols * ES);
      const Rsrc ry = buf_rsrc(MODE != 1 ? reinterpret_cast<const uint8_t*>(y) + r_begin * cols * OS : nullptr,
                               MODE != 1 ? nr * cols * OS : 0);
      for (int64_t r0 = 0; r0 < nr; r0 += W * U) {
        Raw8<BF16> aw[U], bw[GATED ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t so = (uint32_t)((r0 + (int64_t)u * W) * xcols * ES);
          load8_raw<BF16>(rx, vx, so, aw[u]);
          if constexpr (GATED) load8_raw<BF16>(rx, vx + (uint32_t)(cols * ES), so, bw[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float a[8], o[8];
          unpack8_raw<BF16>(aw[u], a);
          if constexpr (GATED) {
            float b[8];
            unpack8_raw<BF16>(bw[u], b);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = act_fwd<ACT>(a[i]) * b[i];
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = act_fwd<ACT>(a[i]);
          }
          const uint32_t so = (uint32_t)((r0 + (int64_t)u * W) * cols * OS);
          if constexpr (MODE == 0) {
            store8_buf<OUT == kBF16>(ry, vy, so, o);
          } else if constexpr (MODE == 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(o[i]));
          } else if (y_nks > 0) {
            // tiled codes (the next GEMM's A): 8 codes, half of one 16-byte slot; rows past
            // the chunk (read as zero) belong to the next chunk and are not written
            const int64_t rc = r0 + (int64_t)u * W + w;
            if (rc < nr)
              *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(y) + tiled_offset(r_begin + rc, col, y_nks, 0)) =
                  encode8(o, qscale);
          } else {
            store8_codes_buf(ry, vy, so, encode8(o, qscale));
          }
        }
      }
    }
  }
  if constexpr (MODE == 1) {
    __shared__ float red[W];
    block_max_store(m, amax + (blockIdx.y * gridDim.x + blockIdx.x), red);
  }
}

// The capped grid of the amax mode: its workgroup count is the number of
// partial maxima.
dim3 act_amax_grid(int64_t rows, int64_t cols, bool gated) {
  const int64_t rpc = dact_rows_per_chunk(rows, cols, gated);
  const int64_t chunks = (rows + rpc - 1) / rpc;
  const int64_t strips = (cols + kDactStrip - 1) / kDactStrip;
  return dim3((unsigned)strips, (unsigned)min(chunks, max((int64_t)1, (int64_t)kAmaxBlocks / strips)));
}

template <bool BF16>
hipError_t act_dispatch(const void* x, int64_t rows, int64_t cols, int act, bool gated, int mode,
                        void* y, int y_dtype, float* amax, float* so, float* sio, hipStream_t s, bool y_tiled) {
  if (rows <= 0) return hipSuccess;
  if (y_tiled && (mode != 2 || cols > kTiledMaxRowBytes)) return hipErrorInvalidValue;
  const int64_t nks = y_tiled ? tiled_stages(cols) : 0;   // E4M3 codes: one byte per column
  const int64_t rpc = dact_rows_per_chunk(rows, cols, gated);
  const int64_t chunks = (rows + rpc - 1) / rpc;
  const int64_t strips = (cols + kDactStrip - 1) / kDactStrip;
  const dim3 grid((unsigned)strips, (unsigned)chunks);
  // amax pass: at most kAmaxBlocks workgroups (one partial maximum each)
  const dim3 grid_amax = act_amax_grid(rows, cols, gated);
  constexpr int T = 64 * kActWaves;
#define TE_ACT_CASE(A, G)                                                                                      \
  if (mode == 1) launch_kernel(act_kernel<BF16, A, G, 1, kF32>, grid_amax, T, 0, s, x, rows, cols, rpc, y, amax, so, sio, nks);   \
  else if (mode == 2) launch_kernel(act_kernel<BF16, A, G, 2, kE4M3>, grid, T, 0, s, x, rows, cols, rpc, y, amax, so, sio, nks); \
  else if (y_dtype == kBF16) launch_kernel(act_kernel<BF16, A, G, 0, kBF16>, grid, T, 0, s, x, rows, cols, rpc, y, amax, so, sio, nks); \
  else launch_kernel(act_kernel<BF16, A, G, 0, kF32>, grid, T, 0, s, x, rows, cols, rpc, y, amax, so, sio, nks);
#define TE_ACT_G(A) if (gated) { TE_ACT_CASE(A, true) } else { TE_ACT_CASE(A, false) }
  switch (act) {
    case kRelu: TE_ACT_G(kRelu) break;
    case kGelu: TE_ACT_G(kGelu) break;
    case kGeluErf: TE_ACT_G(kGeluErf) break;
    case kSilu: TE_ACT_G(kSilu) break;
    default: TE_ACT_G(kLinear) break;
  }
#undef TE_ACT_G
#undef TE_ACT_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_zero(float* p, int n, hipStream_t s) {
  LaunchScope scope("fill_zero", s);
  launch_kernel(fill_zero_kernel, (n + 255) / 256, 256, 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_fill_zero_bytes(void* p, int64_t nbytes, hipStream_t s) {
  LaunchScope scope("fill_zero", s);
  const int64_t words = nbytes / 4;
  launch_kernel(fill_zero_words_kernel, (unsigned)((words + 255) / 256), 256, 0, s, reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

hipError_t launch_empty_meta(float* amax, float* scale, float* scale_inv, hipStream_t s) {
  LaunchScope scope("empty_meta", s);
  launch_kernel(empty_meta_kernel, 1, 64, 0, s, amax, scale, scale_inv);
  return hipGetLastError();
}

hipError_t launch_amax(const void* x, int64_t n, int x_dtype, float* amax, hipStream_t s) {
  return launch_amax2(x, n, amax, nullptr, 0, nullptr, x_dtype, s);
}

hipError_t launch_amax2(const void* x0, int64_t n0, float* amax0, const void* x1, int64_t n1, float* amax1,
                        int x_dtype, hipStream_t s) {
  LaunchScope scope("amax", s);
  // one atomic per workgroup on the job's address: few workgroups, each looping
  const unsigned b0 = min(grid_for(n0 / 8, kUnroll), kAmaxBlocks / 2);
  const unsigned b1 = n1 > 0 ? min(grid_for(n1 / 8, kUnroll), kAmaxBlocks / 2) : 0u;
  const AmaxJob j0{x0, n0 / 8, amax0}, j1{x1, n1 / 8, amax1};
  if (x_dtype == kBF16) launch_kernel(amax_kernel<true>, b0 + b1, kThreads, 0, s, j0, j1, b0);
  else launch_kernel(amax_kernel<false>, b0 + b1, kThreads, 0, s, j0, j1, b0);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int64_t n, int x_dtype, uint8_t* codes, const float* amax,
                           float* scale_out, float* scale_inv_out, hipStream_t s) {
  LaunchScope scope("quantize", s);
  const unsigned grid = grid_for(n / 8, 4);
  if (x_dtype == kBF16)
    launch_kernel(quantize_kernel<true>, grid, kThreads, 0, s, x, n / 8, codes, amax, scale_out, scale_inv_out);
  else
    launch_kernel(quantize_kernel<false>, grid, kThreads, 0, s, x, n / 8, codes, amax, scale_out, scale_inv_out);
  return hipGetLastError();
}

hipError_t launch_quantize_transpose(const void* x, int64_t rows, int64_t cols, int x_dtype,
                                     uint8_t* codes_t, const float* amax, float* scale_out,
                                     float* scale_inv_out, hipStream_t s, bool tiled) {
  return launch_quantize_transpose2(x, rows, cols, codes_t, amax, scale_out, scale_inv_out, nullptr, 0, 0, nullptr,
                                    nullptr, nullptr, nullptr, x_dtype, s, tiled, false, 0);
}

hipError_t launch_quantize_transpose2(const void* x0, int64_t rows0, int64_t cols0, uint8_t* codes_t0,
                                      const float* amax0, float* scale0, float* scale_inv0, const void* x1,
                                      int64_t rows1, int64_t cols1, uint8_t* codes_t1, const float* amax1,
                                      float* scale1, float* scale_inv1, int x_dtype, hipStream_t s, bool tiled0,
                                      bool tiled1, int64_t split0) {
  LaunchScope scope("quantize_transpose", s);
  // codes_t rows are K = rows of x long
  if ((tiled0 && rows0 > kTiledMaxRowBytes) || (tiled1 && rows1 > kTiledMaxRowBytes) ||
      (split0 > 0 && (!tiled0 || 2 * split0 != cols0)))
    return hipErrorInvalidValue;
  auto tiles = [](int64_t r, int64_t c) {   // < 2^17 for weights < 2 GiB
    return (unsigned)(((c + kQtCols - 1) / kQtCols) * ((r + kQtRows - 1) / kQtRows));
  };
  const unsigned t0 = tiles(rows0, cols0), t1 = rows1 > 0 ? tiles(rows1, cols1) : 0u;
  const QtJob j0{x0, rows0, cols0, codes_t0, amax0, scale0, scale_inv0, tiled0 ? tiled_stages(rows0) : 0, split0};
  const QtJob j1{x1, rows1, cols1, codes_t1, amax1, scale1, scale_inv1, tiled1 ? tiled_stages(rows1) : 0, 0};
  if (x_dtype == kBF16) launch_kernel(quantize_transpose_kernel<true>, t0 + t1, kThreads, 0, s, j0, j1, t0);
  else launch_kernel(quantize_transpose_kernel<false>, t0 + t1, kThreads, 0, s, j0, j1, t0);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* x, int64_t rows, int64_t cols, void* y, hipStream_t s) {
  LaunchScope scope("transpose", s);
  const unsigned tiles = (unsigned)(((rows + kTrTile - 1) / kTrTile) * ((cols + kTrTile - 1) / kTrTile));
  launch_kernel(transpose_bf16_kernel, tiles, kThreads, 0, s, reinterpret_cast<const uint16_t*>(x), rows, cols,
                reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, int64_t n, const float* scale_inv, void* y,
                             int y_dtype, hipStream_t s) {
  LaunchScope scope("dequantize", s);
  const unsigned grid = grid_for(n / 8, 4);
  if (y_dtype == kBF16) launch_kernel(dequantize_kernel<true>, grid, kThreads, 0, s, codes, n / 8, scale_inv, y);
  else launch_kernel(dequantize_kernel<false>, grid, kThreads, 0, s, codes, n / 8, scale_inv, y);
  return hipGetLastError();
}

int64_t act_amax_blocks(int64_t rows, int64_t cols, bool gated) {
  if (rows <= 0) return 0;
  const dim3 g = act_amax_grid(rows, cols, gated);
  return (int64_t)g.x * g.y;
}

hipError_t launch_amax_finalize(const float* part, int64_t n, float* amax, float* scale, float* scale_inv,
                                hipStream_t s) {
  LaunchScope scope("amax_finalize", s);
  launch_kernel(amax_finalize_kernel, 1, kFinThreads, 0, s, part, n, amax, scale, scale_inv);
  return hipGetLastError();
}

hipError_t launch_act(const void* x, int64_t rows, int64_t cols, int x_dtype, int act, bool gated,
                      int mode, void* y, int y_dtype, float* amax, float* scale_out,
                      float* scale_inv_out, hipStream_t s, bool y_tiled) {
  static const char* names[3] = {"act_lu", "act_amax", "act_quant"};
  LaunchScope scope(names[mode], s);
  if (x_dtype == kBF16)
    return act_dispatch<true>(x, rows, cols, act, gated, mode, y, y_dtype, amax, scale_out, scale_inv_out, s,
                              y_tiled);
  return act_dispatch<false>(x, rows, cols, act, gated, mode, y, y_dtype, amax, scale_out, scale_inv_out, s,
                             y_tiled);
}


// Workgroups along the row axis (= rows of partial column sums): one per
// work chunk, at most about TE_DACT_RESIDENT_BLOCKS workgroups in all; a
// workgroup then takes every gridDim.y-th chunk.
int64_t dact_row_chunks(int64_t rows, int64_t cols, bool gated) {
  if (rows <= 0) return 1;
  const int64_t rpc = dact_rows_per_chunk(rows, cols, gated);
  const int64_t work = (rows + rpc - 1) / rpc;
  const int64_t strips = (cols + kDactStrip - 1) / kDactStrip;
  const int64_t cap = max((int64_t)1, (int64_t)TE_DACT_RESIDENT_BLOCKS / strips);
  return work < cap ? work : cap;
}

int64_t dact_blocks(int64_t rows, int64_t cols, bool gated) {
  return ((cols + kDactStrip - 1) / kDactStrip) * dact_row_chunks(rows, cols, gated);
}

namespace {
template <int MODE>
hipError_t dact_dispatch(const void* grad, const void* x, int64_t rows, int64_t cols, int dtype, int act, bool gated,
                         void* dx, float* partials, float* amax_part, const float* amax, hipStream_t s,
                         void* act_out = nullptr) {
  const int64_t chunks = dact_row_chunks(rows, cols, gated);
  const int64_t rpc = dact_rows_per_chunk(rows, cols, gated);
  const dim3 grid((unsigned)((cols + kDactStrip - 1) / kDactStrip), (unsigned)chunks);
#define TE_DACT(B, A, G) launch_kernel(dact_kernel<B, A, G, MODE>, grid, 64 * kDactWaves, 0, s, grad, x, rows, cols, rpc, dx, partials, amax_part, amax, act_out)
#define TE_DACT_G(B, A) if (gated) TE_DACT(B, A, true); else TE_DACT(B, A, false);
#define TE_DACT_A(B)                                   \
  switch (act) {                                       \
    case kRelu: TE_DACT_G(B, kRelu) break;             \
    case kGelu: TE_DACT_G(B, kGelu) break;             \
    case kGeluErf: TE_DACT_G(B, kGeluErf) break;       \
    case kSilu: TE_DACT_G(B, kSilu) break;             \
    default: TE_DACT_G(B, kLinear) break;              \
  }
  if (dtype == kBF16) { TE_DACT_A(true) } else { TE_DACT_A(false) }
#undef TE_DACT_A
#undef TE_DACT_G
#undef TE_DACT
  return hipGetLastError();
}

hipError_t dbias_finalize(const float* partials, int64_t rows, int64_t cols, bool gated, void* dbias,
                          int dbias_dtype, hipStream_t s) {
  LaunchScope scope("dbias_finalize", s);
  const int64_t chunks = dact_row_chunks(rows, cols, gated);
  const int64_t n = (gated ? 2 : 1) * cols;
  const unsigned g2 = (unsigned)((n + 63) / 64);
  if (dbias_dtype == kBF16) launch_kernel(dbias_finalize_kernel<kBF16>, g2, 64 * kFinWaves, 0, s, partials, chunks, n, dbias);
  else launch_kernel(dbias_finalize_kernel<kF32>, g2, 64 * kFinWaves, 0, s, partials, chunks, n, dbias);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_dact_dbias(const void* grad, const void* x, int64_t rows, int64_t cols, int dtype,
                             int act, bool gated, void* dx, void* dbias, int dbias_dtype,
                             float* partials, hipStream_t s) {
  {
    LaunchScope scope("dact_dbias", s);
    const hipError_t e = dact_dispatch<kDactStore>(grad, x, rows, cols, dtype, act, gated, dx,
                                                   dbias != nullptr ? partials : nullptr, nullptr, nullptr, s);
    if (e != hipSuccess) return e;
  }
  if (dbias != nullptr) return dbias_finalize(partials, rows, cols, gated, dbias, dbias_dtype, s);
  return hipSuccess;
}

hipError_t launch_dact_dbias_act(const void* grad, const void* x, int64_t rows, int64_t cols, int dtype,
                                 int act, bool gated, void* dx, void* act_out, void* dbias, int dbias_dtype,
                                 float* partials, hipStream_t s) {
  {
    LaunchScope scope("dact_dbias_act", s);
    const hipError_t e = dact_dispatch<kDactStoreAct>(grad, x, rows, cols, dtype, act, gated, dx,
                                                      dbias != nullptr ? partials : nullptr, nullptr, nullptr, s,
                                                      act_out);
    if (e != hipSuccess) return e;
  }
  if (dbias != nullptr) return dbias_finalize(partials, rows, cols, gated, dbias, dbias_dtype, s);
  return hipSuccess;
}

hipError_t launch_colsum(const void* x, int64_t rows, int64_t cols, int dtype, void* sum, int sum_dtype,
                         float* partials, hipStream_t s) {
  {
    LaunchScope scope("colsum", s);
    // the linear activation's gradient is 1: dact's column partials of grad = x
    const hipError_t e = dact_dispatch<kDactSum>(x, x, rows, cols, dtype, kLinear, false, nullptr, partials,
                                                 nullptr, nullptr, s);
    if (e != hipSuccess) return e;
  }
  return dbias_finalize(partials, rows, cols, false, sum, sum_dtype, s);
}

hipError_t launch_dact_dbias_quantize(const void* grad, const void* x, int64_t rows, int64_t cols, int dtype,
                                      int act, bool gated, uint8_t* codes, float* amax, float* scale,
                                      float* scale_inv, void* dbias, int dbias_dtype, float* partials,
                                      float* amax_part, hipStream_t s) {
  {
    LaunchScope scope("dact_dbias_amax", s);
    const hipError_t e = dact_dispatch<kDactAmax>(grad, x, rows, cols, dtype, act, gated, nullptr,
                                                  dbias != nullptr ? partials : nullptr, amax_part, nullptr, s);
    if (e != hipSuccess) return e;
  }
  if (dbias != nullptr) {
    const hipError_t e = dbias_finalize(partials, rows, cols, gated, dbias, dbias_dtype, s);
    if (e != hipSuccess) return e;
  }
  {
    LaunchScope scope("amax_finalize", s);
    launch_kernel(amax_finalize_kernel, 1, kFinThreads, 0, s, amax_part, dact_blocks(rows, cols, gated), amax, scale, scale_inv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  LaunchScope scope("dact_quant", s);
  return dact_dispatch<kDactQuant>(grad, x, rows, cols, dtype, act, gated, codes, nullptr, nullptr, amax, s);
}

}  // namespace te
