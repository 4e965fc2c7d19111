// Host-side launchers of the gfx950 kernels (internal to the library).
// Every launcher assumes its arguments were validated by the C ABI layer and
// returns the HIP error of its launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace te {

// Element types as in te_dtype.
enum { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

// Activation kinds (kernel template parameters).
enum ActKind { kRelu = 0, kGelu = 1, kGeluErf = 2, kSilu = 3, kLinear = 4 };

// Per-kernel timing: while timing is on, the launches made inside a scope
// carry its two HIP events (launch_kernel below), which the runtime stamps
// with the first kernel's start and the last kernel's end, with no separate
// event packets around the dispatches. A scope without a launch records both
// events back to back.
struct LaunchScope {
  LaunchScope(const char* name, hipStream_t s);
  ~LaunchScope();
  int slot;
  int prev;
  hipStream_t stream;
};
// Events for a kernel launched in the innermost timing scope (both null
// unless timing is on): the scope's start event on its first launch, its stop
// event on every launch.
void scope_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through this: the arguments are
// converted to the kernel's parameter types, and the active scope's events
// ride on the dispatch.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  scope_launch_events(&e0, &e1);
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0u, static_cast<KArgs>(args)...);
}

// ---------------------------------------------------------------- GEMM operand tiles
// The MFMA GEMMs stream a K-contiguous operand [rows, K] in k stages of 64
// bytes per row and 256 rows per workgroup tile. An operand that the library
// writes itself for one of its own GEMMs (the normalised input, the
// activation, the quantised kernels; never a caller's tensor) is stored
// "tiled": as the sequence of those stages, each exactly the image the GEMM
// keeps in LDS, so that every load instruction of the GEMM reads one
// contiguous KiB instead of sixteen 64-byte pieces a row pitch apart.
//   block (t, s): rows [256 t, 256 t + 256) x bytes [64 s, 64 s + 64) of each
//   row, 16 KiB at (t * S + s) * 16 KiB, S = tiled_stages(row bytes); inside
//   it row r sits at 64 r with its 16-byte chunk c at slot c ^ ((r / 4) % 4)
//   (the GEMMs' LDS chunk swizzle).
// Split layout (the gated GEMM1's transposed kernel, whose 256-row tile is
// rows [128 t, 128 t + 128) of the first half and the same rows of the second
// half [split, 2 split)): block rows 0..127 and 128..255 hold those two runs.
// Bytes of a block past the operand's rows or K are never written or read
// (the GEMMs' range checks return zeros there). tiled_offset() in
// gemm_lds.hpp maps (row, byte) to the layout.
constexpr int kTiledBlockShift = 14;   // 16 KiB blocks
// Longest tiled row: keeps every stage's block offset (the GEMMs' scalar
// buffer offset, up to three stages past the end) far below 2^31.
constexpr int64_t kTiledMaxRowBytes = (int64_t)1 << 20;
inline int64_t tiled_stages(int64_t row_bytes) { return (row_bytes + 63) / 64; }
inline int64_t tiled_row_tiles(int64_t rows, int64_t split) {
  return split > 0 ? (split + 127) / 128 : (rows + 255) / 256;
}
inline size_t tiled_bytes(int64_t rows, int64_t row_bytes, int64_t split) {
  return (size_t)(tiled_row_tiles(rows, split) * tiled_stages(row_bytes)) << kTiledBlockShift;
}

// ---------------------------------------------------------------- norm
enum NormMode { kNormStore = 0, kNormAmax = 1, kNormQuant = 2 };
// kNormStore: y (F32/BF16) and optional mu/rsigma.
// kNormAmax : no y; one partial maximum of |normalised value| per workgroup
//             into part[0, norm_amax_parts(rows)), optional mu/rsigma.
// kNormQuant: y = E4M3 codes with the scale from the maximum of those
//             partials; writes *amax, *scale_out and *scale_inv_out.
// part is required by the two fp8 modes (norm_amax_parts(rows) floats).
// y_tiled: y (BF16 or E4M3) in the tiled GEMM operand layout.
// Floats that a call's first pass sets to zero for the passes after it to
// raise with atomics (amax slots): n floats from `first`, and up to three
// single floats elsewhere (nullptr: none).
struct ClearList {
  float* first = nullptr;
  int n = 0;
  float* one[3] = {nullptr, nullptr, nullptr};
};
// clear (amax mode only): workgroup 0 zeroes the listed floats, so that no
// separate fill launch precedes the pass.
hipError_t launch_norm(const void* x, const void* gamma, const void* beta, int64_t rows,
                       int64_t hidden, int x_dtype, bool rms, bool zcg, float eps, int mode,
                       int y_dtype, void* y, float* mu, float* rsigma, float* amax,
                       float* scale_out, float* scale_inv_out, float* part, hipStream_t s,
                       bool y_tiled = false, const ClearList* clear = nullptr);
int64_t norm_amax_parts(int64_t rows);

// ---------------------------------------------------------------- elementwise
hipError_t launch_fill_zero(float* p, int n, hipStream_t s);
// Zero nbytes (a multiple of 4) at p.
hipError_t launch_fill_zero_bytes(void* p, int64_t nbytes, hipStream_t s);
// amax = 0, scale = 1, scale_inv = 1 (metadata of an empty tensor).
hipError_t launch_empty_meta(float* amax, float* scale, float* scale_inv, hipStream_t s);

// amax of |x| over n elements into *amax (atomic max, *amax must start at 0).
hipError_t launch_amax(const void* x, int64_t n, int x_dtype, float* amax, hipStream_t s);
// The same for two tensors of one dtype in one launch (n1 = 0: only the first).
hipError_t launch_amax2(const void* x0, int64_t n0, float* amax0, const void* x1, int64_t n1, float* amax1,
                        int x_dtype, hipStream_t s);

// codes[i] = E4M3(x[i] * scale), scale from *amax; writes scale/scale_inv.
hipError_t launch_quantize(const void* x, int64_t n, int x_dtype, uint8_t* codes,
                           const float* amax, float* scale_out, float* scale_inv_out,
                           hipStream_t s);

// Quantise a [rows, cols] matrix and store it transposed as [cols, rows]
// codes (K-contiguous operand layout for the fp8 GEMM); tiled: in the tiled
// GEMM operand layout, split as described there (0: plain).
hipError_t launch_quantize_transpose(const void* x, int64_t rows, int64_t cols, int x_dtype,
                                     uint8_t* codes_t, const float* amax, float* scale_out,
                                     float* scale_inv_out, hipStream_t s, bool tiled = false);
// The same for two matrices of one dtype in one launch (rows1 = 0: only the
// first), each tiled or not; split0 applies to the first.
hipError_t launch_quantize_transpose2(const void* x0, int64_t rows0, int64_t cols0, uint8_t* codes_t0,
                                      const float* amax0, float* scale0, float* scale_inv0, const void* x1,
                                      int64_t rows1, int64_t cols1, uint8_t* codes_t1, const float* amax1,
                                      float* scale1, float* scale_inv1, int x_dtype, hipStream_t s,
                                      bool tiled0 = false, bool tiled1 = false, int64_t split0 = 0);
// y [cols, rows] = x [rows, cols]^T, bf16; rows and cols multiples of 16.
hipError_t launch_transpose_bf16(const void* x, int64_t rows, int64_t cols, void* y, hipStream_t s);

hipError_t launch_dequantize(const uint8_t* codes, int64_t n, const float* scale_inv, void* y,
                             int y_dtype, hipStream_t s);

// Activation forward: x [rows, G*cols] -> y [rows, cols].
// mode 0: store y (F32/BF16); 1: amax only, one partial maximum per workgroup
// into amax[0 .. act_amax_blocks()); 2: E4M3 codes using *amax, in the tiled
// GEMM operand layout when y_tiled.
hipError_t launch_act(const void* x, int64_t rows, int64_t cols, int x_dtype, int act,
                      bool gated, int mode, void* y, int y_dtype, float* amax,
                      float* scale_out, float* scale_inv_out, hipStream_t s, bool y_tiled = false);
int64_t act_amax_blocks(int64_t rows, int64_t cols, bool gated);
// Max of n partial maxima -> amax; scale = 448 / amax (1 if 0), scale_inv.
hipError_t launch_amax_finalize(const float* part, int64_t n, float* amax, float* scale, float* scale_inv,
                                hipStream_t s);

// dact + dbias. partials: fp32 workspace of dact_partials_floats() floats.
int64_t dact_row_chunks(int64_t rows, int64_t cols, bool gated);
// Normalisation backward. norm_bwd_team_waves() is 0 when a row does not fit
// one workgroup's registers (hidden above 16384 bf16 / 8192 fp32);
// norm_bwd_fits() also checks the LDS of the column-sum combine. part_g and
// part_b: fp32 workspace of norm_bwd_blocks() * hidden floats each.
int norm_bwd_team_waves(int64_t hidden, int dtype);
int64_t norm_bwd_blocks(int64_t rows, int64_t hidden, int dtype);
bool norm_bwd_fits(int64_t hidden, int dtype);
hipError_t launch_norm_bwd(const void* dy, const void* x, const float* mu, const float* rsigma, const void* gamma,
                           int64_t rows, int64_t hidden, int dtype, bool rms, bool zcg, void* dx, void* dgamma,
                           void* dbeta, int dparam_dtype, float* part_g, float* part_b, hipStream_t s);

// Number of dact workgroups (one partial amax each in the quantising variant).
int64_t dact_blocks(int64_t rows, int64_t cols, bool gated);
hipError_t launch_dact_dbias(const void* grad, const void* x, int64_t rows, int64_t cols,
                             int dtype, int act, bool gated, void* dx, void* dbias,
                             int dbias_dtype, float* partials, hipStream_t s);
// The same, also writing act_out [rows, cols] = act(x) (gated: act(a) * b) in
// dtype, the values launch_act's store mode writes, from the same read of x.
hipError_t launch_dact_dbias_act(const void* grad, const void* x, int64_t rows, int64_t cols, int dtype,
                                 int act, bool gated, void* dx, void* act_out, void* dbias, int dbias_dtype,
                                 float* partials, hipStream_t s);
// Column sums of x [rows, cols] (fp32, fixed order) into sum [cols];
// partials: dact_row_chunks(rows, cols, false) * cols floats.
hipError_t launch_colsum(const void* x, int64_t rows, int64_t cols, int dtype, void* sum, int sum_dtype,
                         float* partials, hipStream_t s);
// dact + dbias with the activation gradient quantised to E4M3 (current
// scaling): pass 1 computes dx for the bias partials and per-workgroup amax
// partials (amax_part: dact_blocks() floats), a one-workgroup kernel reduces
// them into amax / scale / scale_inv, pass 2 recomputes dx and writes codes.
hipError_t launch_dact_dbias_quantize(const void* grad, const void* x, int64_t rows, int64_t cols, int dtype,
                                      int act, bool gated, uint8_t* codes, float* amax, float* scale,
                                      float* scale_inv, void* dbias, int dbias_dtype, float* partials,
                                      float* amax_part, hipStream_t s);

// ---------------------------------------------------------------- GEMMs
// Epilogue applied to h = acc * scale + bias (scale = 1 unless fp8):
//   out   : act(h) (or act(h_a) * h_b when gated), NULL to skip
//   h_out : h rounded to the element type, NULL to skip
//   amax  : atomic max of |act(h_rounded)|, NULL to skip (fp8 forward)
struct Epilogue {
  const void* bias;       // [n_b] of the GEMM's element type, or NULL
  void* out;              // [M, n_out]
  void* h_out;            // [M, n_b]
  float* amax;
  int act;                // ActKind
  bool gated;
  const char* name = nullptr;   // timing-scope name (default: from act / gated)
  bool out_f32 = false;   // out is fp32 (plain ungated epilogue without h_out / amax only)
  bool out_tiled = false; // out (bf16) in the tiled GEMM operand layout (the next GEMM's A)
};

// bf16: C[M, n_out] from A [M, K] (row-major, or tiled when a_tiled) and
// B [K, n_b] (row-major).
hipError_t launch_gemm_bf16(const void* A, const void* B, int64_t M, int64_t n_b, int64_t K,
                            const Epilogue& ep, hipStream_t s, bool a_tiled = false);

// bf16 with A^T [K, M] and B [K, n_b] (both row-major with K the row index),
// linear epilogue: the weight-gradient GEMMs of the backward.
hipError_t launch_gemm_bf16_at(const void* At, const void* B, int64_t M, int64_t n_b, int64_t K,
                               const Epilogue& ep, hipStream_t s);

// fp8: A codes [M, K] and B^T codes [n_b, K] (both K-contiguous, each
// row-major or tiled; a gated B^T is tiled with split n_b / 2); the
// accumulator is multiplied by scale_inv(amax_a) * scale_inv(amax_b).
hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* Bt, int64_t M, int64_t n_b,
                           int64_t K, const float* amax_a, const float* amax_b,
                           const Epilogue& ep, hipStream_t s, bool a_tiled = false, bool b_tiled = false);

// fp32: all operands fp32.
hipError_t launch_gemm_f32(const float* A, const float* B, int64_t M, int64_t n_b, int64_t K,
                           const Epilogue& ep, hipStream_t s);

}  // namespace te
