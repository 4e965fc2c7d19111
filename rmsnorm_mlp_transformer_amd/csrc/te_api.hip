// C ABI of the library: argument validation, workspace layout and the launch
// sequence of every entry point declared in include/te_mi355x.h.
//
// Every entry point validates all of its arguments before the first HIP call,
// so a failed call writes nothing and the validation paths run without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "probe.hpp"
#include "te_kernels.hpp"
#include "../../include/te_mi355x.h"

namespace {

thread_local std::string g_error;

te_status fail(te_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

te_status ok() {
  g_error.clear();
  return TE_SUCCESS;
}

te_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define TE_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)
#define TE_ARG(cond, ...) TE_REQUIRE(cond, TE_ERR_INVALID_ARGUMENT, __VA_ARGS__)
#define TE_HIP(expr, what)                                   \
  do {                                                       \
    const hipError_t e_ = (expr);                            \
    if (e_ != hipSuccess) return hip_status(e_, what);       \
  } while (0)

size_t esize(int dt) { return dt == TE_F32 ? 4 : dt == TE_BF16 ? 2 : 1; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool feature_ok(int64_t n) { return n > 0 && n % 16 == 0 && n <= (int64_t)1 << 22; }
// The GEMMs address a weight matrix through one buffer descriptor with 32-bit
// byte offsets: it must stay below 2 GiB.
bool weight_ok(int64_t rows, int64_t cols, int dtype) { return rows * cols * (int64_t)esize(dtype) < ((int64_t)1 << 31); }
bool valid_act(int a) { return a >= TE_ACT_RELU && a <= TE_ACT_GEGLU_ERF; }
bool is_gated(int a) { return a >= TE_ACT_REGLU; }
int act_kind(int a) {
  switch (a) {
    case TE_ACT_RELU: case TE_ACT_REGLU: return te::kRelu;
    case TE_ACT_GELU: case TE_ACT_GEGLU: return te::kGelu;
    case TE_ACT_GELU_ERF: case TE_ACT_GEGLU_ERF: return te::kGeluErf;
    case TE_ACT_SILU: case TE_ACT_SWIGLU: return te::kSilu;
    default: return te::kLinear;
  }
}
bool meta_ok(const te_fp8_meta* m) {
  return m != nullptr && m->amax != nullptr && m->scale != nullptr && m->scale_inv != nullptr;
}
bool meta_complete(const te_fp8_meta& m) {
  return m.amax != nullptr && m.scale != nullptr && m.scale_inv != nullptr;
}

// Carves 256-byte aligned sub-buffers from the caller's workspace. With a
// NULL base it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
  float* floats(size_t n) { return static_cast<float*>(take(n * sizeof(float))); }
};

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// fp8 metadata slots: caller's meta when complete, else workspace floats.
struct Meta {
  float* amax;
  float* scale;
  float* scale_inv;
};
Meta pick_meta(const te_fp8_meta* user, float* ws3) {
  if (user != nullptr && meta_complete(*user)) return {user->amax, user->scale, user->scale_inv};
  return {ws3, ws3 ? ws3 + 1 : nullptr, ws3 ? ws3 + 2 : nullptr};
}

// ---------------------------------------------------------------- per-kernel timing
struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
  bool started;   // a launch has taken the start event
};
struct TimingTotal {
  std::string name;
  int64_t launches;
  double ms;
};
bool g_timing = false;
std::vector<TimingRec> g_pending;
int g_active = -1;   // g_pending index of the innermost open scope
std::vector<hipEvent_t> g_event_pool;
std::vector<TimingTotal> g_totals;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---------------------------------------------------------------- layouts
// The library's own GEMM operands (normalised input, activation, transposed
// kernel codes) are written in the tiled GEMM operand layout whenever their
// rows are short enough for it; a caller's buffer (the saved codes) stays
// row-major.
bool tiled_ok(int64_t row_bytes) { return row_bytes <= te::kTiledMaxRowBytes; }
// Bytes of a [rows, row_bytes] operand, tiled (split: see te_kernels.hpp) or row-major.
size_t operand_bytes(bool tiled, int64_t rows, int64_t row_bytes, int64_t split = 0) {
  return tiled ? te::tiled_bytes(rows, row_bytes, split) : (size_t)rows * row_bytes;
}

struct DenseWs {
  void* xn;        // normalised input (F32/BF16) or codes
  uint8_t* wt;     // fp8: kernel codes, transposed
  float* metas;    // fp8: 6 floats
  float* npart;    // fp8: the norm amax pass's partial maxima
  bool tiled;      // xn (and wt) in the tiled operand layout
};
DenseWs dense_ws(Carver& c, int64_t rows, int64_t hidden, int64_t out, int dtype, int quant) {
  DenseWs w{};
  if (quant == TE_QUANT_FP8_E4M3_CURRENT) {
    w.tiled = tiled_ok(hidden);
    w.metas = c.floats(6);
    w.npart = c.floats((size_t)te::norm_amax_parts(rows));
    w.xn = c.take(operand_bytes(w.tiled, rows, hidden));
    w.wt = static_cast<uint8_t*>(c.take(operand_bytes(w.tiled, out, hidden)));
  } else {
    w.tiled = dtype == TE_BF16 && tiled_ok(hidden * 2);
    w.xn = c.take(operand_bytes(w.tiled, rows, hidden * esize(dtype)));
  }
  return w;
}

struct MlpWs {
  void* xn;        // normalised input (F32/BF16) or its codes
  void* act;       // activation output (F32/BF16) or its codes
  uint8_t* w1t;    // fp8: kernel1 codes transposed [G*ffn, hidden]
  uint8_t* w2t;    // fp8: kernel2 codes transposed [hidden, ffn]
  void* h1;        // fp8: GEMM1 output + bias1, bf16 [rows, G*ffn] (when not saved)
  float* metas;    // fp8: 12 floats
  float* npart;    // fp8: the norm amax pass's partial maxima
  bool t1, t2;     // the workspace operands of GEMM1 (xn, w1t) / GEMM2 (act, w2t) are tiled
};
MlpWs mlp_ws(Carver& c, int64_t rows, int64_t hidden, int64_t ffn, int dtype, int act, int quant,
             bool need_h1) {
  MlpWs w{};
  const int64_t g = is_gated(act) ? 2 : 1;
  if (quant == TE_QUANT_FP8_E4M3_CURRENT) {
    w.t1 = tiled_ok(hidden);
    w.t2 = tiled_ok(ffn);
    w.metas = c.floats(12);
    w.npart = c.floats((size_t)te::norm_amax_parts(rows));
    w.xn = c.take(operand_bytes(w.t1, rows, hidden));
    w.w1t = static_cast<uint8_t*>(c.take(operand_bytes(w.t1, g * ffn, hidden, g == 2 ? ffn : 0)));
    w.w2t = static_cast<uint8_t*>(c.take(operand_bytes(w.t2, hidden, ffn)));
    if (need_h1) w.h1 = c.take((size_t)rows * g * ffn * 2);
    w.act = c.take(operand_bytes(w.t2, rows, ffn));
  } else {
    const int64_t es = esize(dtype);
    w.t1 = dtype == TE_BF16 && tiled_ok(hidden * 2);
    w.t2 = dtype == TE_BF16 && tiled_ok(ffn * 2);
    w.xn = c.take(operand_bytes(w.t1, rows, hidden * es));
    w.act = c.take(operand_bytes(w.t2, rows, ffn * es));
  }
  return w;
}

te_status check_dtype_quant(te_dtype dtype, te_quant quant) {
  TE_ARG(dtype == TE_F32 || dtype == TE_BF16 || dtype == TE_E4M3, "invalid dtype %d", (int)dtype);
  TE_ARG(quant == TE_QUANT_NONE || quant == TE_QUANT_FP8_E4M3_CURRENT, "invalid quant %d", (int)quant);
  TE_REQUIRE(dtype != TE_E4M3, TE_ERR_UNSUPPORTED, "E4M3 is not an input dtype");
  TE_REQUIRE(!(dtype == TE_F32 && quant != TE_QUANT_NONE), TE_ERR_UNSUPPORTED,
             "fp8 quantisation requires dtype TE_BF16");
  return TE_SUCCESS;
}

// Output dtypes of the forwards: the input dtype, or fp32 from bf16 inputs.
te_status check_y_dtype(te_dtype dtype, te_dtype y_dtype) {
  TE_ARG(y_dtype == TE_F32 || y_dtype == TE_BF16 || y_dtype == TE_E4M3, "invalid y_dtype %d", (int)y_dtype);
  TE_REQUIRE(y_dtype == dtype || (dtype == TE_BF16 && y_dtype == TE_F32), TE_ERR_UNSUPPORTED,
             "y_dtype must be the input dtype or, for TE_BF16 inputs, TE_F32");
  return TE_SUCCESS;
}

te_status check_norm(const void* x, const void* gamma, const void* beta, int64_t rows,
                     int64_t hidden, te_norm_type nt, float eps) {
  TE_ARG(rows >= 0 && rows <= (int64_t)1 << 31, "rows must be in [0, 2^31], got %lld", (long long)rows);
  TE_ARG(feature_ok(hidden), "hidden must be a positive multiple of 16 (at most 2^22), got %lld", (long long)hidden);
  TE_ARG(nt == TE_LAYERNORM || nt == TE_RMSNORM, "invalid norm_type %d", (int)nt);
  TE_ARG(eps >= 0.0f && eps < 1e30f, "epsilon must be finite and >= 0");
  TE_ARG(gamma != nullptr && (x != nullptr || rows == 0), "x and gamma are required");
  TE_ARG(nt == TE_RMSNORM || beta != nullptr, "beta is required for layernorm");
  TE_ARG(aligned16(x) && aligned16(gamma) && (beta == nullptr || aligned16(beta)),
         "x, gamma and beta must be 16-byte aligned");
  return TE_SUCCESS;
}

// Arguments shared by the dact + dbias entry points; dx is the output (dx, or
// the codes of the quantising variant), named dx_name in the messages.
te_status check_dact(const void* grad, const void* x, int64_t rows, int64_t cols, te_dtype dtype, te_act_type act_type,
                     const void* dx, const char* dx_name, const void* dbias, te_dtype dbias_dtype) {
  TE_ARG(rows >= 0 && rows <= (int64_t)1 << 31, "rows out of range");
  TE_ARG(feature_ok(cols), "cols must be a positive multiple of 16, got %lld", (long long)cols);
  TE_ARG(valid_act(act_type), "invalid act_type %d", (int)act_type);
  TE_ARG(dtype == TE_F32 || dtype == TE_BF16, "dtype must be TE_F32 or TE_BF16");
  TE_ARG(dbias == nullptr || dbias_dtype == TE_F32 || dbias_dtype == TE_BF16, "dbias_dtype must be TE_F32 or TE_BF16");
  TE_ARG((grad != nullptr && x != nullptr && dx != nullptr) || rows == 0, "grad, x and %s are required", dx_name);
  TE_ARG(aligned16(grad) && aligned16(x) && aligned16(dx) && (dbias == nullptr || aligned16(dbias)),
         "pointers must be 16-byte aligned");
  return TE_SUCCESS;
}

}  // namespace

namespace te {
LaunchScope::LaunchScope(const char* name, hipStream_t s) : slot(-1), prev(g_active), stream(s) {
  if (!g_timing) return;
  hipEvent_t a = pooled_event(), b = pooled_event();
  if (a == nullptr || b == nullptr) return;
  g_pending.push_back({name, a, b, false});
  slot = (int)g_pending.size() - 1;
  g_active = slot;
}
LaunchScope::~LaunchScope() {
  if (slot < 0) return;
  TimingRec& r = g_pending[slot];
  if (!r.started) {   // nothing was launched: an empty interval
    (void)hipEventRecord(r.start, stream);
    (void)hipEventRecord(r.stop, stream);
  }
  g_active = prev;
}
void scope_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_active < 0) return;
  TimingRec& r = g_pending[g_active];
  if (!r.started) {
    *start = r.start;
    r.started = true;
  }
  *stop = r.stop;
}
}  // namespace te

extern "C" {

const char* te_last_error(void) { return g_error.c_str(); }
te_status te_probe_mfma(int fp8, int64_t iters, int blocks, float* sink, uint64_t* ticks, void* stream) {
  TE_ARG(blocks >= 1 && iters >= 1, "blocks and iters must be at least 1");
  TE_ARG(sink != nullptr, "sink is required");
  TE_HIP(te::launch_mfma_probe(fp8 != 0, iters, blocks, sink, ticks, as_stream(stream)), "mfma probe");
  return ok();
}

const char* te_version(void) { return "temi355x 0.1.0 (gfx950)"; }

// ---------------------------------------------------------------- timing
te_status te_timing_enable(int enable) {
  g_timing = enable != 0;
  return ok();
}
int te_timing_collect(void) {
  for (auto& r : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      TimingTotal* t = nullptr;
      for (auto& e : g_totals)
        if (e.name == r.name) t = &e;
      if (t == nullptr) {
        g_totals.push_back({r.name, 0, 0.0});
        t = &g_totals.back();
      }
      t->launches += 1;
      t->ms += ms;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_pending.clear();
  return (int)g_totals.size();
}
te_status te_timing_get(int i, const char** name, int64_t* launches, double* total_ms) {
  TE_ARG(i >= 0 && i < (int)g_totals.size(), "timing index %d out of range", i);
  if (name) *name = g_totals[i].name.c_str();
  if (launches) *launches = g_totals[i].launches;
  if (total_ms) *total_ms = g_totals[i].ms;
  return ok();
}
void te_timing_reset(void) {
  te_timing_collect();
  g_totals.clear();
}

// ---------------------------------------------------------------- norm
size_t te_layernorm_fwd_workspace_size(int64_t rows, int64_t hidden, te_dtype x_dtype, te_dtype y_dtype) {
  (void)hidden;
  (void)x_dtype;
  if (rows <= 0 || y_dtype != TE_E4M3) return 0;
  Carver c(nullptr);
  c.floats((size_t)te::norm_amax_parts(rows));
  return c.off;
}

te_status te_layernorm_fwd(const void* x, const void* gamma, const void* beta, int64_t rows,
                           int64_t hidden, te_dtype x_dtype, te_norm_type norm_type,
                           int zero_centered_gamma, float epsilon, void* y, te_dtype y_dtype,
                           const te_fp8_meta* y_meta, float* mu, float* rsigma, void* workspace,
                           size_t workspace_bytes, void* stream) {
  te_status st = check_norm(x, gamma, beta, rows, hidden, norm_type, epsilon);
  if (st != TE_SUCCESS) return st;
  TE_ARG(x_dtype == TE_F32 || x_dtype == TE_BF16, "x_dtype must be TE_F32 or TE_BF16");
  TE_ARG(y_dtype == TE_F32 || y_dtype == TE_BF16 || y_dtype == TE_E4M3, "invalid y_dtype");
  TE_ARG((y != nullptr || rows == 0) && aligned16(y), "y is required and must be 16-byte aligned");
  TE_ARG(y_dtype != TE_E4M3 || meta_ok(y_meta), "E4M3 output needs y_meta with amax, scale, scale_inv");
  const size_t need = te_layernorm_fwd_workspace_size(rows, hidden, x_dtype, y_dtype);
  TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
             workspace_bytes, need);
  TE_ARG(need == 0 || (workspace != nullptr && aligned16(workspace)), "workspace is required (16-byte aligned)");
  hipStream_t s = as_stream(stream);
  if (rows == 0) {
    if (y_dtype == TE_E4M3) TE_HIP(te::launch_empty_meta(y_meta->amax, y_meta->scale, y_meta->scale_inv, s), "meta");
    return ok();
  }
  const bool rms = norm_type == TE_RMSNORM;
  if (y_dtype != TE_E4M3) {
    TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, x_dtype, rms, zero_centered_gamma != 0, epsilon,
                           te::kNormStore, y_dtype, y, mu, rsigma, nullptr, nullptr, nullptr, nullptr, s),
           "norm");
    return ok();
  }
  Carver c(workspace);
  float* part = c.floats((size_t)te::norm_amax_parts(rows));
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, x_dtype, rms, zero_centered_gamma != 0, epsilon,
                         te::kNormAmax, y_dtype, nullptr, mu, rsigma, nullptr, nullptr, nullptr, part, s),
         "norm amax");
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, x_dtype, rms, zero_centered_gamma != 0, epsilon,
                         te::kNormQuant, y_dtype, y, nullptr, nullptr, y_meta->amax, y_meta->scale,
                         y_meta->scale_inv, part, s),
         "norm quantise");
  return ok();
}

// ---------------------------------------------------------------- activation
size_t te_act_lu_workspace_size(int64_t rows, int64_t cols, te_act_type act_type, te_dtype y_dtype) {
  if (rows <= 0 || cols <= 0 || y_dtype != TE_E4M3) return 0;
  Carver c(nullptr);
  c.floats((size_t)te::act_amax_blocks(rows, cols, is_gated(act_type)));
  return c.off;
}

te_status te_act_lu(const void* x, int64_t rows, int64_t cols, te_dtype x_dtype, te_act_type act_type,
                    void* y, te_dtype y_dtype, const te_fp8_meta* y_meta, void* workspace,
                    size_t workspace_bytes, void* stream) {
  TE_ARG(rows >= 0 && rows <= (int64_t)1 << 31, "rows out of range");
  TE_ARG(feature_ok(cols), "cols must be a positive multiple of 16, got %lld", (long long)cols);
  TE_ARG(valid_act(act_type), "invalid act_type %d", (int)act_type);
  TE_ARG(x_dtype == TE_F32 || x_dtype == TE_BF16, "x_dtype must be TE_F32 or TE_BF16");
  TE_ARG(y_dtype == TE_F32 || y_dtype == TE_BF16 || y_dtype == TE_E4M3, "invalid y_dtype");
  TE_ARG(((x != nullptr && y != nullptr) || rows == 0) && aligned16(x) && aligned16(y),
         "x and y are required, 16-byte aligned");
  TE_ARG(y_dtype != TE_E4M3 || meta_ok(y_meta), "E4M3 output needs y_meta with amax, scale, scale_inv");
  const size_t need = te_act_lu_workspace_size(rows, cols, act_type, y_dtype);
  TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
             workspace_bytes, need);
  TE_ARG(need == 0 || (workspace != nullptr && aligned16(workspace)), "workspace is required (16-byte aligned)");
  hipStream_t s = as_stream(stream);
  if (rows == 0) {
    if (y_dtype == TE_E4M3) TE_HIP(te::launch_empty_meta(y_meta->amax, y_meta->scale, y_meta->scale_inv, s), "meta");
    return ok();
  }
  const bool g = is_gated(act_type);
  const int k = act_kind(act_type);
  if (y_dtype != TE_E4M3) {
    TE_HIP(te::launch_act(x, rows, cols, x_dtype, k, g, 0, y, y_dtype, nullptr, nullptr, nullptr, s), "act");
    return ok();
  }
  // current scaling: per-workgroup maxima of |act(x)| into the workspace, their
  // max (and the scale) into y_meta, then the codes
  Carver c(workspace);
  float* part = c.floats((size_t)te::act_amax_blocks(rows, cols, g));
  TE_HIP(te::launch_act(x, rows, cols, x_dtype, k, g, 1, nullptr, y_dtype, part, nullptr, nullptr, s), "act amax");
  TE_HIP(te::launch_amax_finalize(part, te::act_amax_blocks(rows, cols, g), y_meta->amax, y_meta->scale,
                                  y_meta->scale_inv, s),
         "amax");
  TE_HIP(te::launch_act(x, rows, cols, x_dtype, k, g, 2, y, y_dtype, y_meta->amax, y_meta->scale,
                        y_meta->scale_inv, s),
         "act quantise");
  return ok();
}

size_t te_dact_dbias_workspace_size(int64_t rows, int64_t cols, te_act_type act_type) {
  if (rows <= 0 || cols <= 0) return 0;
  const bool g = is_gated(act_type);
  Carver c(nullptr);
  c.floats((size_t)te::dact_row_chunks(rows, cols, g) * (g ? 2 : 1) * cols);
  return c.off;
}

te_status te_dact_dbias(const void* grad, const void* x, int64_t rows, int64_t cols, te_dtype dtype,
                        te_act_type act_type, void* dx, void* dbias, te_dtype dbias_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  te_status st = check_dact(grad, x, rows, cols, dtype, act_type, dx, "dx", dbias, dbias_dtype);
  if (st != TE_SUCCESS) return st;
  const size_t need = te_dact_dbias_workspace_size(rows, cols, act_type);
  if (dbias != nullptr) {
    TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL,
               "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    TE_ARG(workspace != nullptr && aligned16(workspace), "workspace is required (16-byte aligned)");
  }
  hipStream_t s = as_stream(stream);
  const bool g = is_gated(act_type);
  if (rows == 0) {   // the bias gradient of an empty batch is zero
    if (dbias != nullptr) TE_HIP(te::launch_fill_zero_bytes(dbias, (g ? 2 : 1) * cols * (int64_t)esize(dbias_dtype), s), "fill");
    return ok();
  }
  Carver c(workspace);
  float* partials = dbias != nullptr ? c.floats((size_t)te::dact_row_chunks(rows, cols, g) * (g ? 2 : 1) * cols) : nullptr;
  TE_HIP(te::launch_dact_dbias(grad, x, rows, cols, dtype, act_kind(act_type), g, dx, dbias, dbias_dtype,
                               partials, s),
         "dact_dbias");
  return ok();
}

// ---------------------------------------------------------------- dact + dbias without allocation
// The fp32 column partials of te_dact_dbias_noalloc live in this static device
// array (one copy per GPU, held until the process ends). Its device address is
// looked up once per device with hipGetSymbolAddress; in host code the array's
// name is only a host-side stand-in and is never passed to a kernel.
}  // extern "C"
namespace {
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
te_status scratch_address(float** out) {
  int dev = -1;
  TE_HIP(hipGetDevice(&dev), "hipGetDevice");
  TE_REQUIRE(dev >= 0 && dev < kMaxDevices, TE_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    TE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    TE_REQUIRE(p != nullptr, TE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<float*>(g_scratch_ptr[dev]);
  return TE_SUCCESS;
}
}  // namespace
extern "C" {

size_t te_dact_dbias_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

te_status te_dact_dbias_noalloc(const void* grad, const void* x, int64_t rows, int64_t cols, te_dtype dtype,
                                te_act_type act_type, void* dx, void* dbias, te_dtype dbias_dtype, void* stream) {
  te_status st = check_dact(grad, x, rows, cols, dtype, act_type, dx, "dx", dbias, dbias_dtype);
  if (st != TE_SUCCESS) return st;
  const bool g = is_gated(act_type);
  const size_t need = rows > 0 ? (size_t)te::dact_row_chunks(rows, cols, g) * (g ? 2 : 1) * cols * sizeof(float) : 0;
  TE_REQUIRE(need <= kNoallocScratchBytes, TE_ERR_UNSUPPORTED,
             "the bias partials of %lld x %lld need %zu bytes; the static scratch holds %zu", (long long)rows,
             (long long)cols, need, kNoallocScratchBytes);
  hipStream_t s = as_stream(stream);
  if (rows == 0) {   // the bias gradient of an empty batch is zero
    if (dbias != nullptr) TE_HIP(te::launch_fill_zero_bytes(dbias, (g ? 2 : 1) * cols * (int64_t)esize(dbias_dtype), s), "fill");
    return ok();
  }
  float* partials = nullptr;
  if (dbias != nullptr) {
    te_status st = scratch_address(&partials);
    if (st != TE_SUCCESS) return st;
  }
  // every partial the finalize pass reads is written by the dact pass first:
  // nothing in the scratch has to start at zero
  TE_HIP(te::launch_dact_dbias(grad, x, rows, cols, dtype, act_kind(act_type), g, dx, dbias, dbias_dtype,
                               partials, s),
         "dact_dbias");
  return ok();
}

size_t te_dact_dbias_quantize_workspace_size(int64_t rows, int64_t cols, te_act_type act_type) {
  if (rows <= 0 || cols <= 0) return 0;
  const bool g = is_gated(act_type);
  Carver c(nullptr);
  c.floats((size_t)te::dact_row_chunks(rows, cols, g) * (g ? 2 : 1) * cols);
  c.floats((size_t)te::dact_blocks(rows, cols, g));
  return c.off;
}

te_status te_dact_dbias_quantize(const void* grad, const void* x, int64_t rows, int64_t cols, te_dtype dtype,
                                 te_act_type act_type, uint8_t* dx_codes, const te_fp8_meta* dx_meta, void* dbias,
                                 te_dtype dbias_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  te_status st = check_dact(grad, x, rows, cols, dtype, act_type, dx_codes, "dx_codes", dbias, dbias_dtype);
  if (st != TE_SUCCESS) return st;
  TE_ARG(meta_ok(dx_meta), "dx_meta with amax, scale and scale_inv is required");
  const size_t need = te_dact_dbias_quantize_workspace_size(rows, cols, act_type);
  TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
             workspace_bytes, need);
  TE_ARG(need == 0 || (workspace != nullptr && aligned16(workspace)), "workspace is required (16-byte aligned)");
  hipStream_t s = as_stream(stream);
  const bool g = is_gated(act_type);
  if (rows == 0) {   // empty: zero bias gradient, meta of an empty tensor
    if (dbias != nullptr) TE_HIP(te::launch_fill_zero_bytes(dbias, (g ? 2 : 1) * cols * (int64_t)esize(dbias_dtype), s), "fill");
    TE_HIP(te::launch_empty_meta(dx_meta->amax, dx_meta->scale, dx_meta->scale_inv, s), "meta");
    return ok();
  }
  Carver c(workspace);
  float* partials = c.floats((size_t)te::dact_row_chunks(rows, cols, g) * (g ? 2 : 1) * cols);
  float* amax_part = c.floats((size_t)te::dact_blocks(rows, cols, g));
  TE_HIP(te::launch_dact_dbias_quantize(grad, x, rows, cols, dtype, act_kind(act_type), g, dx_codes, dx_meta->amax,
                                        dx_meta->scale, dx_meta->scale_inv, dbias, dbias_dtype, partials, amax_part, s),
         "dact_dbias_quantize");
  return ok();
}

// ---------------------------------------------------------------- layernorm MLP backward
namespace {
struct MlpBwdWs {
  void* xn; void* act; void* dact; void* dh1; void* dxn;
  void* wt;   // kernel2^T, then kernel1^T (the data-gradient GEMMs' N-contiguous B operand)
  float* part_dact; float* part_b2; float* part_g; float* part_beta;
};
MlpBwdWs mlp_bwd_ws(Carver& c, int64_t rows, int64_t hidden, int64_t ffn, int act) {
  const int64_t g = is_gated(act) ? 2 : 1;
  MlpBwdWs w{};
  w.xn = c.take((size_t)rows * hidden * 2);
  w.act = c.take((size_t)rows * ffn * 2);
  w.dact = c.take((size_t)rows * ffn * 2);
  w.dh1 = c.take((size_t)rows * g * ffn * 2);
  w.dxn = c.take((size_t)rows * hidden * 2);
  w.wt = c.take((size_t)hidden * g * ffn * 2);
  w.part_dact = c.floats((size_t)te::dact_row_chunks(rows, ffn, g == 2) * g * ffn);
  w.part_b2 = c.floats((size_t)te::dact_row_chunks(rows, hidden, false) * hidden);
  const int64_t nb = te::norm_bwd_blocks(rows, hidden, TE_BF16);
  w.part_g = c.floats((size_t)nb * hidden);
  w.part_beta = c.floats((size_t)nb * hidden);
  return w;
}
}  // namespace

size_t te_layernorm_mlp_bwd_workspace_size(int64_t rows, int64_t hidden, int64_t ffn, te_act_type act_type) {
  if (rows <= 0 || hidden <= 0 || ffn <= 0) return 0;
  Carver c(nullptr);
  mlp_bwd_ws(c, rows, hidden, ffn, act_type);
  return c.off;
}

te_status te_layernorm_mlp_bwd(const void* grad, const void* x, const void* gamma, const void* beta,
                               const void* kernel1, const void* kernel2, const float* mu, const float* rsigma,
                               const void* h1, int64_t rows, int64_t hidden, int64_t ffn, te_dtype dtype,
                               te_norm_type norm_type, int zero_centered_gamma, float epsilon, te_act_type act_type,
                               void* dx, void* dgamma, void* dbeta, void* dkernel1, void* dbias1, void* dkernel2,
                               void* dbias2, te_dtype dparam_dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  TE_REQUIRE(dtype == TE_BF16, TE_ERR_UNSUPPORTED, "the backward supports dtype TE_BF16 only");
  te_status st = check_norm(x, gamma, beta, rows, hidden, norm_type, epsilon);
  if (st != TE_SUCCESS) return st;
  TE_ARG(feature_ok(ffn), "ffn must be a positive multiple of 16 (at most 2^22), got %lld", (long long)ffn);
  TE_ARG(valid_act(act_type), "invalid act_type %d", (int)act_type);
  const bool gated = is_gated(act_type), rms = norm_type == TE_RMSNORM;
  const int64_t nb1 = (gated ? 2 : 1) * ffn;
  TE_REQUIRE(weight_ok(hidden, nb1, dtype) && weight_ok(ffn, hidden, dtype) && weight_ok(rows, nb1, dtype) &&
                 weight_ok(rows, hidden, dtype),
             TE_ERR_UNSUPPORTED, "kernels and [rows, features] activations must be smaller than 2 GiB");
  TE_REQUIRE(te::norm_bwd_fits(hidden, dtype), TE_ERR_UNSUPPORTED, "hidden too wide for the normalisation backward");
  TE_ARG(dparam_dtype == TE_F32 || dparam_dtype == TE_BF16, "dparam_dtype must be TE_F32 or TE_BF16");
  TE_ARG(rows == 0 || (grad != nullptr && h1 != nullptr && rsigma != nullptr && (rms || mu != nullptr) &&
                       dx != nullptr),
         "grad, h1, rsigma, (LayerNorm) mu and dx are required");
  TE_ARG(kernel1 != nullptr && kernel2 != nullptr && dkernel1 != nullptr && dkernel2 != nullptr,
         "kernels and their gradients are required");
  TE_ARG(aligned16(grad) && aligned16(h1) && aligned16(dx) && aligned16(kernel1) && aligned16(kernel2) &&
             aligned16(dkernel1) && aligned16(dkernel2) && aligned16(dgamma) && aligned16(dbeta) &&
             aligned16(dbias1) && aligned16(dbias2),
         "pointers must be 16-byte aligned");
  if (rms) dbeta = nullptr;
  const size_t need = te_layernorm_mlp_bwd_workspace_size(rows, hidden, ffn, act_type);
  TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
             workspace_bytes, need);
  TE_ARG(need == 0 || (workspace != nullptr && aligned16(workspace)), "workspace is required (16-byte aligned)");
  hipStream_t s = as_stream(stream);
  const int64_t ps = esize(dparam_dtype);
  if (rows == 0) {   // every parameter gradient of an empty batch is zero
    TE_HIP(te::launch_fill_zero_bytes(dkernel1, hidden * nb1 * 2, s), "fill");
    TE_HIP(te::launch_fill_zero_bytes(dkernel2, ffn * hidden * 2, s), "fill");
    for (void* p : {dgamma, dbeta, dbias2})
      if (p != nullptr) TE_HIP(te::launch_fill_zero_bytes(p, hidden * ps, s), "fill");
    if (dbias1 != nullptr) TE_HIP(te::launch_fill_zero_bytes(dbias1, nb1 * ps, s), "fill");
    return ok();
  }
  Carver c(workspace);
  MlpBwdWs w = mlp_bwd_ws(c, rows, hidden, ffn, act_type);
  const int k = act_kind(act_type);
  const te::Epilogue lin{nullptr, nullptr, nullptr, nullptr, te::kLinear, false};
  // the normalised input (GEMM1's A operand), recomputed
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zero_centered_gamma != 0, epsilon, te::kNormStore,
                         dtype, w.xn, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s), "norm");
  // GEMM2's data gradient: dact = grad @ kernel2^T. The data-gradient GEMMs run
  // on the N-contiguous kernel with a transposed copy of the weight (one
  // streaming pass), faster than the K-contiguous kernel on the weight as stored.
  te::Epilogue e = lin;
  e.out = w.dact;
  e.name = "gemm_bf16_dgrad";
  TE_HIP(te::launch_transpose_bf16(kernel2, ffn, hidden, w.wt, s), "transpose kernel2");
  TE_HIP(te::launch_gemm_bf16(grad, w.wt, rows, ffn, hidden, e, s), "dgrad2");
  // activation backward with dbias1; the same pass recomputes the activation
  // output from its read of h1 for GEMM2's weight gradient (one read of h1)
  TE_HIP(te::launch_dact_dbias_act(w.dact, h1, rows, ffn, dtype, k, gated, w.dh1, w.act, dbias1, dparam_dtype,
                                   w.part_dact, s),
         "dact");
  // GEMM2's weight gradient dkernel2 = act^T @ grad, dbias2 = sum of grad
  e.name = nullptr;
  e.out = dkernel2;
  TE_HIP(te::launch_gemm_bf16_at(w.act, grad, ffn, hidden, rows, e, s), "wgrad2");
  if (dbias2 != nullptr) TE_HIP(te::launch_colsum(grad, rows, hidden, dtype, dbias2, dparam_dtype, w.part_b2, s), "dbias2");
  // GEMM1: dxn = dh1 @ kernel1^T, dkernel1 = xn^T @ dh1
  e.out = w.dxn;
  e.name = "gemm_bf16_dgrad";
  TE_HIP(te::launch_transpose_bf16(kernel1, hidden, nb1, w.wt, s), "transpose kernel1");
  TE_HIP(te::launch_gemm_bf16(w.dh1, w.wt, rows, hidden, nb1, e, s), "dgrad1");
  e.name = nullptr;
  e.out = dkernel1;
  TE_HIP(te::launch_gemm_bf16_at(w.xn, w.dh1, hidden, nb1, rows, e, s), "wgrad1");
  // normalisation backward
  TE_HIP(te::launch_norm_bwd(w.dxn, x, mu, rsigma, gamma, rows, hidden, dtype, rms, zero_centered_gamma != 0, dx,
                             dgamma, dbeta, dparam_dtype, w.part_g, w.part_beta, s),
         "norm backward");
  return ok();
}

// ---------------------------------------------------------------- normalisation backward
size_t te_layernorm_bwd_workspace_size(int64_t rows, int64_t hidden, te_dtype dtype) {
  if (rows <= 0 || hidden <= 0) return 0;
  const int64_t blocks = te::norm_bwd_blocks(rows, hidden, dtype);
  Carver c(nullptr);
  c.floats((size_t)blocks * hidden);
  c.floats((size_t)blocks * hidden);
  return c.off;
}

te_status te_layernorm_bwd(const void* dy, const void* x, const float* mu, const float* rsigma, const void* gamma,
                           int64_t rows, int64_t hidden, te_dtype dtype, te_norm_type norm_type,
                           int zero_centered_gamma, void* dx, void* dgamma, void* dbeta, te_dtype dparam_dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  TE_ARG(rows >= 0 && rows <= (int64_t)1 << 31, "rows out of range");
  TE_ARG(feature_ok(hidden), "hidden must be a positive multiple of 16, got %lld", (long long)hidden);
  TE_ARG(dtype == TE_F32 || dtype == TE_BF16, "dtype must be TE_F32 or TE_BF16");
  TE_ARG(norm_type == TE_LAYERNORM || norm_type == TE_RMSNORM, "invalid norm_type %d", (int)norm_type);
  TE_REQUIRE(te::norm_bwd_fits(hidden, dtype), TE_ERR_UNSUPPORTED,
             "hidden %lld too wide for the normalisation backward (at most 16384 bf16 / 8192 fp32)", (long long)hidden);
  const bool rms = norm_type == TE_RMSNORM;
  if (rms) dbeta = nullptr;
  TE_ARG((dgamma == nullptr && dbeta == nullptr) || dparam_dtype == TE_F32 || dparam_dtype == TE_BF16,
         "dparam_dtype must be TE_F32 or TE_BF16");
  TE_ARG(gamma != nullptr && aligned16(gamma), "gamma is required (16-byte aligned)");
  TE_ARG(rows == 0 || (dy != nullptr && x != nullptr && dx != nullptr && rsigma != nullptr && (rms || mu != nullptr)),
         "dy, x, dx, rsigma and (LayerNorm) mu are required");
  TE_ARG(aligned16(dy) && aligned16(x) && aligned16(dx) && (dgamma == nullptr || aligned16(dgamma)) &&
             (dbeta == nullptr || aligned16(dbeta)),
         "pointers must be 16-byte aligned");
  const size_t need = te_layernorm_bwd_workspace_size(rows, hidden, dtype);
  const bool params = dgamma != nullptr || dbeta != nullptr;
  if (params) {
    TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
               workspace_bytes, need);
    TE_ARG(need == 0 || (workspace != nullptr && aligned16(workspace)), "workspace is required (16-byte aligned)");
  }
  hipStream_t s = as_stream(stream);
  if (rows == 0) {   // parameter gradients of an empty batch are zero
    if (dgamma != nullptr) TE_HIP(te::launch_fill_zero_bytes(dgamma, hidden * (int64_t)esize(dparam_dtype), s), "fill");
    if (dbeta != nullptr) TE_HIP(te::launch_fill_zero_bytes(dbeta, hidden * (int64_t)esize(dparam_dtype), s), "fill");
    return ok();
  }
  float *part_g = nullptr, *part_b = nullptr;
  if (params) {
    Carver c(workspace);
    const int64_t blocks = te::norm_bwd_blocks(rows, hidden, dtype);
    part_g = c.floats((size_t)blocks * hidden);
    part_b = c.floats((size_t)blocks * hidden);
  }
  TE_HIP(te::launch_norm_bwd(dy, x, mu, rsigma, gamma, rows, hidden, dtype, rms, zero_centered_gamma != 0, dx, dgamma,
                             dbeta, dparam_dtype, part_g, part_b, s),
         "norm backward");
  return ok();
}

// ---------------------------------------------------------------- quantiser
te_status te_quantize(const void* x, int64_t n, te_dtype x_dtype, uint8_t* codes, const te_fp8_meta* meta,
                      void* stream) {
  TE_ARG(n >= 0 && n % 16 == 0, "n must be a non-negative multiple of 16");
  TE_ARG(x_dtype == TE_F32 || x_dtype == TE_BF16, "x_dtype must be TE_F32 or TE_BF16");
  TE_ARG(x != nullptr && codes != nullptr && aligned16(x) && aligned16(codes), "x and codes are required, 16-byte aligned");
  TE_ARG(meta_ok(meta), "meta with amax, scale and scale_inv is required");
  hipStream_t s = as_stream(stream);
  TE_HIP(te::launch_fill_zero(meta->amax, 1, s), "fill");
  if (n > 0) TE_HIP(te::launch_amax(x, n, x_dtype, meta->amax, s), "amax");
  TE_HIP(te::launch_quantize(x, n, x_dtype, codes, meta->amax, meta->scale, meta->scale_inv, s), "quantise");
  return ok();
}

te_status te_dequantize(const uint8_t* codes, int64_t n, const te_fp8_meta* meta, void* y, te_dtype y_dtype,
                        void* stream) {
  TE_ARG(n >= 0 && n % 16 == 0, "n must be a non-negative multiple of 16");
  TE_ARG(y_dtype == TE_F32 || y_dtype == TE_BF16, "y_dtype must be TE_F32 or TE_BF16");
  TE_ARG(codes != nullptr && y != nullptr && aligned16(codes) && aligned16(y), "codes and y are required, 16-byte aligned");
  TE_ARG(meta != nullptr && meta->scale_inv != nullptr, "meta->scale_inv is required");
  if (n == 0) return ok();
  TE_HIP(te::launch_dequantize(codes, n, meta->scale_inv, y, y_dtype, as_stream(stream)), "dequantise");
  return ok();
}

// ---------------------------------------------------------------- layernorm + dense
size_t te_layernorm_dense_fwd_workspace_size(int64_t rows, int64_t hidden, int64_t out_features, te_dtype dtype,
                                             te_quant quant) {
  if (rows < 0 || hidden <= 0 || out_features <= 0) return 0;
  Carver c(nullptr);
  dense_ws(c, rows, hidden, out_features, dtype, quant);
  return c.off;
}

te_status te_layernorm_dense_fwd(const void* x, const void* kernel, const void* gamma, const void* beta,
                                 const void* bias, int64_t rows, int64_t hidden, int64_t out_features,
                                 te_dtype dtype, te_norm_type norm_type, int zero_centered_gamma, float epsilon,
                                 te_quant quant, void* y, te_dtype y_dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  te_status st = check_dtype_quant(dtype, quant);
  if (st != TE_SUCCESS) return st;
  st = check_y_dtype(dtype, y_dtype);
  if (st != TE_SUCCESS) return st;
  st = check_norm(x, gamma, beta, rows, hidden, norm_type, epsilon);
  if (st != TE_SUCCESS) return st;
  TE_ARG(feature_ok(out_features), "out_features must be a positive multiple of 16 (at most 2^22)");
  TE_REQUIRE(weight_ok(hidden, out_features, dtype), TE_ERR_UNSUPPORTED, "kernel must be smaller than 2 GiB");
  TE_ARG(kernel != nullptr && (y != nullptr || rows == 0) && aligned16(kernel) && aligned16(y),
         "kernel and y are required, 16-byte aligned");
  TE_ARG(bias == nullptr || aligned16(bias), "bias must be 16-byte aligned");
  const size_t need = te_layernorm_dense_fwd_workspace_size(rows, hidden, out_features, dtype, quant);
  TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
             workspace_bytes, need);
  TE_ARG(need == 0 || (workspace != nullptr && aligned16(workspace)), "workspace is required (16-byte aligned)");
  if (rows == 0) return ok();
  hipStream_t s = as_stream(stream);
  Carver c(workspace);
  DenseWs w = dense_ws(c, rows, hidden, out_features, dtype, quant);
  const bool rms = norm_type == TE_RMSNORM, zcg = zero_centered_gamma != 0;
  te::Epilogue ep{bias, y, nullptr, nullptr, te::kLinear, false};
  ep.out_f32 = dtype == TE_BF16 && y_dtype == TE_F32;
  if (quant == TE_QUANT_NONE) {
    TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zcg, epsilon, te::kNormStore, dtype, w.xn,
                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, s, w.tiled), "norm");
    if (dtype == TE_F32)
      TE_HIP(te::launch_gemm_f32(static_cast<const float*>(w.xn), static_cast<const float*>(kernel), rows,
                                 out_features, hidden, ep, s), "gemm");
    else
      TE_HIP(te::launch_gemm_bf16(w.xn, kernel, rows, out_features, hidden, ep, s, w.tiled), "gemm");
    return ok();
  }
  float* mx = w.metas;      // amax, scale, scale_inv of the normalised input
  float* mw = w.metas + 3;  // ... of the kernel
  te::ClearList clear;   // the kernel's amax, raised by atomics (x's is written)
  clear.first = w.metas;
  clear.n = 6;
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zcg, epsilon, te::kNormAmax, TE_E4M3, nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, w.npart, s, false, &clear), "norm amax");
  TE_HIP(te::launch_amax(kernel, hidden * out_features, dtype, mw, s), "kernel amax");
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zcg, epsilon, te::kNormQuant, TE_E4M3, w.xn,
                         nullptr, nullptr, mx, mx + 1, mx + 2, w.npart, s, w.tiled), "norm quantise");
  TE_HIP(te::launch_quantize_transpose(kernel, hidden, out_features, dtype, w.wt, mw, mw + 1, mw + 2, s, w.tiled),
         "kernel quantise");
  TE_HIP(te::launch_gemm_fp8(static_cast<const uint8_t*>(w.xn), w.wt, rows, out_features, hidden, mx, mw, ep, s,
                             w.tiled, w.tiled),
         "fp8 gemm");
  return ok();
}

// ---------------------------------------------------------------- layernorm MLP
size_t te_layernorm_mlp_fwd_workspace_size(int64_t rows, int64_t hidden, int64_t ffn, te_dtype dtype,
                                           te_act_type act_type, te_quant quant) {
  if (rows < 0 || hidden <= 0 || ffn <= 0) return 0;
  Carver c(nullptr);
  mlp_ws(c, rows, hidden, ffn, dtype, act_type, quant, true);
  return c.off;
}

te_status te_layernorm_mlp_fwd(const void* x, const void* gamma, const void* beta, const void* kernel1,
                               const void* bias1, const void* kernel2, const void* bias2, int64_t rows,
                               int64_t hidden, int64_t ffn, te_dtype dtype, te_norm_type norm_type,
                               int zero_centered_gamma, float epsilon, te_act_type act_type, te_quant quant,
                               void* y, te_dtype y_dtype, const te_mlp_saved* saved, void* workspace,
                               size_t workspace_bytes, void* stream) {
  te_status st = check_dtype_quant(dtype, quant);
  if (st != TE_SUCCESS) return st;
  st = check_y_dtype(dtype, y_dtype);
  if (st != TE_SUCCESS) return st;
  st = check_norm(x, gamma, beta, rows, hidden, norm_type, epsilon);
  if (st != TE_SUCCESS) return st;
  TE_ARG(feature_ok(ffn), "ffn must be a positive multiple of 16 (at most 2^22), got %lld", (long long)ffn);
  TE_ARG(valid_act(act_type), "invalid act_type %d", (int)act_type);
  TE_REQUIRE(weight_ok(hidden, (is_gated(act_type) ? 2 : 1) * ffn, dtype) && weight_ok(ffn, hidden, dtype),
             TE_ERR_UNSUPPORTED, "kernels must be smaller than 2 GiB");
  TE_ARG(kernel1 != nullptr && kernel2 != nullptr && (y != nullptr || rows == 0),
         "kernel1, kernel2 and y are required");
  TE_ARG(aligned16(kernel1) && aligned16(kernel2) && aligned16(y) && (bias1 == nullptr || aligned16(bias1)) &&
             (bias2 == nullptr || aligned16(bias2)),
         "tensors must be 16-byte aligned");
  void* h1_user = saved ? saved->h1 : nullptr;
  float* mu = saved ? saved->mu : nullptr;
  float* rsigma = saved ? saved->rsigma : nullptr;
  TE_ARG(h1_user == nullptr || aligned16(h1_user), "saved->h1 must be 16-byte aligned");
  if (saved != nullptr)
    TE_ARG(aligned16(saved->xq) && aligned16(saved->w1q_t) && aligned16(saved->w2q_t) && aligned16(saved->actq),
           "saved code buffers must be 16-byte aligned");
  const size_t need = te_layernorm_mlp_fwd_workspace_size(rows, hidden, ffn, dtype, act_type, quant);
  TE_REQUIRE(workspace_bytes >= need, TE_ERR_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu bytes",
             workspace_bytes, need);
  TE_ARG(workspace != nullptr && aligned16(workspace), "workspace is required (16-byte aligned)");
  if (rows == 0) return ok();

  hipStream_t s = as_stream(stream);
  Carver c(workspace);
  MlpWs w = mlp_ws(c, rows, hidden, ffn, dtype, act_type, quant, true);
  const bool rms = norm_type == TE_RMSNORM, zcg = zero_centered_gamma != 0;
  const bool gated = is_gated(act_type);
  const int k = act_kind(act_type);
  const int64_t nb1 = (gated ? 2 : 1) * ffn;

  if (quant == TE_QUANT_NONE) {
    TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zcg, epsilon, te::kNormStore, dtype, w.xn, mu,
                           rsigma, nullptr, nullptr, nullptr, nullptr, s, w.t1), "norm");
    te::Epilogue e1{bias1, w.act, h1_user, nullptr, k, gated};
    e1.out_tiled = w.t2;
    te::Epilogue e2{bias2, y, nullptr, nullptr, te::kLinear, false};
    e2.out_f32 = dtype == TE_BF16 && y_dtype == TE_F32;
    if (dtype == TE_F32) {
      TE_HIP(te::launch_gemm_f32(static_cast<const float*>(w.xn), static_cast<const float*>(kernel1), rows, nb1,
                                 hidden, e1, s), "gemm1");
      TE_HIP(te::launch_gemm_f32(static_cast<const float*>(w.act), static_cast<const float*>(kernel2), rows,
                                 hidden, ffn, e2, s), "gemm2");
    } else {
      TE_HIP(te::launch_gemm_bf16(w.xn, kernel1, rows, nb1, hidden, e1, s, w.t1), "gemm1");
      TE_HIP(te::launch_gemm_bf16(w.act, kernel2, rows, hidden, ffn, e2, s, w.t2), "gemm2");
    }
    return ok();
  }

  Meta mx = pick_meta(saved ? &saved->x_meta : nullptr, w.metas);
  Meta m1 = pick_meta(saved ? &saved->w1_meta : nullptr, w.metas + 3);
  Meta ma = pick_meta(saved ? &saved->act_meta : nullptr, w.metas + 6);
  Meta m2 = pick_meta(saved ? &saved->w2_meta : nullptr, w.metas + 9);
  void* h1 = h1_user != nullptr ? h1_user : w.h1;
  // a caller's code buffer replaces the workspace one and is written row-major
  bool tx = w.t1, tw1 = w.t1, tw2 = w.t2, ta = w.t2;
  if (saved != nullptr) {
    if (saved->xq != nullptr) { w.xn = saved->xq; tx = false; }
    if (saved->w1q_t != nullptr) { w.w1t = saved->w1q_t; tw1 = false; }
    if (saved->w2q_t != nullptr) { w.w2t = saved->w2q_t; tw2 = false; }
    if (saved->actq != nullptr) { w.act = saved->actq; ta = false; }
  }
  // the amax slots raised by atomics (both kernels' and act's; x's is
  // written) are zeroed by the first pass, with the workspace metas
  te::ClearList clear;
  clear.first = w.metas;
  clear.n = 12;
  int nclear = 0;
  for (const Meta* m : {&m1, &ma, &m2})
    if (m->amax < w.metas || m->amax >= w.metas + 12) clear.one[nclear++] = m->amax;
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zcg, epsilon, te::kNormAmax, TE_E4M3, nullptr, mu,
                         rsigma, nullptr, nullptr, nullptr, w.npart, s, false, &clear), "norm amax");
  TE_HIP(te::launch_amax2(kernel1, hidden * nb1, m1.amax, kernel2, ffn * hidden, m2.amax, dtype, s), "kernel amax");
  TE_HIP(te::launch_norm(x, gamma, beta, rows, hidden, dtype, rms, zcg, epsilon, te::kNormQuant, TE_E4M3, w.xn,
                         nullptr, nullptr, mx.amax, mx.scale, mx.scale_inv, w.npart, s, tx), "norm quantise");
  TE_HIP(te::launch_quantize_transpose2(kernel1, hidden, nb1, w.w1t, m1.amax, m1.scale, m1.scale_inv, kernel2, ffn,
                                        hidden, w.w2t, m2.amax, m2.scale, m2.scale_inv, dtype, s, tw1, tw2,
                                        gated && tw1 ? ffn : 0),
         "kernel quantise");
  te::Epilogue e1{bias1, nullptr, h1, ma.amax, k, gated};
  TE_HIP(te::launch_gemm_fp8(static_cast<const uint8_t*>(w.xn), w.w1t, rows, nb1, hidden, mx.amax, m1.amax, e1, s,
                             tx, tw1),
         "fp8 gemm1");
  TE_HIP(te::launch_act(h1, rows, ffn, TE_BF16, k, gated, 2, w.act, TE_E4M3, ma.amax, ma.scale, ma.scale_inv, s,
                        ta),
         "act quantise");
  te::Epilogue e2{bias2, y, nullptr, nullptr, te::kLinear, false};
  e2.out_f32 = y_dtype == TE_F32;
  TE_HIP(te::launch_gemm_fp8(static_cast<const uint8_t*>(w.act), w.w2t, rows, hidden, ffn, ma.amax, m2.amax, e2, s,
                             ta, tw2),
         "fp8 gemm2");
  return ok();
}

}  // extern "C"
