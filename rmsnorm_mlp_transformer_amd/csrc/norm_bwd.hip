// Row-wise LayerNorm / RMSNorm backward for gfx950: dx, dgamma and dbeta from
// dy, x and the forward's saved statistics ("NVIDIA TransformerEngine JAX
// LayerNorm Dense", Description: the backward pass gives the gradients of
// every input, x, gamma and beta among them, from the saved forward context).
//
// With xhat = (x - mean) * rsigma (RMSNorm: x * rsigma), g = gamma or
// 1 + gamma, and dxhat = dy * g:
//   LayerNorm: dx = rsigma * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))
//   RMSNorm:   dx = rsigma * (dxhat - xhat * mean(dxhat * xhat))
//   dgamma = sum over rows of dy * xhat, dbeta = sum over rows of dy.
//
// A workgroup of 16 waves is split into teams of TW waves; a team owns one
// row at a time, each lane holding CPL 16-byte chunks of it (one for rows of
// up to 8192 bf16 / 4096 fp32 values, two for wider ones, so a row of up to
// CPL * 64 * TW chunks). Each team keeps the raw chunks of its next DEPTH
// rows in flight in a register ring while it reduces the current one. The
// two row means are reduced across the team through LDS (one barrier per
// row, double-buffered; the barrier waits for LDS only, so the prefetched
// loads stay in flight). The column sums for dgamma and dbeta stay in
// registers across the workgroup's rows; at the end the teams add theirs in
// a fixed order through LDS and the workgroup writes one row of fp32
// partials, which a second kernel sums over the workgroups in a fixed order
// (bitwise reproducible).
#include "te_common.hpp"
#include "te_kernels.hpp"
#include "gemm_lds.hpp"

namespace te {
namespace {

constexpr int kBwdWaves = 16;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdColFloats = 30720;          // LDS for the teams' column sums (120 KiB)
// rows in flight per team beyond the one being reduced
#ifndef TE_NORM_BWD_DEPTH
#define TE_NORM_BWD_DEPTH 1
#endif
constexpr int kBwdDepth = TE_NORM_BWD_DEPTH;

template <bool BF16>
struct Chunk {
  static constexpr int VEC = BF16 ? 8 : 4;    // elements per 16-byte chunk
  static __device__ __forceinline__ void unpack(const uint4& c, float* f) {
    if constexpr (BF16) {
      f[0] = bf16_lo(c.x); f[1] = bf16_hi(c.x); f[2] = bf16_lo(c.y); f[3] = bf16_hi(c.y);
      f[4] = bf16_lo(c.z); f[5] = bf16_hi(c.z); f[6] = bf16_lo(c.w); f[7] = bf16_hi(c.w);
    } else {
      f[0] = __uint_as_float(c.x); f[1] = __uint_as_float(c.y);
      f[2] = __uint_as_float(c.z); f[3] = __uint_as_float(c.w);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    if constexpr (BF16) {
      return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                        pack_bf16x2(f[6], f[7]));
    } else {
      return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
  }
};

struct BwdArgs {
  const void* dy; const void* x; const float* mu; const float* rsigma; const void* gamma;
  int64_t rows, hidden; int zcg; int tw;      // waves per team (1, 2, 4, 8 or 16)
  int64_t rows_per_block;
  void* dx; float* part_g; float* part_b;     // partials [gridDim.x, hidden] (nullable)
};

// One row's raw data: the lane's chunks of dy and x and the row's statistics.
template <int CPL>
struct RowRaw {
  i32x4_t dy[CPL], x[CPL];
  float mu, rs;
};

template <bool BF16, bool RMS, int CPL, int DEPTH>
__global__ void __launch_bounds__(kBwdThreads) norm_bwd_kernel(BwdArgs a) {
  using C = Chunk<BF16>;
  constexpr int VEC = C::VEC;
  constexpr int R = DEPTH + 1;                // ring slots
  __shared__ float red[2][kBwdWaves][2];
  __shared__ float colbuf[kBwdColFloats];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int tw = a.tw, teams = kBwdWaves / tw;
  const int team = wave / tw, wt = wave % tw;
  const int64_t nch = a.hidden / VEC;
  const float inv_h = 1.0f / (float)a.hidden;
  // the lane's chunks of a row
  int64_t ch[CPL];
  bool cv[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    ch[j] = (int64_t)j * tw * 64 + wt * 64 + lane;
    cv[j] = ch[j] < nch;
  }
  // Row vectors are read and written through a buffer resource over the one
  // row (empty for a row past the end): chunks outside it read as zero and
  // their stores are dropped, with no branch around the 16-byte accesses.
  const uint32_t row_bytes = (uint32_t)(nch * 16);
  auto rsrc_of = [&](const void* base, int64_t row, bool valid) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(base) + (valid ? row : 0) * (int64_t)row_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, valid ? (int)row_bytes : 0,
                                             0x00020000);
  };
  auto unpack = [&](const i32x4_t& v, float* f) {
    C::unpack(make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]), f);
  };
  float g[CPL][VEC];
  const __amdgpu_buffer_rsrc_t rg = rsrc_of(a.gamma, 0, true);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    unpack(__builtin_amdgcn_raw_buffer_load_b128(rg, (uint32_t)ch[j] * 16, 0, 0), g[j]);
#pragma unroll
    for (int i = 0; i < VEC; ++i) g[j][i] = a.zcg ? 1.0f + g[j][i] : g[j][i];
  }
  float acc_g[CPL][VEC], acc_b[CPL][VEC];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int i = 0; i < VEC; ++i) { acc_g[j][i] = 0.0f; acc_b[j][i] = 0.0f; }

  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
  const int64_t r1 = min(r0 + a.rows_per_block, a.rows);
  // the same number of iterations in every team, a multiple of the ring size
  const int64_t iters = (a.rows_per_block + teams - 1) / teams;
  const int64_t iters_r = (iters + R - 1) / R * R;
  // The statistics go through buffer loads as well (every lane reads the
  // row's value), so that they are counted with the row's chunks; a row past
  // the end reads 0 for rsigma (empty range), which zeroes its xhat.
  auto stat_rsrc = [&](const float* base, int64_t row, bool valid) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base) + (valid ? row : 0), (short)0,
                                             valid ? 4 : 0, 0x00020000);
  };
  auto issue = [&](int64_t it, RowRaw<CPL>& w) {
    const int64_t row = r0 + it * teams + team;
    const bool rv = row < r1;
    const __amdgpu_buffer_rsrc_t rdy = rsrc_of(a.dy, row, rv), rx = rsrc_of(a.x, row, rv);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      w.dy[j] = __builtin_amdgcn_raw_buffer_load_b128(rdy, (uint32_t)ch[j] * 16, 0, kBufAuxStream);
      w.x[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)ch[j] * 16, 0, kBufAuxStream);
    }
    if constexpr (!RMS)
      w.mu = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(stat_rsrc(a.mu, row, rv), 0, 0, 0));
    else
      w.mu = 0.0f;
    w.rs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(stat_rsrc(a.rsigma, row, rv), 0, 0, 0));
  };
  auto process = [&](int64_t it, const RowRaw<CPL>& w) {
    const int64_t row = r0 + it * teams + team;
    const bool rv = row < r1;
    float dyv[CPL][VEC], xh[CPL][VEC];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float xv[VEC];
      unpack(w.dy[j], dyv[j]);
      unpack(w.x[j], xv);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        xh[j][i] = cv[j] ? (RMS ? xv[i] : xv[i] - w.mu) * w.rs : 0.0f;
        const float dxh = dyv[j][i] * g[j][i];
        s1 += dxh;
        s2 += dxh * xh[j][i];
      }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const int buf = (int)(it & 1);
    if (lane == 0) {
      red[buf][wave][0] = s1;
      red[buf][wave][1] = s2;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes are done (lgkmcnt 0)
    block_barrier();
    float t1 = 0.0f, t2 = 0.0f;
    for (int k = 0; k < tw; ++k) {              // fixed order over the team's waves
      t1 += red[buf][team * tw + k][0];
      t2 += red[buf][team * tw + k][1];
    }
    const float m1 = RMS ? 0.0f : t1 * inv_h, m2 = t2 * inv_h;
    const __amdgpu_buffer_rsrc_t rdx = rsrc_of(a.dx, row, rv);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float d[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        d[i] = w.rs * (dyv[j][i] * g[j][i] - m1 - xh[j][i] * m2);
        acc_g[j][i] += dyv[j][i] * xh[j][i];   // dy and xhat are 0 outside the row
        acc_b[j][i] += dyv[j][i];
      }
      const uint4 o = C::pack(d);
      __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{(int)o.x, (int)o.y, (int)o.z, (int)o.w}, rdx,
                                             (uint32_t)ch[j] * 16, 0, 0);
    }
  };
  RowRaw<CPL> ring[R];
#pragma unroll
  for (int q = 0; q < DEPTH; ++q) issue(q, ring[q]);
  for (int64_t it0 = 0; it0 < iters_r; it0 += R) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      issue(it0 + q + DEPTH, ring[(q + DEPTH) % R]);
      __builtin_amdgcn_sched_barrier(0);
      process(it0 + q, ring[q]);
    }
  }
  if (a.part_g == nullptr) return;   // no parameter gradients requested (uniform)

  // teams 1.. hand their column sums to team 0 through LDS; team 0 adds them in
  // team order and writes the workgroup's partial row
  const int nb = RMS ? 1 : 2;
  __syncthreads();
  if (team > 0) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if (cv[j]) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int64_t col = ch[j] * VEC + i;
          colbuf[((team - 1) * nb + 0) * a.hidden + col] = acc_g[j][i];
          if constexpr (!RMS) colbuf[((team - 1) * nb + 1) * a.hidden + col] = acc_b[j][i];
        }
      }
    }
  }
  __syncthreads();
  if (team == 0) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if (cv[j]) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const int64_t col = ch[j] * VEC + i;
          float sg = acc_g[j][i], sb = acc_b[j][i];
          for (int t = 1; t < teams; ++t) {
            sg += colbuf[((t - 1) * nb + 0) * a.hidden + col];
            if constexpr (!RMS) sb += colbuf[((t - 1) * nb + 1) * a.hidden + col];
          }
          a.part_g[(int64_t)blockIdx.x * a.hidden + col] = sg;
          if constexpr (!RMS) a.part_b[(int64_t)blockIdx.x * a.hidden + col] = sb;
        }
      }
    }
  }
}

// Sum of the per-workgroup partial rows: 16 threads per column each add a
// fixed, contiguous range of rows, then one of them adds the 16 results in
// order (a fixed order: bitwise reproducible). blockIdx.y selects the
// parameter (0: dgamma, 1: dbeta), so both sums take one launch; the row
// loop is unrolled so that four loads per thread are in flight.
struct FinJob {
  const float* part;
  void* out;            // nullable: the parameter is not wanted
};
template <int OUT>
__global__ void __launch_bounds__(256) param_finalize_kernel(FinJob j0, FinJob j1, int64_t blocks, int64_t n) {
  constexpr int S = 16;
  __shared__ float red[S][16];
  const FinJob& j = blockIdx.y == 0 ? j0 : j1;
  if (j.out == nullptr) return;   // uniform across the workgroup
  const int cl = threadIdx.x % 16, sp = threadIdx.x / 16;
  const int64_t c = (int64_t)blockIdx.x * 16 + cl;
  const int64_t per = (blocks + S - 1) / S;
  const int64_t k0 = sp * per, k1 = min(k0 + per, blocks);
  float s = 0.0f;
  if (c < n) {
    int64_t k = k0;
    for (; k + 4 <= k1; k += 4) {
      const float a0 = j.part[k * n + c], a1 = j.part[(k + 1) * n + c];
      const float a2 = j.part[(k + 2) * n + c], a3 = j.part[(k + 3) * n + c];
      s += a0;
      s += a1;
      s += a2;
      s += a3;
    }
    for (; k < k1; ++k) s += j.part[k * n + c];
  }
  red[sp][cl] = s;
  __syncthreads();
  if (sp == 0 && c < n) {
    float t = red[0][cl];
#pragma unroll
    for (int q = 1; q < S; ++q) t += red[q][cl];
    if constexpr (OUT == kBF16) reinterpret_cast<uint16_t*>(j.out)[c] = f32_to_bf16(t);
    else reinterpret_cast<float*>(j.out)[c] = t;
  }
}

}  // namespace

// Chunks per lane: one while a row fits the 16 waves that way, else two.
int norm_bwd_chunks_per_lane(int64_t hidden, int dtype) {
  const int64_t nch = hidden / (dtype == kBF16 ? 8 : 4);
  return nch <= 64 * kBwdWaves ? 1 : 2;
}

int norm_bwd_team_waves(int64_t hidden, int dtype) {
  const int64_t nch = hidden / (dtype == kBF16 ? 8 : 4);
  const int cpl = norm_bwd_chunks_per_lane(hidden, dtype);
  int tw = 1;
  while (tw < kBwdWaves && cpl * 64 * (int64_t)tw < nch) tw *= 2;
  return cpl * 64 * (int64_t)tw >= nch ? tw : 0;
}

int64_t norm_bwd_blocks(int64_t rows, int64_t hidden, int dtype) {
  const int tw = norm_bwd_team_waves(hidden, dtype);
  if (tw == 0 || rows <= 0) return 0;
  const int64_t teams = kBwdWaves / tw;
  const int64_t want = (rows + teams - 1) / teams;   // at least one row per team
  return want < 256 ? want : 256;                    // one 16-wave workgroup per CU
}

bool norm_bwd_fits(int64_t hidden, int dtype) {
  const int tw = norm_bwd_team_waves(hidden, dtype);
  if (tw == 0) return false;
  const int64_t teams = kBwdWaves / tw;
  return (teams - 1) * 2 * hidden <= kBwdColFloats;
}

hipError_t launch_norm_bwd(const void* dy, const void* x, const float* mu, const float* rsigma, const void* gamma,
                           int64_t rows, int64_t hidden, int dtype, bool rms, bool zcg, void* dx, void* dgamma,
                           void* dbeta, int dparam_dtype, float* part_g, float* part_b, hipStream_t s) {
  const int tw = norm_bwd_team_waves(hidden, dtype);
  const int64_t blocks = norm_bwd_blocks(rows, hidden, dtype);
  if (tw == 0 || !norm_bwd_fits(hidden, dtype)) return hipErrorInvalidValue;
  const bool params = dgamma != nullptr || dbeta != nullptr;
  {
    LaunchScope scope("norm_bwd", s);
    BwdArgs a{dy, x, mu, rsigma, gamma, rows, hidden, zcg ? 1 : 0, tw, (rows + blocks - 1) / blocks, dx,
              params ? part_g : nullptr, params ? part_b : nullptr};
    const bool one = norm_bwd_chunks_per_lane(hidden, dtype) == 1;
#define TE_NBWD(B, RM) \
  (one ? launch_kernel(norm_bwd_kernel<B, RM, 1, kBwdDepth>, (unsigned)blocks, kBwdThreads, 0, s, a) \
       : launch_kernel(norm_bwd_kernel<B, RM, 2, 0>, (unsigned)blocks, kBwdThreads, 0, s, a))
    if (dtype == kBF16) {
      if (rms) TE_NBWD(true, true);
      else TE_NBWD(true, false);
    } else {
      if (rms) TE_NBWD(false, true);
      else TE_NBWD(false, false);
    }
#undef TE_NBWD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!params) return hipSuccess;
  LaunchScope scope("norm_bwd_finalize", s);
  const FinJob jg{part_g, dgamma}, jb{part_b, rms ? nullptr : dbeta};
  const dim3 g((unsigned)((hidden + 15) / 16), jb.out != nullptr ? 2u : 1u);
  if (dparam_dtype == kBF16) launch_kernel(param_finalize_kernel<kBF16>, g, 256, 0, s, jg, jb, blocks, hidden);
  else launch_kernel(param_finalize_kernel<kF32>, g, 256, 0, s, jg, jb, blocks, hidden);
  return hipGetLastError();
}

}  // namespace te
