// gfx950 memory primitives shared by the MFMA GEMMs: buffer resources with
// hardware range checking, direct global->LDS loads and the transposing LDS
// read.
//
// buffer_load ... lds: each lane of the wave fetches 16 bytes at
// base + voffset + soffset and the wave writes them to LDS at
// M0 + 16 * lane, i.e. one instruction fills 1 KiB of LDS in lane order.
// Offsets at or beyond the resource's num_records read as zero, which the
// GEMMs use for ragged tiles instead of branches.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, the four 8-byte chunks
// addressed by lanes 4i .. 4i+3 form row i (16 consecutive 16-bit values)
// and lane j of the group receives element j of rows 0..3. With row i = B[k+i]
// [n .. n+15] this hands lane j the four consecutive k values of column n+j,
// the layout the MFMA wants for its B operand.
#pragma once

#include "te_common.hpp"

namespace te {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Word 3 of a raw (untyped, stride 0) buffer descriptor on the gfx9 family.
constexpr int kBufferWord3 = 0x00020000;
// A byte offset that is always beyond num_records: the load returns zeros.
constexpr uint32_t kOffNone = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// 16 bytes per lane from the buffer into LDS at lds (wave-uniform) + 16 * lane.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ i16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

// Wait until at most N vector-memory loads (including LDS-DMA) of the wave
// are still in flight (gfx9 s_waitcnt encoding: vmcnt split over bits 3:0 and
// 15:14; expcnt and lgkmcnt left at their maxima so they are not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// As wait_vmcnt<N>(), and also wait for every LDS read of the wave.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// would wait for every outstanding load (vmcnt 0) and drain the LDS-DMA
// pipeline. LDS-DMA completion is ordered explicitly with wait_vmcnt<N>()
// before the barrier, and every LDS read of a stage completes before its
// MFMAs issue; the empty asm statements keep the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk slot swizzle for a tile whose rows hold CPR 16-byte chunks: slot =
// chunk ^ swz(row). Rows r .. r + 15 read at the same chunk then fall on 16
// distinct 4-dword bank groups (row stride CPR * 4 dwords, 64 banks).
template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}

// Byte offset of byte kb of row `row` of a tiled GEMM operand (te_kernels.hpp)
// with nks k stages per row tile and the given split (0: plain).
__device__ __forceinline__ int64_t tiled_offset(int64_t row, int64_t kb, int64_t nks, int64_t split) {
  int64_t t;
  int r;
  if (split > 0) {
    const bool hi = row >= split;
    const int64_t q = hi ? row - split : row;
    t = q >> 7;
    r = (int)(q & 127) + (hi ? 128 : 0);
  } else {
    t = row >> 8;
    r = (int)(row & 255);
  }
  const int c = (int)(kb >> 4) & 3;
  return ((t * nks + (kb >> 6)) << kTiledBlockShift) + r * 64 + ((c ^ chunk_swizzle<4>(r)) << 4) + (kb & 15);
}

}  // namespace te
