// The MFMA issue-rate probe behind te_probe_mfma (a measurement aid).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace te {

// blocks workgroups of 256 threads, each wave four chains of iters MFMAs
// (bf16, or E4M3 with fp8); sink: blocks * 256 floats; ticks: 2 uint64 or NULL.
hipError_t launch_mfma_probe(bool fp8, int64_t iters, int blocks, float* sink, uint64_t* ticks, hipStream_t s);

}  // namespace te
