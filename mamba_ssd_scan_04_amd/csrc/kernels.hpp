// Host-side launchers of the four SSD kernels (each in its own .hip file).
#pragma once

#include <hip/hip_runtime.h>

#include "ssd_common.hpp"

namespace ssd {

// dtype/state dtype codes follow ssd_dtype: 0 = fp32, 1 = bf16.
hipError_t launch_chunk_cumsum(const Params& p, hipStream_t s);
hipError_t launch_chunk_state(const Params& p, int dtype, int state_dtype, hipStream_t s);
hipError_t launch_state_passing(const Params& p, int state_dtype, hipStream_t s);
hipError_t launch_chunk_scan(const Params& p, int dtype, int state_dtype, hipStream_t s);
hipError_t launch_zero_fill(float* dst, int64_t n, hipStream_t s);
hipError_t launch_step(const Params& p, int dtype, hipStream_t s);
hipError_t launch_total_decay(const float* dt, const float* A, float* total, int64_t batch, int64_t T, int64_t H,
                              hipStream_t s);
hipError_t launch_gated_rmsnorm(const void* y, const void* z, const float* w, float eps, int64_t rows, int64_t groups,
                                int64_t cg, void* out, int dtype, hipStream_t s);
hipError_t launch_fold(int64_t K, int64_t BH, int64_t NP, const float* totals, const float* finals, const float* init,
                       float* entering, hipStream_t s);

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus();

}  // namespace ssd
