// Attainable-peak probes for the roofline: what the matrix cores and HBM
// deliver on this chip when nothing else limits them, to set beside the
// datasheet peaks the kernels are reported against. Built into its own
// library (libssd_peak.so); nothing on the SSD path calls it.
//
//   ssd_peak_mfma_bf16   every wave issues a long chain of
//                        v_mfma_f32_32x32x16_bf16 on register operands, four
//                        independent accumulators deep so that the matrix
//                        pipe never waits on a result; 32*32*16*2 = 32768
//                        flop per instruction.
//   ssd_peak_stream      y = x over n 16-byte vectors, grid-stride, four
//                        non-temporal loads in flight per thread, then their
//                        stores: a plain read + write stream (bytes moved =
//                        2 * 16 * n).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 pk_bf16x8;
typedef __attribute__((ext_vector_type(16))) float pk_f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned pk_u32x4;

namespace {

constexpr int kAcc = 4;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* out) {
    pk_bf16x8 a, b;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(1.0f + 0.001f * (float)(lane + k));
        b[k] = (__bf16)(0.5f - 0.001f * (float)(lane - k));
    }
    pk_f32x16 acc[kAcc];
#pragma unroll
    for (int u = 0; u < kAcc; ++u)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[u][k] = 0.0f;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < kAcc; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kAcc; ++u)
#pragma unroll
        for (int k = 0; k < 16; ++k) s += acc[u][k];
    // one value per thread, so the chain cannot be dropped
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// grid-stride over groups of kUnroll vectors per thread: all of a group's
// loads are issued before its stores, so each wave keeps kUnroll loads in
// flight
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void stream_kernel(const pk_u32x4* __restrict__ x, pk_u32x4* __restrict__ y,
                                                     int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        pk_u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], y + i + u * stride);
    }
    for (; i < n; i += stride) y[i] = x[i];
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 256 threads (4 waves), each wave issuing
// iters * 4 MFMAs; out holds blocks * 256 floats. Total flop =
// blocks * 4 * iters * 4 * 32768. Returns a hipError_t value (0 = success).
int ssd_peak_mfma_bf16(int64_t blocks, int64_t iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, out);
    return (int)hipGetLastError();
}

// Copies n 16-byte vectors from x to y (both 16-byte aligned device buffers
// of at least 16 * n bytes) with `blocks` workgroups of 256 threads.
int ssd_peak_stream(const void* x, void* y, int64_t n, int64_t blocks, hipStream_t stream) {
    if (n <= 0 || blocks <= 0 || !x || !y) return (int)hipErrorInvalidValue;
    if (((uintptr_t)x | (uintptr_t)y) & 15) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const pk_u32x4*>(x), static_cast<pk_u32x4*>(y), n);
    return (int)hipGetLastError();
}

}  // extern "C"
