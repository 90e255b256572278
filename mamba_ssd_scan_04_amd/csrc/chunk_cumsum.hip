// ssd_chunk_cumsum: in-chunk cumulative decay in log space.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2, first step of the
// block decomposition: the running products of the decays inside each chunk.
// With a_t = exp(dt_t * A_h) the cumulative product over a chunk is exp of the
// inclusive prefix sum of dt_t * A_h; keeping the sum (not the product) avoids fp32 underflow within a
// chunk. The prefix is a parallel (Hillis-Steele) scan across a wavefront,
// the parallel associative scan of the paper's appendix B.2.2.
//
// Grid: (chunk, head block of 16, batch); 256 threads. The [Q x 16] block of
// dt is read row-wise into LDS (64 contiguous bytes per token), then each
// wavefront scans 4 heads, one head at a time: lane l owns Q/64 consecutive
// tokens, scans them serially, and a wavefront scan of the lane totals gives
// the offsets. The result row cs[b, h, c, 0:Q] is written contiguously.
// Tokens past the end of the sequence count as dt = 0, so a short last chunk
// repeats its final value.
#include "kernels.hpp"

namespace ssd {

constexpr int kCsHeads = 16;
constexpr int kMaxQ = 256;

__global__ __launch_bounds__(256) void ssd_chunk_cumsum_kernel(Params p) {
    __shared__ float tile[kMaxQ][kCsHeads + 1];
    const int c = blockIdx.x;
    const int h0 = blockIdx.y * kCsHeads;
    const int64_t b = blockIdx.z;
    const int Q = (int)p.chunk;
    const int64_t T = p.seqlen, H = p.nheads;
    const int nh = (int)min<int64_t>(kCsHeads, H - h0);
    const int64_t t0 = (int64_t)c * Q;
    const int qc = (int)min<int64_t>(Q, T - t0);   // real tokens in this chunk

    for (int idx = threadIdx.x; idx < Q * kCsHeads; idx += blockDim.x) {
        const int j = idx / kCsHeads, hh = idx % kCsHeads;
        const int64_t t = t0 + j;
        float v = 0.0f;
        if (hh < nh && t < T) v = p.dt[(b * T + t) * H + h0 + hh] * p.A[h0 + hh];
        tile[j][hh] = v;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per = Q >= 64 ? Q / 64 : 1;    // tokens per lane
    const int active = Q / per;              // lanes holding tokens
    for (int hh = wave; hh < nh; hh += 4) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (k < per && lane < active) ? tile[lane * per + k][hh] : 0.0f;
        chunk_prefix(v, per, active, qc, lane);
        float* out = p.cs + ((b * H + h0 + hh) * p.nchunks + c) * Q;
        if (lane < active) {
            if (per == 4) {
                f32x4 o;
                o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
                *reinterpret_cast<f32x4*>(out + lane * 4) = o;
            } else {
                for (int k = 0; k < per; ++k) out[lane * per + k] = v[k];
            }
        }
    }
}

hipError_t launch_chunk_cumsum(const Params& p, hipStream_t s) {
    dim3 grid((unsigned)p.nchunks, (unsigned)((p.nheads + kCsHeads - 1) / kCsHeads), (unsigned)p.batch);
    hipLaunchKernelGGL(ssd_chunk_cumsum_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void ssd_zero_fill_kernel(float* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = 0.0f;
}

hipError_t launch_zero_fill(float* dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(ssd_zero_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, n);
    return hipGetLastError();
}

}  // namespace ssd
