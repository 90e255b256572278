// Sequence (context) parallelism across shards of one long sequence.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 8: a long sequence is cut
// along T into K shards; each shard runs the SSD transform on its own tokens
// and only the boundary state h (N x P per head) passes from one shard to the
// next. A shard run from a zero state ends in its local final state F_k; the
// state entering shard k + 1 is then
//
//   H_{k+1} = exp(Lambda_k) H_k + F_k,   H_0 = the initial state (or 0),
//
// with Lambda_k = sum over the shard's tokens of dt_t A_h, the log of the
// product of its decays (the same step as the state passing between chunks,
// Knowl 2, one level up). Running shard k again from H_k gives its exact
// output. Two kernels:
//
//   ssd_total_decay_kernel  Lambda[b,h] = A_h * sum_t dt[b,t,h]: one thread per
//                           (b, h) and a 16-way split of t over the wavefronts
//                           of a workgroup, summed through LDS in a fixed order.
//   ssd_fold_kernel         the chain above for every state element: each
//                           thread owns 4 consecutive elements of one (b, h)
//                           state and walks the shards in order.
#include "kernels.hpp"

namespace ssd {

constexpr int kDecayLanes = 64;    // heads per workgroup
constexpr int kDecaySplit = 16;    // wavefronts per workgroup, each a residue class of t

__global__ __launch_bounds__(kDecayLanes * kDecaySplit) void ssd_total_decay_kernel(const float* __restrict__ dt,
                                                                                     const float* __restrict__ A,
                                                                                     float* __restrict__ total,
                                                                                     int64_t T, int64_t H) {
    __shared__ float part[kDecaySplit][kDecayLanes];
    const int lane = threadIdx.x % kDecayLanes, w = threadIdx.x / kDecayLanes;
    const int64_t h = (int64_t)blockIdx.x * kDecayLanes + lane, b = blockIdx.y;
    float acc = 0.0f;
    if (h < H) {
        const float* row = dt + b * T * H + h;
        for (int64_t t = w; t < T; t += kDecaySplit) acc += row[t * H];
    }
    part[w][lane] = acc;
    __syncthreads();
    if (w == 0 && h < H) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < kDecaySplit; ++k) s += part[k][lane];
        total[b * H + h] = s * A[h];
    }
}

__global__ __launch_bounds__(256) void ssd_fold_kernel(int64_t K, int64_t BH, int64_t NP,
                                                       const float* __restrict__ totals,
                                                       const float* __restrict__ finals,
                                                       const float* __restrict__ init, float* __restrict__ entering) {
    const int64_t E = BH * NP;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= E) return;
    const int64_t bh = i / NP;   // NP is a multiple of 4: the 4 elements share one (b, h)
    f32x4 run;
    if (init) {
        run = *reinterpret_cast<const f32x4*>(init + i);
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) run[r] = 0.0f;
    }
    for (int64_t k = 0; k < K; ++k) {
        *reinterpret_cast<f32x4*>(entering + k * E + i) = run;
        const float a = expf(totals[k * BH + bh]);
        const f32x4 f = *reinterpret_cast<const f32x4*>(finals + k * E + i);
#pragma unroll
        for (int r = 0; r < 4; ++r) run[r] = a * run[r] + f[r];
    }
    *reinterpret_cast<f32x4*>(entering + K * E + i) = run;
}

hipError_t launch_total_decay(const float* dt, const float* A, float* total, int64_t batch, int64_t T, int64_t H,
                              hipStream_t s) {
    dim3 grid((unsigned)((H + kDecayLanes - 1) / kDecayLanes), (unsigned)batch);
    hipLaunchKernelGGL(ssd_total_decay_kernel, grid, dim3(kDecayLanes * kDecaySplit), 0, s, dt, A, total, T, H);
    return hipGetLastError();
}

hipError_t launch_fold(int64_t K, int64_t BH, int64_t NP, const float* totals, const float* finals, const float* init,
                       float* entering, hipStream_t s) {
    const int64_t threads = BH * NP / 4;
    dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL(ssd_fold_kernel, grid, dim3(256), 0, s, K, BH, NP, totals, finals, init, entering);
    return hipGetLastError();
}

}  // namespace ssd
