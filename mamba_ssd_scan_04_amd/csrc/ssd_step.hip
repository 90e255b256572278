// ssd_step: one token of the recurrence, for decoding.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 1, the linear
// (recurrent) form taken one token at a time: the inference mode whose memory
// per head is the N x P state alone. With the discretisation of the forward
// path (dt, the per-head A, the skip term D):
//
//   state[b,h] <- exp(dt[b,h] A[h]) state[b,h] + dt[b,h] B[b,g] x[b,h]^T
//   y[b,h]      = C[b,g]^T state[b,h] + D[h] x[b,h]
//
// The state is [N][P] per head in fp32, the layout of the forward's final
// state (so a prompt's final state continues here), updated in place. The
// kernel streams the states: one workgroup per (head, batch); a thread owns 4
// consecutive p of every (256 / (P/4))-th row n, updates them with 16-byte
// loads and stores (consecutive threads cover a row), and accumulates its
// part of C^T state; the parts are summed over the row groups through LDS.
#include "kernels.hpp"

namespace ssd {

constexpr int kStepThreads = 256;

template <typename T>
__global__ __launch_bounds__(kStepThreads) void ssd_step_kernel(Params p) {
    __shared__ f32x4 part[kStepThreads];
    const int64_t H = p.nheads, P = p.headdim, N = p.dstate, G = p.ngroups;
    const int64_t h = blockIdx.x, b = blockIdx.y;
    const int64_t g = h / p.heads_per_group;
    const int tpr = (int)P / 4;               // threads per state row
    const int ngrp = kStepThreads / tpr;      // row groups
    const int t = threadIdx.x, pq = t % tpr, rg = t / tpr;
    const int p0 = pq * 4;

    const float dtv = p.dt[b * H + h];
    const float a = expf(dtv * p.A[h]);
    const T* xh = static_cast<const T*>(p.x) + (b * H + h) * P + p0;
    float xv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) xv[k] = to_f32(xh[k]);
    const T* Bg = static_cast<const T*>(p.B) + (b * G + g) * N;
    const T* Cg = static_cast<const T*>(p.C) + (b * G + g) * N;
    float* st = p.final_state + (b * H + h) * N * P + p0;

    f32x4 acc;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = 0.0f;
    for (int64_t n = rg; n < N; n += ngrp) {
        f32x4 hv = *(const __attribute__((address_space(1))) f32x4*)(st + n * P);
        const float u = dtv * to_f32(Bg[n]);
        const float c = to_f32(Cg[n]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hv[k] = a * hv[k] + u * xv[k];
            acc[k] += c * hv[k];
        }
        stg(reinterpret_cast<f32x4*>(st + n * P), hv);
    }
    part[t] = acc;
    __syncthreads();
    if (rg == 0) {
        f32x4 s = part[pq];
        for (int r = 1; r < ngrp; ++r) {
            const f32x4 v = part[r * tpr + pq];
#pragma unroll
            for (int k = 0; k < 4; ++k) s[k] += v[k];
        }
        const float Dh = p.D[h];
        T* yh = static_cast<T*>(p.y) + (b * H + h) * P + p0;
#pragma unroll
        for (int k = 0; k < 4; ++k) yh[k] = from_f32<T>(s[k] + Dh * xv[k]);
    }
}

hipError_t launch_step(const Params& p, int dtype, hipStream_t s) {
    dim3 grid((unsigned)p.nheads, (unsigned)p.batch);
    if (dtype == 1)
        hipLaunchKernelGGL(ssd_step_kernel<bf16>, grid, dim3(kStepThreads), 0, s, p);
    else
        hipLaunchKernelGGL(ssd_step_kernel<float>, grid, dim3(kStepThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace ssd
