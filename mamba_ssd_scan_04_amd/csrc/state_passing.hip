// ssd_state_passing: the inter-chunk recurrence on chunk states.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2, the sequential loop
// h_{c+1} = (a_0 ... a_{Q-1} of chunk c) h_c + S_c with h_0 = 0 and
// h_final = h_{T/Q} (the state-passing / chunkwise mode of appendix B.3.2).
// The product of a chunk's decays is exp(cs_last).
//
// Every state element follows its own scalar recurrence, so the kernel is a
// pure stream: each thread owns 4 consecutive elements of one (batch, head)
// N x P state and walks the chunks in order, reading S_c and overwriting it in
// place with h_c (the state entering chunk c). Loads for 4 chunks are issued
// before their stores so the memory system sees independent requests; the
// running state stays in fp32 registers whatever the storage type.
//
// Grid: (P*N / 1024, head, batch), 256 threads.
#include "kernels.hpp"

namespace ssd {

template <typename ST> struct Quad;
template <> struct Quad<float> {
    static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ void store(float* p, const f32x4& v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct Quad<bf16> {
    static __device__ __forceinline__ f32x4 load(const bf16* p) {
        const bf16x4 r = *reinterpret_cast<const bf16x4*>(p);
        f32x4 v;
        v[0] = to_f32(r[0]); v[1] = to_f32(r[1]); v[2] = to_f32(r[2]); v[3] = to_f32(r[3]);
        return v;
    }
    static __device__ __forceinline__ void store(bf16* p, const f32x4& v) {
        bf16x4 r;
        r[0] = from_f32<bf16>(v[0]); r[1] = from_f32<bf16>(v[1]);
        r[2] = from_f32<bf16>(v[2]); r[3] = from_f32<bf16>(v[3]);
        *reinterpret_cast<bf16x4*>(p) = r;
    }
};

constexpr int kPassUnroll = 4;

template <typename ST>
__global__ __launch_bounds__(256) void ssd_state_passing_kernel(Params p) {
    const int64_t H = p.nheads, P = p.headdim, N = p.dstate, Q = p.chunk, nc = p.nchunks;
    const int64_t PN = P * N;
    const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    if (e >= PN) return;
    const float* lam = p.cs + (b * H + h) * nc * Q + (Q - 1);   // chunk c's total at lam[c*Q]
    ST* st = static_cast<ST*>(p.states) + (b * nc * H + h) * PN + e;
    const int64_t cstride = H * PN;

    f32x4 run;
    run[0] = run[1] = run[2] = run[3] = 0.0f;
    for (int64_t c0 = 0; c0 < nc; c0 += kPassUnroll) {
        f32x4 s[kPassUnroll];
        float a[kPassUnroll];
#pragma unroll
        for (int u = 0; u < kPassUnroll; ++u) {
            if (c0 + u < nc) {
                s[u] = Quad<ST>::load(st + (c0 + u) * cstride);
                a[u] = exp2f(lam[(c0 + u) * Q] * kLog2e);
            }
        }
#pragma unroll
        for (int u = 0; u < kPassUnroll; ++u) {
            if (c0 + u < nc) {
                Quad<ST>::store(st + (c0 + u) * cstride, run);
                run = a[u] * run + s[u];
            }
        }
    }
    // element e = pr * N + n of the transposed [P][N] state -> final [N][P]
    const int64_t pr = e / N, n = e % N;
    float* fin = p.final_state + (b * H + h) * PN;
#pragma unroll
    for (int k = 0; k < 4; ++k) fin[(n + k) * P + pr] = run[k];
}

template <typename ST>
static hipError_t launch_sp(const Params& p, hipStream_t s) {
    const int64_t PN = p.headdim * p.dstate;
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)p.nheads, (unsigned)p.batch);
    hipLaunchKernelGGL((ssd_state_passing_kernel<ST>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_state_passing(const Params& p, int state_dtype, hipStream_t s) {
    return state_dtype == 1 ? launch_sp<bf16>(p, s) : launch_sp<float>(p, s);
}

}  // namespace ssd
