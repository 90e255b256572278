// ssd_state_passing: the inter-chunk recurrence on chunk states.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2, the sequential loop
// h_{c+1} = (a_0 ... a_{Q-1} of chunk c) h_c + S_c with h_0 = 0 (or a given
// initial state) and h_final = h_{T/Q} (the state-passing / chunkwise mode of
// appendix B.3.2). The product of a chunk's decays is exp(cs_last).
//
// Every state element follows its own scalar recurrence, so the kernel is a
// pure stream: each thread owns 8 consecutive elements of one (batch, head)
// N x P state and walks the chunks in order, reading S_c and overwriting it in
// place with h_c (the state entering chunk c). The running state stays in
// fp32 registers whatever the storage type; the final state is transposed
// through LDS.
//
// Grid: (P*N / 2048, head, batch), 256 threads.
#include "kernels.hpp"

namespace ssd {

// 8 consecutive state elements <-> fp32
template <typename ST> struct Oct;
template <> struct Oct<float> {
    typedef f32x8 raw;
    static __device__ __forceinline__ raw load(const float* p) { return ldg8(p); }
    static __device__ __forceinline__ f32x8 widen(const raw& r) { return r; }
    static __device__ __forceinline__ void store(float* p, const f32x8& v) {
        f32x4 lo, hi;
        lo[0] = v[0]; lo[1] = v[1]; lo[2] = v[2]; lo[3] = v[3];
        hi[0] = v[4]; hi[1] = v[5]; hi[2] = v[6]; hi[3] = v[7];
        stg(reinterpret_cast<f32x4*>(p), lo);
        stg(reinterpret_cast<f32x4*>(p + 4), hi);
    }
};
template <> struct Oct<bf16> {
    typedef bf16x8 raw;
    static __device__ __forceinline__ raw load(const bf16* p) { return ldg8(p); }
    static __device__ __forceinline__ f32x8 widen(const raw& r) {
        f32x8 v;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = to_f32(r[k]);
        return v;
    }
    static __device__ __forceinline__ void store(bf16* p, const f32x8& v) {
        bf16x8 r;
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = from_f32<bf16>(v[k]);
        stg(reinterpret_cast<bf16x8*>(p), r);
    }
};

constexpr int kPassWin = 8;          // chunks whose loads are in flight together
constexpr int kPassThreads = 256;
constexpr int kPassElems = 8;        // consecutive state elements per thread

// Each thread owns 8 consecutive elements of one (batch, head) [P][N] state.
// The chunk states are read in windows of 8 chunks, the next window's loads
// issued before the current window is folded (h <- a h + S, storing h before
// each fold), so up to 16 loads per thread are in flight.
// VARLEN: packed documents; a chunk in which a document starts (the id of its
// last token differs from that of the token before the chunk, or from the
// first token's for chunk 0) passes no state on: its decay is 0 ("Transformers
// are SSMs", Knowl 8).
template <typename ST, bool VARLEN>
__global__ __launch_bounds__(kPassThreads) void ssd_state_passing_kernel(Params p) {
    // the block's rows of the final state, row stride N + 1 (no bank conflicts
    // on the transposed reads); at most 2048 / 16 = 128 rows
    __shared__ float fin_tile[kPassThreads * kPassElems + kPassThreads * kPassElems / 16];
    const int64_t H = p.nheads, P = p.headdim, N = p.dstate, Q = p.chunk, nc = p.nchunks;
    const int64_t PN = P * N;
    const int64_t e0 = (int64_t)blockIdx.x * kPassThreads * kPassElems;   // first element of the block
    const int64_t e = e0 + (int64_t)threadIdx.x * kPassElems;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const bool live = e < PN;
    const float* lam = p.cs + (b * H + h) * nc * Q + (Q - 1);   // chunk c's total at lam[c*Q]
    ST* st = static_cast<ST*>(p.states) + (b * nc * H + h) * PN + (live ? e : 0);
    const int64_t cstride = H * PN;
    using O = Oct<ST>;

    // the running state starts at h_0: zero, or the given initial state
    // ([N][P] per head, so element pr * N + n of the transposed state is
    // init[n * P + pr])
    f32x8 run;
#pragma unroll
    for (int k = 0; k < 8; ++k) run[k] = 0.0f;
    if (p.init_state && live) {
        const float* ini = p.init_state + (b * H + h) * PN;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t i = e + k, pr = i / N, n = i % N;
            run[k] = ini[n * P + pr];
        }
    }
    typename O::raw cur[kPassWin], nxt[kPassWin];
    float acur[kPassWin], anxt[kPassWin];
    const int* sq = VARLEN ? p.seq_idx + b * p.seqlen : nullptr;
    auto load_win = [&](typename O::raw (&w)[kPassWin], float (&a)[kPassWin], int64_t c0) {
#pragma unroll
        for (int u = 0; u < kPassWin; ++u) {
            const int64_t c = c0 + u < nc ? c0 + u : nc - 1;   // clamped: extra loads repeat the last chunk
            w[u] = O::load(st + c * cstride);
            a[u] = lam[c * Q];
            if constexpr (VARLEN) {
                const int64_t tl = min<int64_t>((c + 1) * Q, p.seqlen) - 1, tp = c > 0 ? c * Q - 1 : 0;
                if (sq[tl] != sq[tp]) a[u] = -INFINITY;   // exp gives exactly 0
            }
        }
    };
    if (live) load_win(cur, acur, 0);
    for (int64_t c0 = 0; c0 < nc; c0 += kPassWin) {
        if (live && c0 + kPassWin < nc) load_win(nxt, anxt, c0 + kPassWin);
        if (live) {
#pragma unroll
            for (int u = 0; u < kPassWin; ++u) {
                if (c0 + u < nc) {
                    O::store(st + (c0 + u) * cstride, run);
                    const float a = exp2f(acur[u] * kLog2e);
                    const f32x8 sv = O::widen(cur[u]);
#pragma unroll
                    for (int k = 0; k < 8; ++k) run[k] = a * run[k] + sv[k];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kPassWin; ++u) {
            cur[u] = nxt[u];
            acur[u] = anxt[u];
        }
    }
    // element e0 + i = pr * N + n of the transposed [P][N] state goes to the
    // final state [N][P]: through LDS, so that a thread writes whole rows of
    // the block's (p range) x (n) tile
    if (live) {
        const int64_t i0 = (int64_t)threadIdx.x * kPassElems;   // element i0 + k = r * N + n of the block
#pragma unroll
        for (int k = 0; k < 8; ++k) fin_tile[((i0 + k) / N) * (N + 1) + (i0 + k) % N] = run[k];
    }
    __syncthreads();
    const int64_t rows = (PN - e0) < (int64_t)kPassThreads * kPassElems ? (PN - e0) / N
                                                                          : (int64_t)kPassThreads * kPassElems / N;
    const int64_t pr0 = e0 / N;
    float* fin = p.final_state + (b * H + h) * PN;
    // the tile holds rows pr0 .. pr0+rows-1 (all N columns); write column n
    // of those rows, i.e. fin[n][pr0 .. pr0+rows-1]
    for (int64_t i = threadIdx.x; i < rows * N; i += kPassThreads) {
        const int64_t n = i / rows, r = i % rows;
        fin[n * P + pr0 + r] = fin_tile[r * (N + 1) + n];
    }
}

template <typename ST>
static hipError_t launch_sp(const Params& p, hipStream_t s) {
    const int64_t PN = p.headdim * p.dstate;
    const int64_t per_block = (int64_t)kPassThreads * kPassElems;
    dim3 grid((unsigned)((PN + per_block - 1) / per_block), (unsigned)p.nheads, (unsigned)p.batch);
    if (p.seq_idx)
        hipLaunchKernelGGL((ssd_state_passing_kernel<ST, true>), grid, dim3(kPassThreads), 0, s, p);
    else
        hipLaunchKernelGGL((ssd_state_passing_kernel<ST, false>), grid, dim3(kPassThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_state_passing(const Params& p, int state_dtype, hipStream_t s) {
    return state_dtype == 1 ? launch_sp<bf16>(p, s) : launch_sp<float>(p, s);
}

}  // namespace ssd
