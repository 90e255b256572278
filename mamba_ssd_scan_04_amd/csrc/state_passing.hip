// ssd_state_passing: the inter-chunk recurrence on chunk states.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2, the sequential loop
// h_{c+1} = (a_0 ... a_{Q-1} of chunk c) h_c + S_c with h_0 = 0 (or a given
// initial state) and h_final = h_{T/Q} (the state-passing / chunkwise mode of
// appendix B.3.2). The product of a chunk's decays is exp(cs_last).
//
// Every state element follows its own scalar recurrence, so the kernel is a
// pure stream: each thread owns E consecutive elements of one (batch, head)
// N x P state (E = 8, or 4 when the states are too few to give the chip
// enough wavefronts at 8) and walks the chunks in order, reading S_c and
// overwriting it in place with h_c (the state entering chunk c). The running
// state stays in fp32 registers whatever the storage type; the final state is
// transposed through LDS.
//
// Grid: (P*N / (256 E), head, batch), 256 threads.
#include "kernels.hpp"

namespace ssd {

// E consecutive state elements (one vector load or store) <-> fp32
template <typename ST, int E> struct Pack {
    typedef ST raw __attribute__((ext_vector_type(E)));
    static __device__ __forceinline__ raw load(const ST* p) {
        return *(const __attribute__((address_space(1))) raw*)p;
    }
    static __device__ __forceinline__ void widen(const raw& r, float (&v)[E]) {
#pragma unroll
        for (int k = 0; k < E; ++k) v[k] = to_f32(r[k]);
    }
    static __device__ __forceinline__ void store(ST* p, const float (&v)[E]) {
        raw r;
#pragma unroll
        for (int k = 0; k < E; ++k) r[k] = from_f32<ST>(v[k]);
        *(__attribute__((address_space(1))) raw*)p = r;
    }
};

constexpr int kPassWin = 8;          // chunks whose loads are in flight together
constexpr int kPassThreads = 256;

// Each thread owns E consecutive elements of one (batch, head) [P][N] state.
// The chunk states are read in windows of 8 chunks, the next window's loads
// issued before the current window is folded (h <- a h + S, storing h before
// each fold), so up to 16 loads per thread are in flight.
// VARLEN: packed documents; a chunk in which a document starts (the id of its
// last token differs from that of the token before the chunk, or from the
// first token's for chunk 0) passes no state on: its decay is 0 ("Transformers
// are SSMs", Knowl 8).
template <typename ST, int E, bool VARLEN>
__global__ __launch_bounds__(kPassThreads) void ssd_state_passing_kernel(Params p) {
    constexpr int kPassElems = E;
    // the block's rows of the final state, row stride N + 1 (no bank conflicts
    // on the transposed reads); at most 256 E / 16 rows
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
    using O = Pack<ST, E>;

    // the running state starts at h_0: zero, or the given initial state
    // ([N][P] per head, so element pr * N + n of the transposed state is
    // init[n * P + pr])
    float run[E];
#pragma unroll
    for (int k = 0; k < E; ++k) run[k] = 0.0f;
    if (p.init_state && live) {
        const float* ini = p.init_state + (b * H + h) * PN;
#pragma unroll
        for (int k = 0; k < E; ++k) {
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
                    float sv[E];
                    O::widen(cur[u], sv);
#pragma unroll
                    for (int k = 0; k < E; ++k) run[k] = a * run[k] + sv[k];
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
        for (int k = 0; k < E; ++k) fin_tile[((i0 + k) / N) * (N + 1) + (i0 + k) % N] = run[k];
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

template <typename ST, int E>
static hipError_t launch_sp(const Params& p, hipStream_t s) {
    const int64_t PN = p.headdim * p.dstate;
    const int64_t per_block = (int64_t)kPassThreads * E;
    dim3 grid((unsigned)((PN + per_block - 1) / per_block), (unsigned)p.nheads, (unsigned)p.batch);
    if (p.seq_idx)
        hipLaunchKernelGGL((ssd_state_passing_kernel<ST, E, true>), grid, dim3(kPassThreads), 0, s, p);
    else
        hipLaunchKernelGGL((ssd_state_passing_kernel<ST, E, false>), grid, dim3(kPassThreads), 0, s, p);
    return hipGetLastError();
}

// 8 elements per thread, or 4 when 8 would leave fewer than 8 wavefronts per
// compute unit (small states or few heads)
template <typename ST>
static hipError_t launch_sp_e(const Params& p, hipStream_t s) {
    const int64_t waves8 = p.batch * p.nheads * p.headdim * p.dstate / 8 / 64;
    return waves8 < 8 * (int64_t)device_cus() ? launch_sp<ST, 4>(p, s) : launch_sp<ST, 8>(p, s);
}

hipError_t launch_state_passing(const Params& p, int state_dtype, hipStream_t s) {
    return state_dtype == 1 ? launch_sp_e<bf16>(p, s) : launch_sp_e<float>(p, s);
}

}  // namespace ssd
