// ssd_chunk_state: the right-factor state of every chunk.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2, step "compute right
// factor chunk state S = B^T (decayed X)". "Decayed" is read as: token j of
// the chunk is scaled by the decay from j to the chunk's end,
// exp(cs_last - cs_j) = a_{j+1} ... a_{last} (so that chaining chunk states
// reproduces the recurrence exactly), and by its step dt_j (the input term of
// the discretised recurrence). Per (batch, chunk, head):
//
//   S^T[p, n] = sum_j  x[j, p] * w_j * B[j, n],   w_j = exp(cs_last - cs_j) * dt_j
//
// a (P x Q) . (Q x N) product on the matrix cores. The product is stored
// transposed ([P][N], n contiguous) because the chunk scan consumes the
// carried state as a k-major (n-contiguous) operand.
//
// Grid: (chunk, head, batch), 256 threads = 4 wavefronts. The chunk's tokens
// are consumed in blocks of 64: x (scaled by w in fp32, then rounded to the
// operand type) and B are staged transposed in LDS, and every wavefront
// accumulates its share of the (P/32) x (N/32) output tiles.
#include "kernels.hpp"
#include "transpose.hpp"

namespace ssd {

constexpr int kStateKB = 64;
constexpr int kMaxChunk = 256;

template <typename T, int PT, int NT, typename ST>
__global__ __launch_bounds__(256) void ssd_chunk_state_kernel(Params p) {
    constexpr int PP = PT * 32, NP = NT * 32;
    constexpr int LD = kStateKB + 16 / (int)sizeof(T);     // 16-byte row padding
    constexpr int TILES = PT * NT, TPW = (TILES + 3) / 4;
    constexpr int XSB = (kStateKB / 8) * (PP / 8);          // 8x8 blocks of x per token block
    constexpr int NSB = XSB + (kStateKB / 8) * (NP / 8);
    __shared__ __attribute__((aligned(16))) T xs[PP * LD];
    __shared__ __attribute__((aligned(16))) T bs[NP * LD];
    __shared__ float wts[kMaxChunk];

    const int c = blockIdx.x;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int Q = (int)p.chunk;
    const int64_t TL = p.seqlen, H = p.nheads, P = p.headdim, N = p.dstate, G = p.ngroups;
    const int64_t g = h / p.heads_per_group;
    const int64_t t0 = (int64_t)c * Q;
    const float* csrow = p.cs + ((b * H + h) * p.nchunks + c) * Q;
    const float last = csrow[Q - 1];
    for (int j = threadIdx.x; j < Q; j += blockDim.x) {
        const int64_t t = t0 + j;
        wts[j] = (t < TL) ? exp2f((last - csrow[j]) * kLog2e) * p.dt[(b * TL + t) * H + h] : 0.0f;
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hf = lane >> 5, l32 = lane & 31;
    f32x16 acc[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) acc[k] = zero16();

    const T* xg = static_cast<const T*>(p.x);
    const T* bg = static_cast<const T*>(p.B);
    for (int kb = 0; kb < Q; kb += kStateKB) {
        __syncthreads();  // wts ready (first block) / previous block consumed
        for (int sb = threadIdx.x; sb < NSB; sb += blockDim.x) {
            const bool isx = sb < XSB;
            const int s2 = isx ? sb : sb - XSB;
            const int ngrp = isx ? PP / 8 : NP / 8;
            const int col = (s2 % ngrp) * 8, tg = s2 / ngrp;
            const int64_t limit = isx ? P : N;
            float v[8][8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int j = kb + tg * 8 + r;
                const int64_t t = t0 + j;
                const bool ok = (j < Q) && (t < TL) && (col < limit);
                const T* src = isx ? xg + ((b * TL + t) * H + h) * P + col
                                   : bg + ((b * TL + t) * G + g) * N + col;
                load_row8<T>(v[r], src, ok);
                if (isx) {
                    const float s = ok ? wts[j] : 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[r][e] *= s;
                }
            }
            store_transposed8<T>((isx ? xs : bs) + col * LD + tg * 8, LD, v);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kStateKB / 16; ++ks) {
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                const int tile = wave + 4 * k;
                if (tile < TILES) {
                    const int pt = tile / NT, nt = tile % NT;
                    const auto a = load8(xs + (pt * 32 + l32) * LD + ks * 16 + hf * 8);
                    const auto bb = load8(bs + (nt * 32 + l32) * LD + ks * 16 + hf * 8);
                    mma_k16(acc[k], a, bb);
                }
            }
        }
    }

    ST* sg = static_cast<ST*>(p.states) + ((b * p.nchunks + c) * H + h) * P * N;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int tile = wave + 4 * k;
        if (tile < TILES) {
            const int pt = tile / NT, nt = tile % NT;
            const int64_t n = nt * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t pr = pt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (pr < P && n < N) sg[pr * N + n] = from_f32<ST>(acc[k][r]);
            }
        }
    }
}

template <typename T, int PT, int NT, typename ST>
static hipError_t launch_cs(const Params& p, hipStream_t s) {
    dim3 grid((unsigned)p.nchunks, (unsigned)p.nheads, (unsigned)p.batch);
    hipLaunchKernelGGL((ssd_chunk_state_kernel<T, PT, NT, ST>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename T, typename ST>
static hipError_t dispatch_cs(const Params& p, hipStream_t s) {
    const int pt = (int)((p.headdim + 31) / 32), nt = (int)((p.dstate + 31) / 32);
#define SSD_CS_CASE(PT_, NT_) \
    if (pt == PT_ && nt == NT_) return launch_cs<T, PT_, NT_, ST>(p, s);
#define SSD_CS_ROW(PT_) SSD_CS_CASE(PT_, 1) SSD_CS_CASE(PT_, 2) SSD_CS_CASE(PT_, 4) SSD_CS_CASE(PT_, 8)
    SSD_CS_ROW(1) SSD_CS_ROW(2) SSD_CS_ROW(4)
#undef SSD_CS_ROW
#undef SSD_CS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_state(const Params& p, int dtype, int state_dtype, hipStream_t s) {
    if (dtype == 1 && state_dtype == 1) return dispatch_cs<bf16, bf16>(p, s);
    if (dtype == 1) return dispatch_cs<bf16, float>(p, s);
    return dispatch_cs<float, float>(p, s);
}

}  // namespace ssd
