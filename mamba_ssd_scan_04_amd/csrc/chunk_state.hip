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
// a (P x Q) . (Q x N) product on the matrix cores, stored transposed ([P][N],
// n contiguous) because the chunk scan consumes the carried state as a
// k-major operand.
//
// Work split. One workgroup (4 wavefronts) takes one chunk and up to HPW heads
// of one group, which share B. The chunk is consumed in blocks of 32 tokens,
// double-buffered in LDS: while the matrix cores work on block k, the copy
// engine path (global_load_lds, no registers) fills block k+1. B and x blocks
// stay token-major in LDS (swizzled rows); the token-contiguous operand
// fragments come out of LDS transpose reads, and w is applied to the x
// fragment in registers. Each wavefront owns one head and PT/WPH of its
// 32-row p tiles against all N/32 n tiles.
#include "kernels.hpp"

namespace ssd {

constexpr int kStateKB = 32;     // tokens per pipeline block

template <typename T, int PT, int NT>
struct StateCfg {
    static constexpr int TILES = PT * NT;
    static constexpr int WPH = TILES <= 8 ? 1 : TILES / 8;   // wavefronts per head
    static constexpr int HPW = 4 / WPH;                      // heads per workgroup
    static constexpr int PTW = PT / WPH;                     // p tiles per wavefront
    static constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte chunk
    static constexpr int XRC = PT * 32 / EPC;                // chunks per x row
    static constexpr int BRC = NT * 32 / EPC;                // chunks per B row
    static constexpr int XBYTES = kStateKB * XRC * 16;       // one head's x block
    static constexpr int BBYTES = kStateKB * BRC * 16;
    static constexpr int BUF = BBYTES + HPW * XBYTES;        // one pipeline buffer
    static constexpr int LDS = 2 * BUF + HPW * 256 * 4;      // + w vectors (Q <= 256)
};

template <typename T, int PT, int NT, typename ST>
__global__ __launch_bounds__(256) void ssd_chunk_state_kernel(Params p) {
    using Cfg = StateCfg<T, PT, NT>;
    constexpr int HPW = Cfg::HPW, WPH = Cfg::WPH, PTW = Cfg::PTW, NP = NT * 32;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::LDS];
    float* wv = reinterpret_cast<float*>(smem + 2 * Cfg::BUF);   // [HPW][Q]

    const int Q = (int)p.chunk;
    const int64_t T_ = p.seqlen, H = p.nheads, P = p.headdim, N = p.dstate, G = p.ngroups;
    const int64_t hpg = p.heads_per_group, nc = p.nchunks;
    const int nhb = (int)((hpg + HPW - 1) / HPW);
    int bx = blockIdx.x;
    const int hb = bx % nhb;
    bx /= nhb;
    const int64_t g = bx % G;
    const int c = (int)(bx / G);
    const int64_t b = blockIdx.y;
    const int64_t h0 = g * hpg + (int64_t)hb * HPW;
    const int nh = (int)min<int64_t>(HPW, hpg - (int64_t)hb * HPW);
    const int64_t t0 = (int64_t)c * Q;
    const int qc = (int)min<int64_t>(Q, T_ - t0);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wavefront
    const int hf = lane >> 5, l32 = lane & 31;
    const int64_t tok0 = b * T_ + t0;
    constexpr int ESZ = (int)sizeof(T);

    // decay-to-chunk-end weights w_j for every head of the block
    const float* csbase = p.cs + ((b * H + h0) * nc + c) * Q;
    const float* dtbase = p.dt + tok0 * H + h0;
    for (int idx = threadIdx.x; idx < HPW * Q; idx += blockDim.x) {
        const int hq = idx / Q, j = idx % Q;
        float wj = 0.0f;
        if (hq < nh && j < qc) {
            const float* csr = csbase + (int64_t)hq * nc * Q;
            wj = exp2f((ldg(csr + Q - 1) - ldg(csr + j)) * kLog2e) * ldg(dtbase + hq + (uint32_t)j * (uint32_t)H);
        }
        wv[hq * Q + j] = wj;
    }

    const unsigned char* bbase = static_cast<const unsigned char*>(p.B) + (tok0 * G + g) * N * ESZ;
    const unsigned char* xbase = static_cast<const unsigned char*>(p.x) + (tok0 * H + h0) * P * ESZ;
    const uint32_t bstride = (uint32_t)(G * N * ESZ), xstride = (uint32_t)(H * P * ESZ);
    const int xvalid = (int)(P * ESZ / 16), bvalid = (int)(N * ESZ / 16);
    auto issue = [&](int blk, int buf) {
        unsigned char* base = smem + buf * Cfg::BUF;
        // rows of the block past the chunk's last token re-read that token (their
        // weight w is 0); a block wholly past it reads only that token
        const int r0 = min(blk * kStateKB, qc - 1);
        const int vrows = min(kStateKB, qc - r0);
        dma_tile<Cfg::BRC>(base, kStateKB, vrows, bvalid, bbase + (uint32_t)r0 * bstride, bstride, wave, 4, lane);
        for (int hq = 0; hq < nh; ++hq)
            dma_tile<Cfg::XRC>(base + Cfg::BBYTES + hq * Cfg::XBYTES, kStateKB, vrows, xvalid,
                               xbase + (uint32_t)r0 * xstride + (int64_t)hq * P * ESZ, xstride, wave, 4, lane);
    };

    const int hh = wave / WPH;           // this wavefront's head within the block
    const int pt0 = (wave % WPH) * PTW;  // its first p tile
    const bool active = hh < nh;
    f32x16 acc[PTW][NT];
#pragma unroll
    for (int i = 0; i < PTW; ++i)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[i][n] = zero16();

    const int nblk = Q / kStateKB;
    issue(0, 0);
    wait_vmem();
    __syncthreads();
    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1;
        if (blk + 1 < nblk) issue(blk + 1, buf ^ 1);
        if (active) {
            const unsigned char* base = smem + buf * Cfg::BUF;
            const T* btile = reinterpret_cast<const T*>(base);
            const T* xtile = reinterpret_cast<const T*>(base + Cfg::BBYTES + hh * Cfg::XBYTES);
            const float* wrow = wv + hh * Q + blk * kStateKB;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                auto rowk = [s](int hf_, int e) { return 16 * s + 8 * hf_ + e; };
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow + 16 * s + 8 * hf);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + 16 * s + 8 * hf + 4);
                typename Vec8<T>::type xf[PTW], bf[NT];
#pragma unroll
                for (int i = 0; i < PTW; ++i) {
                    const auto raw = frag_tr<Cfg::XRC>(xtile, (pt0 + i) * 32, rowk, lane);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xf[i][e] = from_f32<T>(to_f32(raw[e]) * (e < 4 ? w0[e] : w1[e - 4]));
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) bf[n] = frag_tr<Cfg::BRC>(btile, n * 32, rowk, lane);
#pragma unroll
                for (int i = 0; i < PTW; ++i)
#pragma unroll
                    for (int n = 0; n < NT; ++n) mma_k16(acc[i][n], xf[i], bf[n]);
            }
        }
        wait_vmem();
        __syncthreads();
    }

    if (active) {
        const int64_t h = h0 + hh;
        ST* sg = static_cast<ST*>(p.states) + ((b * nc + c) * H + h) * P * N;   // [P][N] of this head
#pragma unroll
        for (int i = 0; i < PTW; ++i) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int64_t col = n * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t pr = (pt0 + i) * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (pr < P && col < N) stg<ST>(sg + (uint32_t)(pr * N + col), from_f32<ST>(acc[i][n][r]));
                }
            }
        }
    }
    (void)NP;
}

template <typename T, int PT, int NT, typename ST>
static hipError_t launch_cs(const Params& p, hipStream_t s) {
    using Cfg = StateCfg<T, PT, NT>;
    const int64_t nhb = (p.heads_per_group + Cfg::HPW - 1) / Cfg::HPW;
    dim3 grid((unsigned)(p.nchunks * p.ngroups * nhb), (unsigned)p.batch);
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
