// ssd_chunk_state: the right-factor state of every chunk.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2, second step of the
// block decomposition: each chunk's state, B^T applied to the inputs after
// their decay to the chunk's end. That decay is read as: token j of
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
// of one group, which share B (fewer heads, more workgroups, when the grid
// would not fill the chip). The chunk is consumed in blocks of 32 tokens
// through a ring of NBUF LDS buffers (three when x streams from HBM, two when
// it stays in the last-level cache): while the matrix cores work on block k,
// buffer loads straight to LDS (no registers) fill blocks k+1 .. k+NBUF-1, and
// the barrier between blocks does not drain them (lds_barrier). B and x blocks
// stay token-major in LDS (swizzled rows); the token-contiguous operand
// fragments come out of LDS transpose reads, and w is applied to the x
// fragment in registers. Each wavefront owns one head and PT/WPH of its
// 32-row p tiles against all N/32 n tiles.
//
// The block's dt travels with the first block's copies into a side tile, so
// the weights w (and, fused, the in-chunk cumulative decay) are computed as
// soon as that block has landed, without a round trip of their own; cs and
// the states are stored at the end.
#include "kernels.hpp"

namespace ssd {

constexpr int kStateKB = 32;     // tokens per pipeline block

// SPLIT: wavefronts per head doubled (half as many heads per workgroup,
// twice as many workgroups) for grids that would not fill the chip.
template <typename T, int PT, int NT, bool SPLIT = false>
struct StateCfg {
    static constexpr int TILES = PT * NT;
    static constexpr int WPH0 = TILES <= 8 ? 1 : TILES / 8;
    static constexpr int WPH = SPLIT ? 2 * WPH0 : WPH0;     // wavefronts per head
    static constexpr int HPW = 4 / WPH;                      // heads per workgroup
    static constexpr int PTW = PT / WPH;                     // p tiles per wavefront
    static constexpr int EPC = 16 / (int)sizeof(T);          // elements per 16-byte chunk
    static constexpr int XRC = PT * 32 / EPC;                // chunks per x row
    static constexpr int BRC = NT * 32 / EPC;                // chunks per B row
    static constexpr int XBYTES = kStateKB * XRC * 16;       // one head's x block
    static constexpr int BBYTES = kStateKB * BRC * 16;
    static constexpr int BUF = BBYTES + HPW * XBYTES;        // one pipeline buffer
    // ring of LDS blocks: three (two in flight while one is used) when two
    // workgroups still fit in a CU's LDS, else two. Two resident workgroups per
    // CU let one's stores and prologue overlap the other's copies and math.
    // side tile: dt [HPW][Q], overwritten in place by w
    static constexpr int SIDE = HPW * 256 * 4;
    static constexpr int NBUF3 = 2 * (3 * BUF + SIDE) <= 160 * 1024 ? 3 : 2;
    // x streamed from HBM (non-temporal copies) keeps NBUF3 buffers; x that
    // stays in the last-level cache is copied one block ahead only (two
    // buffers), since from that cache one block in flight covers the latency
    // and a second one only delays the block needed next
    template <bool XNT> static constexpr int nbuf() { return XNT ? NBUF3 : 2; }
    template <bool XNT> static constexpr int lds() { return nbuf<XNT>() * BUF + SIDE; }
    static constexpr int NDB = (kStateKB * BRC / 64 + 3) / 4;  // B copy instructions per wave
    static constexpr int NDX = (kStateKB * XRC / 64 + 3) / 4;  // x copy instructions per wave per head
};

// Lane byte offsets, relative to the block's first row, of the copies a
// wavefront issues for a full 32-row tile (see dma_tile); -1 = no copy.
template <int RC, int NI>
__device__ __forceinline__ void dma_plan(int (&off)[NI], int valid_chunks, uint32_t row_stride, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k = wave + 4 * i;
        if (k * 64 < kStateKB * RC) {
            const int P = k * 64 + lane, r = P / RC;
            int c = (P % RC) ^ swz<RC>(r);
            c = c < valid_chunks ? c : valid_chunks - 1;
            off[i] = (int)((uint32_t)r * row_stride + 16u * (uint32_t)c);
        } else {
            off[i] = -1;
        }
    }
}
// NT: the non-temporal policy (see dma16p).
template <int NI, bool NT = false>
__device__ __forceinline__ void dma_issue(unsigned char* lds, const unsigned char* gbase, const int (&off)[NI],
                                          int wave) {
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(gbase);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (off[i] >= 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + (wave + 4 * i) * 1024),
                                                     16, (uint32_t)off[i], 0, 0, NT ? 2 : 0);
    }
}

// One 4-byte global -> LDS copy per lane: lane l writes LDS bytes
// [lds + 4 l, lds + 4 l + 4).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, unsigned char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
}

constexpr uint32_t kOob = 0x80000000u;   // buffer offset past every range: the copy reads 0

// FUSED: also compute (and write) cs from dt and A, the step of
// ssd_chunk_cumsum; else read the given cs. VARLEN (with FUSED only): packed
// documents, w_j = 0 for tokens outside the document of the chunk's last
// token (the decay is 0 at a document start, "Transformers are SSMs", Knowl 8).
// XNT: x is copied with the non-temporal policy (the forward's data exceeds
// the last-level cache, so x would not stay there for its second read).
template <typename T, int PT, int NT, typename ST, bool FUSED, bool VARLEN, bool SPLIT, bool XNT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void ssd_chunk_state_kernel(Params p) {
    using Cfg = StateCfg<T, PT, NT, SPLIT>;
    using V8 = typename Vec8<T>::type;
    constexpr int HPW = Cfg::HPW, WPH = Cfg::WPH, PTW = Cfg::PTW;
    constexpr int ESZ = (int)sizeof(T);
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::template lds<XNT>()];
    constexpr int NBUF = Cfg::template nbuf<XNT>();
    float* wv = reinterpret_cast<float*>(smem + NBUF * Cfg::BUF);   // [HPW][QT]: dt, then w

    // Q: tokens per chunk; QT: its rows as tiled, whole 32-token blocks (a
    // 16-token chunk fills half a block, whose other rows get weight 0)
    const int Q = (int)p.chunk;
    const int QT = Q < kStateKB ? kStateKB : Q;
    const int64_t T_ = p.seqlen, H = p.nheads, P = p.headdim, N = p.dstate, G = p.ngroups;
    const int64_t hpg = p.heads_per_group, nc = p.nchunks;
    const int nhb = (int)((hpg + HPW - 1) / HPW);
    const int lin = xcd_logical_block();
    int bx = lin % (int)gridDim.x;
    const int hb = bx % nhb;
    bx /= nhb;
    const int64_t g = bx % G;
    const int c = (int)(bx / G);
    const int64_t b = lin / (int)gridDim.x;
    const int64_t h0 = g * hpg + (int64_t)hb * HPW;
    const int nh = (int)min<int64_t>(HPW, hpg - (int64_t)hb * HPW);
    const int64_t t0 = (int64_t)c * Q;
    const int qc = (int)min<int64_t>(Q, T_ - t0);
    const int64_t tok0 = b * T_ + t0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wavefront
    const int hf = lane >> 5, l32 = lane & 31;

    const float* csbase = p.cs + ((b * H + h0) * nc + c) * Q;
    const float* dtbase = p.dt + tok0 * H + h0;

    const unsigned char* bbase = static_cast<const unsigned char*>(p.B) + (tok0 * G + g) * N * ESZ;
    const unsigned char* xbase = static_cast<const unsigned char*>(p.x) + (tok0 * H + h0) * P * ESZ;
    const uint32_t bstride = (uint32_t)(G * N * ESZ), xstride = (uint32_t)(H * P * ESZ);
    const int xvalid = (int)(P * ESZ / 16), bvalid = (int)(N * ESZ / 16);
    int offb[Cfg::NDB], offx[Cfg::NDX];
    dma_plan<Cfg::BRC, Cfg::NDB>(offb, bvalid, bstride, wave, lane);
    dma_plan<Cfg::XRC, Cfg::NDX>(offx, xvalid, xstride, wave, lane);
    // side tile: lane value fi = (wave + 4i) * 64 + lane is (head fi / QT, token fi % QT)
    const int srounds = (HPW * QT + 255) / 256;
    auto issue_side = [&]() {
        const __amdgpu_buffer_rsrc_t rd = raw_rsrc(dtbase);
        for (int i = 0; i < srounds; ++i) {
            const int fi = (wave + 4 * i) * 64 + lane, hq = fi / QT, j = fi - hq * QT;
            const bool ok = hq < nh && j < qc;
            dma4(rd, ok ? (uint32_t)(j * (int)H + hq) * 4u : kOob, reinterpret_cast<unsigned char*>(wv) + fi * 4);
        }
    };
    auto issue = [&](int blk, unsigned char* base) {
        const int r0 = blk * kStateKB;
        if (r0 + kStateKB <= qc) {          // full block: precomputed lane offsets
            dma_issue<Cfg::NDB>(base, bbase + (uint32_t)r0 * bstride, offb, wave);
            for (int hq = 0; hq < nh; ++hq)
                dma_issue<Cfg::NDX, XNT>(base + Cfg::BBYTES + hq * Cfg::XBYTES,
                                         xbase + (uint32_t)r0 * xstride + (int64_t)hq * P * ESZ, offx, wave);
        } else {
            // rows past the chunk's last token re-read that token (their weight
            // w is 0); a block wholly past it reads only that token
            const int rb = min(r0, qc - 1);
            const int vrows = min(kStateKB, qc - rb);
            dma_tile<Cfg::BRC>(base, kStateKB, vrows, bvalid, bbase + (uint32_t)rb * bstride, bstride, wave, 4, lane);
            for (int hq = 0; hq < nh; ++hq)
                dma_tile<Cfg::XRC>(base + Cfg::BBYTES + hq * Cfg::XBYTES, kStateKB, vrows, xvalid,
                                   xbase + (uint32_t)rb * xstride + (int64_t)hq * P * ESZ, xstride, wave, 4, lane,
                                   XNT);
        }
    };

    const int hh = wave / WPH;           // this wavefront's head within the block
    const int pt0 = (wave % WPH) * PTW;  // its first p tile
    const bool active = hh < nh;
    // transpose-read lane offsets (k rows 8hf + e of the first 16-row group)
    auto rowk0 = [](int hf_, int e) { return 8 * hf_ + e; };
    int xoa[PTW], xob[PTW], boa[NT], bob[NT];
#pragma unroll
    for (int i = 0; i < PTW; ++i) frag_tr_offsets<Cfg::XRC>((pt0 + i) * 32, rowk0, lane, xoa[i], xob[i]);
#pragma unroll
    for (int n = 0; n < NT; ++n) frag_tr_offsets<Cfg::BRC>(n * 32, rowk0, lane, boa[n], bob[n]);

    f32x16 acc[PTW][NT];
#pragma unroll
    for (int i = 0; i < PTW; ++i)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[i][n] = zero16();

    // copies this wavefront issues per block (same set of instruction slots in
    // the planned and the generic path)
    int nb = 0, nx = 0;
#pragma unroll
    for (int i = 0; i < Cfg::NDB; ++i) nb += ((wave + 4 * i) * 64 < kStateKB * Cfg::BRC) ? 1 : 0;
#pragma unroll
    for (int i = 0; i < Cfg::NDX; ++i) nx += ((wave + 4 * i) * 64 < kStateKB * Cfg::XRC) ? 1 : 0;
    const int per_block = nb + nh * nx;

    const int nblk = QT / kStateKB;
    constexpr int AHEAD = NBUF - 1;     // blocks in flight beyond the one in use
    const int hq = wave / WPH;   // = hh: the head this wavefront computes w for
    float Ah = 0.0f;
    if constexpr (FUSED) Ah = p.A[h0 + min(hq, nh - 1)];   // a scalar load, used after the first wait
    for (int k = 0; k < AHEAD && k < nblk; ++k) {
        issue(k, smem + k * Cfg::BUF);
        if (k == 0) issue_side();
    }
    wait_vmem_le_rt(nblk > 1 && AHEAD > 1 ? per_block : 0);   // block 0 and the side tile landed
    lds_barrier();

    // decay-to-chunk-end weights w_j of head hq, computed by the head's first
    // wavefront in place of its dt row. Fused: the in-chunk cumulative decay
    // (the step of ssd_chunk_cumsum, same arithmetic) is formed here and kept
    // for the store at the end.
    const int per = Q >= 64 ? Q / 64 : 1, nact = Q / per;
    float csv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (wave % WPH == 0) {
        float* row = wv + hq * QT;
        float dtv[4], v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) dtv[k] = (k < per && lane < nact) ? row[lane * per + k] : 0.0f;
        float last;
        if constexpr (FUSED) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
#pragma clang fp contract(off)
                v[k] = dtv[k] * Ah;   // a rounded product, as ssd_chunk_cumsum forms it
            }
            chunk_prefix(v, per, nact, qc, lane);
            last = __shfl(v[per - 1], nact - 1, 64);
#pragma unroll
            for (int k = 0; k < 4; ++k) csv[k] = v[k];
        } else {
            const float* csr = csbase + (int64_t)hq * nc * Q;
            last = hq < nh ? ldg(csr + Q - 1) : 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = lane * per + k;
                v[k] = (hq < nh && k < per && lane < nact && j < qc) ? ldg(csr + j) : 0.0f;
            }
        }
        int slast = 0;
        const int* sq = VARLEN ? p.seq_idx + b * T_ + t0 : nullptr;
        if constexpr (VARLEN) slast = sq[qc - 1];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = lane * per + k;
            if (k < per && lane < nact) {
                bool keep = hq < nh && j < qc;
                if constexpr (VARLEN) keep = keep && sq[min(j, qc - 1)] == slast;
                row[j] = keep ? exp2f((last - v[k]) * kLog2e) * dtv[k] : 0.0f;
            }
        }
    }
    lds_barrier();

    // One block: start the copy of block blk + AHEAD into `next`, then run the
    // matrix cores on block blk in `base`. The three LDS regions are passed as
    // non-aliasing pointers so that the compiler knows the reads of `base` and
    // `wrow` do not depend on the copy in flight into `next` and does not wait
    // for it (the copy is waited for explicitly, one block later).
    auto step = [&](int blk, const unsigned char* __restrict__ base, unsigned char* __restrict__ next,
                    const float* __restrict__ wrow) __attribute__((always_inline)) {
        if (blk + AHEAD < nblk) issue(blk + AHEAD, next);
        if (active) {
            const unsigned char* xtile = base + Cfg::BBYTES + hh * Cfg::XBYTES;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int rofs_x = 16 * s * Cfg::XRC * 16, rofs_b = 16 * s * Cfg::BRC * 16;
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow + 16 * s + 8 * hf);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + 16 * s + 8 * hf + 4);
                V8 xf[PTW], bf[NT];
#pragma unroll
                for (int i = 0; i < PTW; ++i) {
                    V8 raw;
                    if constexpr (ESZ == 2) {
                        raw = frag_tr_at(xtile + rofs_x, xoa[i], xob[i]);
                    } else {
                        auto rowk = [s](int hf_, int e) { return 16 * s + 8 * hf_ + e; };
                        raw = frag_tr<Cfg::XRC>(reinterpret_cast<const T*>(xtile), (pt0 + i) * 32, rowk, lane);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xf[i][e] = from_f32<T>(to_f32(raw[e]) * (e < 4 ? w0[e] : w1[e - 4]));
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if constexpr (ESZ == 2) {
                        bf[n] = frag_tr_at(base + rofs_b, boa[n], bob[n]);
                    } else {
                        auto rowk = [s](int hf_, int e) { return 16 * s + 8 * hf_ + e; };
                        bf[n] = frag_tr<Cfg::BRC>(reinterpret_cast<const T*>(base), n * 32, rowk, lane);
                    }
                }
                // out[n][p]: B^T rows as the A operand, scaled x as the B operand,
                // so each lane ends up holding 4 consecutive n of one p
#pragma unroll
                for (int i = 0; i < PTW; ++i)
#pragma unroll
                    for (int n = 0; n < NT; ++n) mma_k16(acc[i][n], bf[n], xf[i]);
            }
        }
    };
    for (int blk = 0; blk < nblk; ++blk) {
        step(blk, smem + (blk % NBUF) * Cfg::BUF, smem + ((blk + AHEAD) % NBUF) * Cfg::BUF,
             wv + hh * QT + blk * kStateKB);
        // block blk+1 must have landed; later blocks may still be in flight
        const int later = min(AHEAD - 1, nblk - 2 - blk);
        wait_vmem_le_rt(later > 0 ? later * per_block : 0);
        lds_barrier();
    }

    if (FUSED && wave % WPH == 0 && hh < nh && lane < nact) {
        float* out = p.cs + ((b * H + h0 + hh) * nc + c) * Q + lane * per;
        if (per == 4) {
            f32x4 o;
            o[0] = csv[0]; o[1] = csv[1]; o[2] = csv[2]; o[3] = csv[3];
            *(__attribute__((address_space(1))) f32x4*)out = o;
        } else {
            for (int k = 0; k < per; ++k) out[k] = csv[k];
        }
    }
    if (active) {
        // accumulator element r of tile (i, n): state row p = (pt0+i)*32 + l32,
        // column n*32 + 8*(r/4) + 4*hf + r%4. bf16: the lane halves swap the
        // halves of quarters 2g and 2g+1 (v_permlane32_swap), so that a lane
        // holds 8 consecutive columns (one 16-byte store); fp32: one quarter
        // (4 columns) per store.
        const int64_t h = h0 + hh;
        ST* sg = static_cast<ST*>(p.states) + ((b * nc + c) * H + h) * P * N;   // [P][N] of this head
#pragma unroll
        for (int i = 0; i < PTW; ++i) {
            const int pr = (pt0 + i) * 32 + l32;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if constexpr (sizeof(ST) == 2) {
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp) {
                        uint32_t w[2][2];
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int gq = 2 * gp + q;
                            bf16x4 v;
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[r] = from_f32<bf16>(acc[i][n][4 * gq + r]);
                            const u32x2 u = __builtin_bit_cast(u32x2, v);
                            w[q][0] = u[0];
                            w[q][1] = u[1];
                        }
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const auto sw = __builtin_amdgcn_permlane32_swap(w[0][k], w[1][k], false, false);
                            w[0][k] = sw[0];
                            w[1][k] = sw[1];
                        }
                        const int col = n * 32 + 8 * (2 * gp + hf);
                        if (pr < P && col < N) {
                            u32x4 o;
                            o[0] = w[0][0]; o[1] = w[0][1]; o[2] = w[1][0]; o[3] = w[1][1];
                            *(__attribute__((address_space(1))) u32x4*)(sg + (uint32_t)(pr * (int)N + col)) = o;
                        }
                    }
                } else {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int col = n * 32 + 8 * gq + 4 * hf;
                        if (pr < P && col < N) {
                            f32x4 v;
                            v[0] = acc[i][n][4 * gq]; v[1] = acc[i][n][4 * gq + 1];
                            v[2] = acc[i][n][4 * gq + 2]; v[3] = acc[i][n][4 * gq + 3];
                            *(__attribute__((address_space(1))) f32x4*)(sg + (uint32_t)(pr * (int)N + col)) = v;
                        }
                    }
                }
            }
        }
    }
}

template <typename T, int PT, int NT, typename ST, bool SPLIT, bool XNT>
static hipError_t launch_cs2(const Params& p, hipStream_t s) {
    using Cfg = StateCfg<T, PT, NT, SPLIT>;
    const int64_t nhb = (p.heads_per_group + Cfg::HPW - 1) / Cfg::HPW;
    dim3 grid((unsigned)(p.nchunks * p.ngroups * nhb), (unsigned)p.batch);
    if (p.fuse_cs && p.seq_idx)
        hipLaunchKernelGGL((ssd_chunk_state_kernel<T, PT, NT, ST, true, true, SPLIT, XNT>), grid, dim3(256), 0, s, p);
    else if (p.fuse_cs)
        hipLaunchKernelGGL((ssd_chunk_state_kernel<T, PT, NT, ST, true, false, SPLIT, XNT>), grid, dim3(256), 0, s, p);
    else if (!p.seq_idx)
        hipLaunchKernelGGL((ssd_chunk_state_kernel<T, PT, NT, ST, false, false, SPLIT, XNT>), grid, dim3(256), 0, s, p);
    else
        return hipErrorInvalidValue;   // document resets need the fused prefix sums
    return hipGetLastError();
}

// Two workgroups fit per compute unit: when the grid of whole head blocks
// would not fill every such slot, halve the heads per workgroup (two
// wavefronts per head) where the p tiles allow it. Such a small grid never
// takes the non-temporal copies.
template <typename T, int PT, int NT, typename ST>
static hipError_t launch_cs(const Params& p, hipStream_t s) {
    using Cfg = StateCfg<T, PT, NT, false>;
    if constexpr (PT >= 2 * Cfg::WPH0) {
        const int64_t nhb = (p.heads_per_group + Cfg::HPW - 1) / Cfg::HPW;
        if (p.batch * p.nchunks * p.ngroups * nhb < 2 * (int64_t)device_cus())
            return launch_cs2<T, PT, NT, ST, true, false>(p, s);
    }
    return p.stream_x ? launch_cs2<T, PT, NT, ST, false, true>(p, s) : launch_cs2<T, PT, NT, ST, false, false>(p, s);
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
