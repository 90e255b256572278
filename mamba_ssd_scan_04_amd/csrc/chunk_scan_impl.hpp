// ssd_chunk_scan: the output of every chunk.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 2: the diagonal-block
// output (L o C B^T) X with the 1-semiseparable chunk mask
// L_ji = a_{i+1} ... a_j (j >= i), the off-diagonal output C (decayed h_c)
// from the state entering the chunk, and their sum; plus the skip term D x.
// "Decayed h_c" is read as row j scaled by a_0 ... a_j = exp(cs_j). Per
// (batch, chunk, head), with X the raw x and the step dt folded into the mask:
//
//   y_j = sum_{i<=j} (C_j . B_i) exp(cs_j - cs_i) dt_i x_i  +  exp(cs_j) C_j^T h_c  +  D x_j
//
// Work split. One workgroup of 8 wavefronts takes one chunk and up to `hpw`
// heads of one group (interleaved: heads h0, h0 + nhb, ...); wavefront w owns
// the 32-token row tile w (rows j), for every head.
//  Phase A, once per workgroup: C B^T does not depend on the head when B and C
//  are shared (Knowl 7), so each wavefront computes its row of 32x32 tiles
//  M^T(kt) = B_kt . C_w^T (kt <= w) on the matrix cores and rounds them to the
//  operand type. The off-diagonal tiles go to LDS (or stay in registers when
//  LDS is too small), the diagonal tile and the wave's C rows stay in
//  registers.
//  Phase B, per head: x (token-major) and h_c ([P][N]) are copied into LDS by
//  buffer loads straight to LDS, double-buffered so the next head's copy
//  overlaps this head's math. The key tiles are processed as a pipeline of
//  stages whose LDS operands are read one stage ahead. For every key tile the
//  lane scales its 16 C B^T values by the decay (exp(cs_j - cs_r) *
//  exp(cs_r - cs_i) dt_i with r the key tile's last token off the diagonal, the
//  per-key factor arriving by a row broadcast; a direct exp with the causal
//  mask on it) and feeds them straight to the next product as its M operand:
//  an accumulator's rows (8g + 4hf + r) become the next product's k index in
//  "fragment order", and the x fragment is read from LDS with transpose reads
//  in the same order. The products are formed transposed (Y^T = X^T M^T), so
//  each lane ends with 16 values of p for one token j. The carried-state term
//  is (C . h_c) with rows scaled by exp(cs_j). The epilogue adds D x_j,
//  optionally multiplies by the gate silu(z) (the Mamba-2 block's output gate,
//  "Transformers are SSMs", Knowl 6) and stores y in 16-byte pieces of token
//  rows.
#pragma once

#include <atomic>

#include "kernels.hpp"

namespace ssd {

constexpr int kScanMaxLds = 160 * 1024;
constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / 64;

// Instantiations of the chunk scan: the plain kernel, the one with the output
// gate in its epilogue, the one with document masks (packed documents), and
// the one with both.
enum ScanVariant { kScanPlain = 0, kScanGate = 1, kScanVarlen = 2, kScanGateVarlen = 3 };

template <typename T, int PT, int NT, typename ST>
struct ScanCfg {
    static constexpr int EPC = 16 / (int)sizeof(T);
    static constexpr int XRC = PT * 32 / EPC;                  // chunks per x row
    static constexpr int HRC = NT * 32 * (int)sizeof(ST) / 16; // chunks per h_c row
    static constexpr int HBYTES = PT * 32 * HRC * 16;          // one head's h_c tile
    static constexpr int KS = NT * 2;                          // k16 steps over n
    static constexpr int CBTILE = 2 * 64 * 8 * (int)sizeof(T);  // one 32x32 C B^T tile, lane-major
    __host__ __device__ static int xbytes(int Q) { return Q * XRC * 16; }
    __host__ __device__ static int vbytes(int Q) { return 3 * Q * 4; }
    // the off-diagonal C B^T tiles of all row tiles (kt < rt), when kept in LDS
    __host__ __device__ static int cbbytes(int Q) { return (Q / 32) * (Q / 32 - 1) / 2 * CBTILE; }
    // bytes of LDS with nbx x buffers, nbh h_c buffers, C B^T in LDS or not,
    // and the chunk's document ids (packed documents) or not
    __host__ __device__ static int lds(int Q, int nbx, int nbh, bool cbl, bool vl = false) {
        return nbx * xbytes(Q) + nbh * HBYTES + 2 * vbytes(Q) + (cbl ? cbbytes(Q) : 0) + (vl ? 4 * Q : 0);
    }
};

// x fragment (B operand of Y += M . X, k = key token in fragment order) at
// 16-row group g16 of column tile pt: bf16 through two transpose reads at
// precomputed offsets; fp32 through plain reads.
template <typename T, int XRC>
__device__ __forceinline__ typename Vec8<T>::type x_frag(const unsigned char* xt, int g16, int pt, const int (&xoa)[4],
                                                        const int (&xob)[4], int lane) {
    if constexpr (sizeof(T) == 2) {
        return frag_tr_at(xt + g16 * 16 * XRC * 16, xoa[pt], xob[pt]);
    } else {
        auto rowk = [g16](int hf_, int e) { return g16 * 16 + 8 * (e >> 2) + 4 * hf_ + (e & 3); };
        return frag_tr<XRC>(reinterpret_cast<const float*>(xt), pt * 32, rowk, lane);
    }
}

// GATE: y *= silu(z) in the epilogue (a separate instantiation, so that the
// plain kernel carries none of its registers). VARLEN: packed documents
// ("Transformers are SSMs", Knowl 8: the decay is 0 at a document start): the
// masked product keeps only key tokens of the query's document (folded once
// into the chunk's C B^T, which does not depend on the head), and the carried
// state reaches only rows in the document of the token before the chunk (its
// own instantiation too).
template <typename T, int PT, int NT, typename ST, int NBX, int NBH, bool CBL, bool GATE, bool VARLEN>
__global__ __launch_bounds__(kScanThreads) void ssd_chunk_scan_kernel(Params p, int hpw) {
    using Cfg = ScanCfg<T, PT, NT, ST>;
    using V8 = typename Vec8<T>::type;
    constexpr int KS = Cfg::KS, XRC = Cfg::XRC, HRC = Cfg::HRC;
    constexpr int ESZ = (int)sizeof(T), SSZ = (int)sizeof(ST);
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    // Q: tokens per chunk (the stride of chunks and of cs rows); QT: the
    // chunk's rows as tiled, whole 32-token tiles (Q = 16 fills half a tile,
    // whose other rows are masked like the tail of a short last chunk)
    const int Q = (int)p.chunk;
    const int QT = Q < 32 ? 32 : Q;
    const int XB = Cfg::xbytes(QT), VB = Cfg::vbytes(QT);
    unsigned char* const hb0 = smem + NBX * XB;
    float* const vb0 = reinterpret_cast<float*>(hb0 + NBH * Cfg::HBYTES);
    unsigned char* const cbl0 = reinterpret_cast<unsigned char*>(vb0) + 2 * VB;   // C B^T tiles (CBL)
    int* const sqv = reinterpret_cast<int*>(cbl0 + (CBL ? Cfg::cbbytes(QT) : 0));   // document ids (VARLEN)

    // ---- block coordinates (uniform) ----
    const int64_t T_ = p.seqlen, H = p.nheads, P = p.headdim, N = p.dstate, G = p.ngroups;
    const int64_t hpg = p.heads_per_group, nc = p.nchunks;
    const int nhb = (int)((hpg + hpw - 1) / hpw);
    const int lin = xcd_logical_block();
    int bx = lin % (int)gridDim.x;
    const int hb = bx % nhb;
    bx /= nhb;
    const int64_t g = bx % G;
    const int c = (int)(bx / G);
    const int64_t b = lin / (int)gridDim.x;
    // this workgroup's heads of the group: h0 + hh * nhb, hh < nh. Interleaved
    // (not consecutive) so that the workgroups of one chunk, running side by
    // side, read and write neighbouring heads' 128-byte row pieces together.
    const int64_t h0 = g * hpg + hb;
    const int nh = (int)((hpg - hb + nhb - 1) / nhb);
    const int64_t hs = nhb;
    const int64_t t0 = (int64_t)c * Q;
    const int qc = (int)min<int64_t>(Q, T_ - t0);
    const int64_t tok0 = b * T_ + t0;            // first token row of the chunk
    const bool hc = c > 0 || p.read_h0 != 0;     // a carried state enters this chunk

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    // Row tile of this wavefront. Waves w and w+4 share a SIMD; with 8 tiles
    // they take tiles s and 7 - s, so every SIMD carries 9 key tiles of work.
    const int RT = QT / 32;
    const int rt = RT == 8 ? (wave < 4 ? wave : 11 - wave) : (wave < RT ? wave : -1);
    const bool active = rt >= 0;
    // the heavier row tiles (the longer chain of key tiles per head) get issue
    // priority over their SIMD partner, which fills the gaps they leave
    if (rt >= 4) __builtin_amdgcn_s_setprio(1);

    const uint32_t bcs = (uint32_t)(G * N);
    const T* cbase = static_cast<const T*>(p.C) + (tok0 * G + g) * N;
    const T* bbase = static_cast<const T*>(p.B) + (tok0 * G + g) * N;
    const unsigned char* xbase = static_cast<const unsigned char*>(p.x) + (tok0 * H + h0) * P * ESZ;
    const uint32_t xstride = (uint32_t)(H * P * ESZ);
    const unsigned char* sbase = static_cast<const unsigned char*>(p.states) + ((b * nc + c) * H + h0) * P * N * SSZ;
    unsigned char* ybase = static_cast<unsigned char*>(p.y) + (tok0 * H + h0) * P * ESZ;
    const float* csbase = p.cs + ((b * H + h0) * nc + c) * Q;
    const float* dtbase = p.dt + tok0 * H + h0;
    const int xvalid = (int)(P * ESZ / 16), hvalid = (int)(N * SSZ / 16);

    // tile copies: lane offsets planned once, the same for every head
    constexpr int NIX = (256 * XRC / 64 + kScanWaves - 1) / kScanWaves;
    constexpr int NIH = (PT * 32 * HRC / 64 + kScanWaves - 1) / kScanWaves;
    int offx[NIX], offh[NIH];
    dma_tile_plan<XRC, NIX>(offx, QT, qc, xvalid, xstride, wave, kScanWaves, lane);
    dma_tile_plan<HRC, NIH>(offh, PT * 32, (int)P, hvalid, (uint32_t)(N * SSZ), wave, kScanWaves, lane);
    // x and the carried states are read once: non-temporal copies when the
    // forward's data cannot stay in the last-level cache
    const bool snt = p.stream_x != 0;
    auto issue_x = [&](int hh, unsigned char* dst) {
        const unsigned char* src = xbase + (int64_t)hh * hs * P * ESZ;
        if (snt)
            dma_tile_issue<NIX, true>(dst, src, offx, wave, kScanWaves);
        else
            dma_tile_issue<NIX>(dst, src, offx, wave, kScanWaves);
    };
    auto issue_h = [&](int hh, unsigned char* dst) {
        const unsigned char* src = sbase + (int64_t)hh * hs * P * N * SSZ;
        if (snt)
            dma_tile_issue<NIH, true>(dst, src, offh, wave, kScanWaves);
        else
            dma_tile_issue<NIH>(dst, src, offh, wave, kScanWaves);
    };
    float vcs = 0.0f, vcr = 0.0f, vdt = 0.0f;   // thread i holds token i of the next head
    // packed documents: thread i < QT holds the id of token i (clamped to the
    // chunk); sprev is the id of the token before the chunk (the first token's
    // for chunk 0, whose carried state is the initial one)
    int vsq = 0, sprev = 0;
    if constexpr (VARLEN) {
        const int* sq = p.seq_idx + b * T_;
        sprev = sq[c > 0 ? t0 - 1 : 0];
        if ((int)threadIdx.x < QT) vsq = sq[t0 + min((int)threadIdx.x, qc - 1)];
    }
    // rows past the chunk's Q tokens (Q = 16) take its last cs value, as the
    // padding of a short last chunk does
    auto load_vec = [&](int hh) {
        const int i = threadIdx.x;
        if (i < QT) {
            const float* csr = csbase + (int64_t)hh * hs * nc * Q;
            vcs = ldg(csr + min(i, Q - 1));
            vcr = ldg(csr + min(i | 31, Q - 1));
            // clamped row, zeroed past the chunk's end in store_vec: a select
            // here would write the register before the load and make the
            // wavefront wait for every older memory operation (the last
            // head's stores) first
            vdt = ldg(dtbase + hh * hs + (uint32_t)min(i, qc - 1) * (uint32_t)H);
        }
    };
    // per-head vectors in LDS, token i of the chunk's tiles (log2 units: c2 = cs log2 e):
    //   [0, QT)    c2_i                            (2^c2_j is the carried-state row scale)
    //   [QT, 2QT)  2^(c2_r - c2_i) dt_i, r = the last token of i's 32-token tile
    //   [2QT,3QT)  dt_i                            (0 past the chunk's end)
    auto store_vec = [&](float* v) {
        const int i = threadIdx.x;
        if (i < QT) {
            const float c2 = vcs * kLog2e, c2r = vcr * kLog2e;
            const float d = i < qc ? vdt : 0.0f;
            v[i] = c2;
            v[QT + i] = exp2f(c2r - c2) * d;
            v[2 * QT + i] = d;
        }
    };

    // D of this workgroup's heads, lane l holding head h0 + l nhb (read per head
    // with a lane broadcast, so no scalar loads sit in the head loop)
    const float dlane = ldg(p.D + h0 + (lane < nh ? lane : 0) * hs);
    // ---- phase A: this wave's C rows and C B^T row of tiles, once per workgroup ----
    // B is staged through LDS in slices of whole 32-token key tiles, in the
    // x buffer that head 0 does not use (or in head 0's, whose copy then
    // starts after phase A); if not even one key tile fits there, B tiles are
    // read from global memory instead. With bf16 operands, two x buffers and
    // C B^T in LDS, the whole of B is copied at once when the key tiles past
    // the first slice fit in the C B^T region (whose tiles are then written
    // only after every wavefront has read B): one round trip to memory, in
    // flight together with head 0's copies (issued after it).
    constexpr int BRC = NT * 32 * ESZ / 16;                    // 16-byte chunks per B row
    constexpr int BTILE = 32 * BRC * 16;                       // one 32-token B tile
    unsigned char* const stg = smem + (NBX == 2 ? XB : 0);
    const int tps = XB / BTILE;                                // B tiles per slice
    const bool bstage = tps > 0;
    // (never with N > 128: the key tiles past the first slice are then larger
    // than the C B^T region at every chunk size)
    constexpr bool BONE_OK = NBX == 2 && CBL && ESZ == 2 && NT <= 4;
    const bool bone = BONE_OK && bstage && (RT - tps) * BTILE <= Cfg::cbbytes(QT);
    const unsigned char* const bbytes = reinterpret_cast<const unsigned char*>(bbase);
    const uint32_t bstride = (uint32_t)(G * N * ESZ);
    const int bvalid = (int)(N * ESZ / 16);
    // head 0's tiles start moving before phase A: after C's loads and the
    // single copy of B where that copy can be taken, else first (where C's
    // rows would otherwise stay live across the copy issue: more spilled
    // registers at N = 256)
    auto issue_head0 = [&]() {
        if (nh > 0) {
            load_vec(0);
            if (NBX == 2 || !bstage) issue_x(0, smem);
            if (hc) issue_h(0, hb0);
        }
    };
    if constexpr (!BONE_OK) issue_head0();
    if (bone) {
        // key tiles [0, tps) into the free x buffer, the rest into the C B^T
        // region; rows past the chunk's last token re-read that token (their
        // products get zero weight), a part wholly past it reads only it
        const int r1 = min(RT, tps) * 32;
        dma_tile<BRC>(stg, r1, qc, bvalid, bbytes, bstride, wave, kScanWaves, lane);
        if (RT > tps) {
            const int rb = min(r1, qc - 1);
            dma_tile<BRC>(cbl0, RT * 32 - r1, qc - rb, bvalid, bbytes + (size_t)rb * bstride, bstride, wave,
                          kScanWaves, lane);
        }
    }

    const int nlast = (int)N - 8;
    V8 creg[KS];
    V8 cb[CBL ? 1 : 7][2];   // key tiles kt < rt, in registers unless kept in LDS
    V8 cbd[2];               // the diagonal tile
    // this row tile's off-diagonal tiles in LDS: tile kt at cbw + kt * CBTILE,
    // lane l's 8 low / 8 high elements at l * 8 and (64 + l) * 8 elements
    unsigned char* const cbw = cbl0 + (rt > 0 ? rt * (rt - 1) / 2 : 0) * Cfg::CBTILE;
    auto off = [&](int row, int ks) {
        return (uint32_t)min(row, qc - 1) * bcs + (uint32_t)min(ks * 16 + hf * 8, nlast);
    };
    // this wave's C rows, zeroed past the chunk's end and past N: where the
    // single copy of B can be taken, where they are first used (a select here
    // would wait for the loads at once, before head 0's copies are issued),
    // else as they load
    auto mask_creg = [&]() {
        const int jl = rt * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) creg[ks] = (jl < qc && ks * 16 + hf * 8 < (int)N) ? creg[ks] : zero8<T>();
    };
    if (active) {
        const int jl = rt * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) creg[ks] = ldg8(cbase + off(jl, ks));
        if constexpr (!BONE_OK) mask_creg();
    }
    if constexpr (BONE_OK) issue_head0();
    // round tile kt of C B^T to the operand type and keep it
    auto round_tile = [&](const f32x16& acc, V8& lo, V8& hi) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo[e] = from_f32<T>(acc[e]);
            hi[e] = from_f32<T>(acc[8 + e]);
        }
    };
    auto place_tile = [&](int kt, const V8& lo, const V8& hi) {
        if (kt < rt) {
            if constexpr (CBL) {
                store8(reinterpret_cast<T*>(cbw + kt * Cfg::CBTILE) + lane * 8, lo);
                store8(reinterpret_cast<T*>(cbw + kt * Cfg::CBTILE) + (64 + lane) * 8, hi);
            } else {
                cb[kt < 7 ? kt : 6][0] = lo;
                cb[kt < 7 ? kt : 6][1] = hi;
            }
        } else {
            cbd[0] = lo;
            cbd[1] = hi;
        }
    };
    auto keep_tile = [&](int kt, const f32x16& acc) {
        V8 lo, hi;
        round_tile(acc, lo, hi);
        place_tile(kt, lo, hi);
    };
    if (bone) {
        // B has landed when every memory operation of this wavefront but its
        // head-0 tile copies has (its vector loads, older, are waited for too)
        int younger = 0;
        if (nh > 0) {
#pragma unroll
            for (int i = 0; i < NIX; ++i) younger += offx[i] >= 0 ? 1 : 0;
            if (hc) {
#pragma unroll
                for (int i = 0; i < NIH; ++i) younger += offh[i] >= 0 ? 1 : 0;
            }
        }
        wait_vmem_le_rt(younger);
        lds_barrier();
        // B's two parts as non-aliasing pointers, so that the compiler knows
        // their reads do not depend on head 0's copies in flight
        auto tiles = [&](const unsigned char* __restrict__ b1, const unsigned char* __restrict__ b2)
            __attribute__((always_inline)) {
            if (active) {
                mask_creg();
                V8 tlo[8], thi[8];
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) {
                    if (kt <= rt) {
                        const T* tb = reinterpret_cast<const T*>(kt < tps ? b1 : b2);
                        const int row = (kt < tps ? kt : kt - tps) * 32 + l32;
                        f32x16 acc = zero16();
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            V8 a = row8<BRC>(tb, row, ks * 16 + hf * 8);
                            if (ks * 16 + hf * 8 >= (int)N) a = zero8<T>();
                            mma_k16(acc, a, creg[ks]);
                        }
                        round_tile(acc, tlo[kt], thi[kt]);
                    }
                }
                lds_barrier();   // every wavefront has read B from the C B^T region
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
                    if (kt <= rt) place_tile(kt, tlo[kt], thi[kt]);
            } else {
                lds_barrier();
            }
        };
        tiles(stg, cbl0);
    } else if (bstage) {
        if constexpr (BONE_OK) {
            if (active) mask_creg();
        }
        for (int s0 = 0; s0 < RT; s0 += tps) {
            const int s1 = min(s0 + tps, RT);
            if (s0 > 0) lds_barrier();   // the previous slice has been read
            // rows past the chunk's last token re-read that token (their
            // products get zero weight); a slice wholly past it reads only it
            const int rb = min(s0 * 32, qc - 1);
            dma_tile<BRC>(stg, (s1 - s0) * 32, qc - rb, bvalid, bbytes + (size_t)rb * bstride, bstride, wave,
                          kScanWaves, lane);
            wait_vmem();
            lds_barrier();
            if (active) {
                for (int kt = s0; kt < s1 && kt <= rt; ++kt) {
                    const int row = (kt - s0) * 32 + l32;
                    f32x16 acc = zero16();
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        V8 a = row8<BRC>(reinterpret_cast<const T*>(stg), row, ks * 16 + hf * 8);
                        if (ks * 16 + hf * 8 >= (int)N) a = zero8<T>();
                        mma_k16(acc, a, creg[ks]);
                    }
                    keep_tile(kt, acc);
                }
            }
        }
        if (NBX == 1 && nh > 0) {   // head 0's x goes where B was staged
            lds_barrier();
            issue_x(0, smem);
        }
    } else if (active) {
        if constexpr (BONE_OK) mask_creg();
        V8 bnext[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bnext[ks] = ldg8(bbase + off(l32, ks));
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            if (kt <= rt) {
                V8 bcur[KS];
                const bool rok = kt * 32 + l32 < qc;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) bcur[ks] = (rok && ks * 16 + hf * 8 < (int)N) ? bnext[ks] : zero8<T>();
                if (kt < rt) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) bnext[ks] = ldg8(bbase + off((kt + 1) * 32 + l32, ks));
                }
                f32x16 acc = zero16();
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) mma_k16(acc, bcur[ks], creg[ks]);
                keep_tile(kt, acc);
            }
        }
    }

    // lane offsets of the x fragments (fragment order), per column tile
    int xoa[4] = {0, 0, 0, 0}, xob[4] = {0, 0, 0, 0};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
            frag_tr_offsets<XRC>(pt * 32, [](int hf_, int e) { return 8 * (e >> 2) + 4 * hf_ + (e & 3); }, lane,
                                 xoa[pt], xob[pt]);
    }
    // h_c fragment rows: row p = pt*32 + l32, swizzle of that row
    const int hsw = swz<HRC>(l32);   // pt*32 leaves the swizzle unchanged

    if (nh > 0) store_vec(vb0);
    if constexpr (VARLEN) {
        if ((int)threadIdx.x < QT) sqv[threadIdx.x] = vsq;
    }
    wait_vmem();
    lds_barrier();
    // packed documents: this lane's query token's document, and the first
    // token of that document within the chunk (0 when it started before the
    // chunk), found by a binary search over the chunk's ids. Ids do not
    // decrease along T, so a key i of the chunk lies in the query's document
    // iff i >= that first token (a key after the query is masked as
    // non-causal anyway).
    int sqj = 0, dstart = 0;
    if constexpr (VARLEN) {
        if (active) {
            const int jq = rt * 32 + l32;
            sqj = sqv[jq];
#pragma unroll
            for (int step = 128; step >= 1; step >>= 1)
                if (dstart + step <= jq && sqv[dstart + step - 1] < sqj) dstart += step;
            // The document mask depends on the (query, key) pair only, not on
            // the head: it is folded once into this wavefront's row of C B^T
            // tiles, which every head then uses as they are. Element idx of
            // tile kt holds key kt*32 + 4hf + 8(idx/4) + idx%4; keys before
            // dstart lie in an earlier document and their C B^T value is set
            // to 0 (exact: their decay factor is at most 1). Tiles no lane of
            // the wavefront needs to mask are left alone.
            auto mask8 = [&](V8& v, int ds, int e0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int idx = e0 + e, off = 8 * (idx >> 2) + (idx & 3);
                    v[e] = off >= ds ? v[e] : from_f32<T>(0.0f);
                }
            };
            for (int kt = 0; kt <= rt; ++kt) {
                const int ds = dstart - (kt * 32 + 4 * hf);
                if (__builtin_amdgcn_readfirstlane(__any(ds > 0) ? 1 : 0) == 0) continue;
                if (kt == rt) {
                    mask8(cbd[0], ds, 0);
                    mask8(cbd[1], ds, 8);
                } else if constexpr (CBL) {
                    T* tp = reinterpret_cast<T*>(cbw + kt * Cfg::CBTILE);
                    V8 lo = load8(tp + lane * 8), hi = load8(tp + (64 + lane) * 8);
                    mask8(lo, ds, 0);
                    mask8(hi, ds, 8);
                    store8(tp + lane * 8, lo);
                    store8(tp + (64 + lane) * 8, hi);
                } else {
                    mask8(cb[kt < 7 ? kt : 6][0], ds, 0);
                    mask8(cb[kt < 7 ? kt : 6][1], ds, 8);
                }
            }
        }
    }

    // ---- phase B: heads ----
    // One head: load the next head's vectors, compute this head from xt / ht /
    // c2v, start the copies of the next head's tiles into xn / hn (when
    // double-buffered), store y, and write the next head's vectors into vn.
    // The copies are issued after the carried-state product, not at the start
    // of the head: a wavefront stalls on issuing them while the memory system
    // still holds the previous head's stores and the other wavefronts'
    // copies, and at the start of the head that stall would delay its first
    // products, which need nothing from memory. The LDS regions are passed as
    // non-aliasing pointers so that the compiler knows this head's LDS reads
    // do not depend on the copies in flight and does not wait for them (they
    // are waited for explicitly at the end of the head). Returns false if
    // some lane skipped a y store.
    // Operands of one 32-token key tile of the masked product, read from LDS
    // one step ahead of their use: the C B^T tile (off the diagonal), the
    // key tile's last c2, x fragments, and per-key vectors held one value per
    // lane in row-broadcast order (lane 16q + n holds key token
    // 8(n/4) + 4(q/2) + n%4 of the tile, which is accumulator element n of
    // every lane of that row's half): u off the diagonal, c2 and dt on it.
    struct Stage {
        V8 m[2];
        float u, d, r;
        V8 xf[2][PT];
    };
    const int bcl = 8 * ((lane & 15) >> 2) + 4 * (lane >> 5) + (lane & 3);   // key token of this lane's slot
    auto head = [&](int hh, const unsigned char* __restrict__ xt, const unsigned char* __restrict__ ht,
                    const float* __restrict__ c2v, const unsigned char* __restrict__ cbt,
                    unsigned char* __restrict__ xn, unsigned char* __restrict__ hn,
                    float* __restrict__ vn, float Dh) __attribute__((always_inline)) {
        const bool more = hh + 1 < nh;
        // the next head's vectors first: their results are then waited for
        // without the copies issued after them
        if (more) load_vec(hh + 1);
        auto issue_next = [&]() {
            if (more) {
                if (NBX == 2) issue_x(hh + 1, xn);
                if (NBH == 2 && hc) issue_h(hh + 1, hn);
            }
        };
        if (!active) issue_next();   // nothing to compute: issue at once
        bool stored_all = true;
        if (active) {
            const float* uv = c2v + QT;
            const float* dtv = c2v + 2 * QT;
            int jl = rt * 32 + l32, qch = qc;
            asm volatile("" : "+v"(jl), "+v"(qch));    // keep per-element compares in the loop
            // The products are formed transposed, Y^T = X^T M^T (+ h^T C^T): the
            // same registers as Y = M X with the A and B operands swapped, which
            // leaves each lane holding 16 values of p for one token j.
            f32x16 acc[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] = zero16();
            const float c2j = c2v[jl];
            // gate inputs of this lane's outputs (token jl), loaded now and
            // used in the epilogue. bf16: 16 bytes per lane in the layout y is
            // stored in (8 consecutive p of row jl, see the epilogue), turned
            // into the accumulator's quarters there by the same lane-half swap;
            // fp32: the 4 p of each accumulator quarter.
            typedef __attribute__((ext_vector_type(4))) T T4;
            T4 zq[PT][GATE && ESZ == 4 ? 4 : 1];
            u32x4 z16[PT][GATE && ESZ == 2 ? 2 : 1];
            if constexpr (GATE) {
                const T* zr = static_cast<const T*>(p.z) +
                              ((tok0 + min(jl, qch - 1)) * H + h0 + (int64_t)hh * hs) * P;
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    if constexpr (ESZ == 2) {
#pragma unroll
                        for (int gp = 0; gp < 2; ++gp) {
                            const int p0 = min(pt * 32 + 8 * (2 * gp + hf), (int)P - 8);
                            z16[pt][gp] = *(const __attribute__((address_space(1))) u32x4*)(zr + p0);
                        }
                    } else {
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const int p0 = min(pt * 32 + 8 * gq + 4 * hf, (int)P - 4);
                            zq[pt][gq] = *(const __attribute__((address_space(1))) T4*)(zr + p0);
                        }
                    }
                }
            }
            // y * silu(z) = y z / (1 + 2^(-z log2 e)), with the hardware exp2 and
            // reciprocal (z -> -inf gives z * rcp(inf) = -0, z -> +inf gives z)
            auto gate = [&](float yv, T zv) {
                const float zf = to_f32(zv);
                return yv * (zf * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-zf * kLog2e)));
            };
            // the carried state reaches row j scaled by 2^c2_j (not at all
            // when a document starts inside the chunk at or before j)
            float ej = exp2f(c2j);
            if constexpr (VARLEN) ej = sqj == sprev ? ej : 0.0f;

            // stage k < rt: off-diagonal key tile k; k == rt: the diagonal tile.
            // Every stage issues the same LDS reads whatever k is (addresses are
            // selected, not branched over, and k is clamped to rt), so that the
            // number of reads in flight is known where each stage's data is
            // waited for and the wait covers only that stage's reads.
            auto load_stage = [&](Stage& st, int k) __attribute__((always_inline)) {
                k = k < rt ? k : rt;
                const bool off = k < rt;
                if constexpr (CBL) {
                    const unsigned char* mp = off ? cbt + k * Cfg::CBTILE : xt;   // xt: any readable LDS
                    st.m[0] = load8(reinterpret_cast<const T*>(mp) + lane * 8);
                    st.m[1] = load8(reinterpret_cast<const T*>(mp) + (64 + lane) * 8);
                } else {
                    st.m[0] = cb[CBL ? 0 : (k < 7 ? k : 6)][0];
                    st.m[1] = cb[CBL ? 0 : (k < 7 ? k : 6)][1];
                }
                st.r = c2v[k * 32 + 31];
                st.u = (off ? uv : c2v)[k * 32 + bcl];
                st.d = dtv[k * 32 + bcl];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) st.xf[s2][pt] = x_frag<T, XRC>(xt, 2 * k + s2, pt, xoa, xob, lane);
            };
            // off the diagonal M = CB 2^(c2_j - c2_r) u_i, no mask; on it
            // M = CB 2^(c2_j - c2_i) dt_i (the difference is exact for i = j),
            // with the causal mask (i <= j) entering as a -inf exponent for
            // i > j (exp2 gives exactly 0)
            auto run_stage = [&](const Stage& st, int k) __attribute__((always_inline)) {
                V8 aop[2];
                if (k < rt) {
                    const float vj = fast_exp2(c2j - st.r);
                    static_for<16>([&](auto I) {
                        constexpr int idx = decltype(I)::value;
                        float val = row_bcast<idx>(st.u) * (to_f32(st.m[idx >> 3][idx & 7]) * vj);
                        aop[idx >> 3][idx & 7] = from_f32<T>(val);
                    });
                } else {
                    const int dj = jl - (k * 32 + 4 * hf);   // element idx is causal iff 8(idx/4) + idx%4 <= dj
                    static_for<16>([&](auto I) {
                        constexpr int idx = decltype(I)::value;
                        constexpr int off = 8 * (idx >> 2) + (idx & 3);
                        const float pen = __int_as_float(((dj - off) >> 31) & (int)0xff800000u);
                        aop[idx >> 3][idx & 7] = from_f32<T>(
                            to_f32(cbd[idx >> 3][idx & 7]) * fast_exp2((c2j - row_bcast<idx>(st.u)) + pen) *
                            row_bcast<idx>(st.d));
                    });
                }
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) mma_k16(acc[pt], st.xf[s2][pt], aop[s2]);
            };

            // ping-pong stages: the operands of stage k+1 are read (all of
            // them issued) before stage k computes; the scheduling barriers
            // keep the compiler from sinking those reads into their uses
            Stage sa, sb;
            if (hc) {   // (h_c^T C^T), then scaled by exp(cs_j)
                // over n in pieces, each piece's h_c fragments read before its
                // products: halves up to N = 128; at N = 256, where the wave's
                // C rows take 64 registers, pieces of 2 k16 steps
                constexpr int KP = KS <= 8 ? KS / 2 : 2, NPC = KS / KP;
                typename Vec8<ST>::type hv[KP][PT];
#pragma unroll
                for (int half = 0; half < NPC; ++half) {
#pragma unroll
                    for (int k2 = 0; k2 < KP; ++k2) {
                        const int ks = half * KP + k2;
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) {
                            const int cbyte = (ks * 16 + hf * 8) * SSZ;   // 16 or 32 bytes
                            const unsigned char* rp = ht + (pt * 32 + l32) * HRC * 16;
                            if constexpr (SSZ == 2) {
                                hv[k2][pt] = *reinterpret_cast<const bf16x8*>(rp + (((cbyte >> 4) ^ hsw) << 4));
                            } else {
                                const f32x4 lo = *reinterpret_cast<const f32x4*>(rp + (((cbyte >> 4) ^ hsw) << 4));
                                const f32x4 hi = *reinterpret_cast<const f32x4*>(rp + ((((cbyte >> 4) + 1) ^ hsw) << 4));
                                hv[k2][pt][0] = lo[0]; hv[k2][pt][1] = lo[1]; hv[k2][pt][2] = lo[2]; hv[k2][pt][3] = lo[3];
                                hv[k2][pt][4] = hi[0]; hv[k2][pt][5] = hi[1]; hv[k2][pt][6] = hi[2]; hv[k2][pt][7] = hi[3];
                            }
                        }
                    }
                    if (half == NPC - 1) load_stage(sa, 0);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int k2 = 0; k2 < KP; ++k2)
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt) mma_k16(acc[pt], cvt8<T>(hv[k2][pt]), creg[half * KP + k2]);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[pt][r] *= ej;
            } else {
                load_stage(sa, 0);
            }
            issue_next();
            // stages 0 .. rt (rt + 1 of them), two per iteration; the reads
            // past stage rt repeat stage rt's and go unused
            for (int k = 0; k <= rt; k += 2) {
                load_stage(sb, k + 1);
                __builtin_amdgcn_sched_barrier(0);
                run_stage(sa, k);
                __builtin_amdgcn_sched_barrier(0);
                load_stage(sa, k + 2);
                __builtin_amdgcn_sched_barrier(0);
                if (k + 1 <= rt) run_stage(sb, k + 1);
                __builtin_amdgcn_sched_barrier(0);
            }

            // epilogue: y = acc + D x. Accumulator quarter gq of column tile pt
            // holds p = 32 pt + 8 gq + 4 hf + (0..3) of token j: read those four
            // x values from the tile and add. For bf16, the two lane halves then
            // swap halves of quarters 2g and 2g+1 (v_permlane32_swap), so that
            // each lane holds 8 consecutive p (16 bytes) and a lane pair writes
            // 32 contiguous bytes of row j; fp32 stores 16 bytes per quarter.
            // this token's x values for the D x term, all read before any is
            // used (one wait instead of one per quarter pair)
            typedef __attribute__((ext_vector_type(4))) T T4x;
            T4x xq[PT][4];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    xq[pt][gq] = *reinterpret_cast<const T4x*>(xt + tile_byte<XRC>(jl, (pt * 32 + 8 * gq + 4 * hf) * ESZ));
            // the next head's vectors, before this head's stores: waiting for
            // their loads then needs only the copies issued after them
            if (more) store_vec(vn);
            unsigned char* yh = ybase + (int64_t)hh * hs * P * ESZ;
            const uint32_t ystride = (uint32_t)(H * P * ESZ);
            const bool jok = jl < qch;
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                if constexpr (ESZ == 2) {
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp) {
                        uint32_t w[2][2];
                        // gate: the row-layout z piece back into quarters 2gp, 2gp+1
                        uint32_t zw[2][2] = {{0u, 0u}, {0u, 0u}};
                        if constexpr (GATE) {
                            zw[0][0] = z16[pt][gp][0]; zw[0][1] = z16[pt][gp][1];
                            zw[1][0] = z16[pt][gp][2]; zw[1][1] = z16[pt][gp][3];
#pragma unroll
                            for (int k = 0; k < 2; ++k) {
                                const auto sw = __builtin_amdgcn_permlane32_swap(zw[0][k], zw[1][k], false, false);
                                zw[0][k] = sw[0];
                                zw[1][k] = sw[1];
                            }
                        }
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int gq = 2 * gp + q;
                            const bf16x4 xv = xq[pt][gq];
                            u32x2 zp;
                            zp[0] = zw[q][0];
                            zp[1] = zw[q][1];
                            const bf16x4 zv = __builtin_bit_cast(bf16x4, zp);
                            bf16x4 yv;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float v = acc[pt][4 * gq + r] + Dh * to_f32(xv[r]);
                                if constexpr (GATE) yv[r] = from_f32<T>(gate(v, zv[r]));
                                else yv[r] = from_f32<T>(v);
                            }
                            const u32x2 wv = __builtin_bit_cast(u32x2, yv);
                            w[q][0] = wv[0];
                            w[q][1] = wv[1];
                        }
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const auto sw = __builtin_amdgcn_permlane32_swap(w[0][k], w[1][k], false, false);
                            w[0][k] = sw[0];
                            w[1][k] = sw[1];
                        }
                        const int p0 = pt * 32 + 8 * (2 * gp + hf);
                        u32x4 out;
                        out[0] = w[0][0]; out[1] = w[0][1]; out[2] = w[1][0]; out[3] = w[1][1];
                        if (jok && p0 < (int)P)
                            *(__attribute__((address_space(1))) u32x4*)(yh + (uint32_t)jl * ystride + p0 * ESZ) = out;
                        else
                            stored_all = false;
                    }
                } else {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int p0 = pt * 32 + 8 * gq + 4 * hf;
                        const f32x4 xv = xq[pt][gq];
                        f32x4 yv;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float v = acc[pt][4 * gq + r] + Dh * xv[r];
                            if constexpr (GATE) yv[r] = gate(v, zq[pt][gq][r]);
                            else yv[r] = v;
                        }
                        if (jok && p0 < (int)P)
                            *(__attribute__((address_space(1))) f32x4*)(yh + (uint32_t)jl * ystride + p0 * ESZ) = yv;
                        else
                            stored_all = false;
                    }
                }
            }
        }
        if (more && !active) store_vec(vn);
        return stored_all;
    };

    for (int hh = 0; hh < nh; ++hh) {
        const int buf = hh & 1;
        unsigned char* const xcur = smem + (NBX == 2 ? buf : 0) * XB;
        unsigned char* const hcur = hb0 + (NBH == 2 ? buf : 0) * Cfg::HBYTES;
        unsigned char* const xnext = smem + (NBX == 2 ? buf ^ 1 : 0) * XB;
        unsigned char* const hnext = hb0 + (NBH == 2 ? buf ^ 1 : 0) * Cfg::HBYTES;
        const bool stored_all = head(hh, xcur, hcur, vb0 + buf * (VB / 4), cbw, xnext, hnext, vb0 + (buf ^ 1) * (VB / 4),
                                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dlane), hh)));
        // the next head's copies were issued before this head's stores: wait
        // for everything but the stores just issued (all lanes stored) or all
        if (__builtin_amdgcn_readfirstlane(__any(!stored_all) ? 1 : 0) == 0 && active)
            wait_vmem_le<(sizeof(T) == 2 ? 2 : 4) * PT>();   // this head's y stores
        else
            wait_vmem();
        lds_barrier();
        if (hh + 1 < nh && (NBX == 1 || (NBH == 1 && hc))) {   // single-buffered tiles
            if (NBX == 1) issue_x(hh + 1, xnext);
            if (NBH == 1 && hc) issue_h(hh + 1, hnext);
            wait_vmem();
            lds_barrier();
        }
    }
}

// Dynamic LDS above the default limit must be allowed per kernel and per
// device; done once per (instantiation, device). Concurrent first calls may
// both set it, which is harmless.
template <typename K>
static hipError_t allow_lds_once(K kern) {
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const uint64_t bit = 1ull << (dev & 63);
    if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kScanMaxLds);
    if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <typename T, int PT, int NT, typename ST, int NBX, int NBH, bool CBL, int VAR>
static hipError_t launch_sc2(const Params& p, int hpw, int lds, hipStream_t s) {
    auto kern = ssd_chunk_scan_kernel<T, PT, NT, ST, NBX, NBH, CBL, VAR == kScanGate || VAR == kScanGateVarlen,
                                      VAR == kScanVarlen || VAR == kScanGateVarlen>;
    hipError_t e = allow_lds_once(kern);
    if (e != hipSuccess) return e;
    const int64_t nhb = (p.heads_per_group + hpw - 1) / hpw;
    dim3 grid((unsigned)(p.nchunks * p.ngroups * nhb), (unsigned)p.batch);
    hipLaunchKernelGGL(kern, grid, dim3(kScanThreads), lds, s, p, hpw);
    return hipGetLastError();
}

// Heads per workgroup. Phase A (C B^T of the chunk, about 1.6 heads' worth of
// work) is paid once per workgroup, so more heads per workgroup amortise it,
// but the workgroups should fill the compute units in whole rounds (one
// workgroup per compute unit at a time). Minimise rounds x (1.6 + the most
// heads any workgroup takes).
static inline int scan_hpw(const Params& p) {
    const int64_t cus = device_cus();
    const int64_t chunks = p.batch * p.nchunks * p.ngroups, hpg = p.heads_per_group;
    int best = 1;
    double best_cost = 1e300;
    for (int64_t h = 1; h <= hpg && h <= 64; ++h) {
        const int64_t nhb = (hpg + h - 1) / h;
        const int64_t most = (hpg + nhb - 1) / nhb;
        const int64_t rounds = (chunks * nhb + cus - 1) / cus;
        const double cost = (double)rounds * (1.6 + (double)most);
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = (int)h;
        }
    }
    return best;
}

template <typename T, int PT, int NT, typename ST, int VAR>
static hipError_t launch_sc(const Params& p, hipStream_t s) {
    using Cfg = ScanCfg<T, PT, NT, ST>;
    const int Q = p.chunk < 32 ? 32 : (int)p.chunk;   // rows as tiled (whole 32-token tiles)
    const int hpw = scan_hpw(p);
    // prefer C B^T in LDS (frees the registers that would hold it), then
    // double-buffered copies
    const bool vl = VAR == kScanVarlen || VAR == kScanGateVarlen;
#define SSD_SC_TRY(NBX_, NBH_, CBL_)                                                           \
    if (Cfg::lds(Q, NBX_, NBH_, CBL_, vl) <= kScanMaxLds)                                      \
        return launch_sc2<T, PT, NT, ST, NBX_, NBH_, CBL_, VAR>(p, hpw, Cfg::lds(Q, NBX_, NBH_, CBL_, vl), s);
    if constexpr (sizeof(T) == 2 && sizeof(ST) == 2) { SSD_SC_TRY(2, 2, true) }
    if constexpr (sizeof(T) == 2) { SSD_SC_TRY(2, 1, true) }
    SSD_SC_TRY(1, 1, true) SSD_SC_TRY(1, 1, false)
#undef SSD_SC_TRY
    return hipErrorInvalidValue;
}

template <typename T, typename ST, int VAR>
static hipError_t dispatch_sc(const Params& p, hipStream_t s) {
    const int pt = (int)((p.headdim + 31) / 32), nt = (int)((p.dstate + 31) / 32);
#define SSD_SC_CASE(PT_, NT_) \
    if (pt == PT_ && nt == NT_) return launch_sc<T, PT_, NT_, ST, VAR>(p, s);
#define SSD_SC_ROW(PT_) SSD_SC_CASE(PT_, 1) SSD_SC_CASE(PT_, 2) SSD_SC_CASE(PT_, 4) SSD_SC_CASE(PT_, 8)
    SSD_SC_ROW(1) SSD_SC_ROW(2) SSD_SC_ROW(4)
#undef SSD_SC_ROW
#undef SSD_SC_CASE
    return hipErrorInvalidValue;
}

}  // namespace ssd
