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
// Work split. One workgroup of 8 wavefronts takes one chunk and `hpw` heads of
// one group; wavefront w owns the 32-token row tile w (rows j), for every head.
//  Phase A, once per workgroup: C B^T does not depend on the head when B and C
//  are shared (Knowl 7), so each wavefront computes its row of 32x32 tiles
//  M^T(kt) = B_kt . C_w^T (kt <= w) on the matrix cores, rounds them to the
//  operand type and keeps them in registers, together with its C rows.
//  Phase B, per head: x (token-major) and h_c ([P][N]) are copied into LDS by
//  global_load_lds, double-buffered so the next head's copy overlaps this
//  head's math. For every key tile the lane scales its 16 register values by
//  the decay (exp(cs_j - cs_r) * exp(cs_r - cs_i) dt_i with r the key tile's
//  last token off the diagonal; a direct exp with the causal mask on it) and
//  feeds them straight to Y += M . X as the A operand: an accumulator's rows
//  (8g + 4hf + r) become the next product's k index in "fragment order", and
//  the x fragment is read from LDS with transpose reads in the same order.
//  The carried-state term is (C . h_c) with rows scaled by exp(cs_j).
//  The epilogue adds D x_j and stores y (lane = column p).
#include "kernels.hpp"

namespace ssd {

constexpr int kScanMaxLds = 160 * 1024;
constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / 64;

template <typename T, int PT, int NT, typename ST>
struct ScanCfg {
    static constexpr int EPC = 16 / (int)sizeof(T);
    static constexpr int XRC = PT * 32 / EPC;                  // chunks per x row
    static constexpr int HRC = NT * 32 * (int)sizeof(ST) / 16; // chunks per h_c row
    static constexpr int HBYTES = PT * 32 * HRC * 16;          // one head's h_c tile
    static constexpr int KS = NT * 2;                          // k16 steps over n
    static constexpr int YBYTES = 8 * PT * 32 * (int)sizeof(T);    // per-wave y staging: 8 rows
    static constexpr int YCHUNKS = YBYTES / 16;                 // 16-byte row segments staged
    static constexpr int NSTORE = (YCHUNKS + 63) / 64;          // store instructions per 8 rows
    __host__ __device__ static int xbytes(int Q) { return Q * XRC * 16; }
    __host__ __device__ static int vbytes(int Q) { return 4 * Q * 4; }
    // bytes of LDS with nbx x buffers and nbh h_c buffers
    __host__ __device__ static int lds(int Q, int nbx, int nbh) {
        return nbx * xbytes(Q) + nbh * HBYTES + 2 * vbytes(Q) + kScanWaves * YBYTES;
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

template <typename T, int PT, int NT, typename ST, int NBX, int NBH>
__global__ __launch_bounds__(kScanThreads) void ssd_chunk_scan_kernel(Params p, int hpw) {
    using Cfg = ScanCfg<T, PT, NT, ST>;
    using V8 = typename Vec8<T>::type;
    constexpr int KS = Cfg::KS, XRC = Cfg::XRC, HRC = Cfg::HRC;
    constexpr int ESZ = (int)sizeof(T), SSZ = (int)sizeof(ST);
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    const int Q = (int)p.chunk;
    const int XB = Cfg::xbytes(Q), VB = Cfg::vbytes(Q);
    unsigned char* const hb0 = smem + NBX * XB;
    float* const vb0 = reinterpret_cast<float*>(hb0 + NBH * Cfg::HBYTES);
    unsigned char* const yst0 = reinterpret_cast<unsigned char*>(vb0) + 2 * VB;

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
    const int64_t h0 = g * hpg + (int64_t)hb * hpw;
    const int nh = (int)min<int64_t>(hpw, hpg - (int64_t)hb * hpw);
    const int64_t t0 = (int64_t)c * Q;
    const int qc = (int)min<int64_t>(Q, T_ - t0);
    const int64_t tok0 = b * T_ + t0;            // first token row of the chunk

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    // Row tile of this wavefront. Waves w and w+4 share a SIMD; with 8 tiles
    // they take tiles s and 7 - s, so every SIMD carries 9 key tiles of work.
    const int RT = Q / 32;
    const int rt = RT == 8 ? (wave < 4 ? wave : 11 - wave) : (wave < RT ? wave : -1);
    const bool active = rt >= 0;
    unsigned char* const yst = yst0 + wave * Cfg::YBYTES;

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

    auto issue_x = [&](int hh, int buf) {
        dma_tile<XRC>(smem + buf * XB, Q, qc, xvalid, xbase + (int64_t)hh * P * ESZ, xstride, wave, kScanWaves, lane);
    };
    auto issue_h = [&](int hh, int buf) {
        dma_tile<HRC>(hb0 + buf * Cfg::HBYTES, PT * 32, (int)P, hvalid, sbase + (int64_t)hh * P * N * SSZ,
                      (uint32_t)(N * SSZ), wave, kScanWaves, lane);
    };
    float vcs = 0.0f, vcr = 0.0f, vdt = 0.0f;   // thread i holds token i of the next head
    auto load_vec = [&](int hh) {
        const int i = threadIdx.x;
        if (i < Q) {
            const float* csr = csbase + (int64_t)hh * nc * Q;
            vcs = ldg(csr + i);
            vcr = ldg(csr + (i | 31));
            vdt = (i < qc) ? ldg(dtbase + hh + (uint32_t)i * (uint32_t)H) : 0.0f;
        }
    };
    auto store_vec = [&](int buf) {
        const int i = threadIdx.x;
        if (i < Q) {
            float* v = vb0 + buf * (VB / 4);
            const float c2 = vcs * kLog2e, c2r = vcr * kLog2e;
            v[i] = c2;
            v[Q + i] = vdt;
            v[2 * Q + i] = exp2f(c2);
            v[3 * Q + i] = exp2f(c2r - c2) * vdt;
        }
    };

    // head 0's tiles start moving before phase A
    if (nh > 0) {
        issue_x(0, 0);
        if (c > 0) issue_h(0, 0);
        load_vec(0);
    }

    // ---- phase A: this wave's C rows and C B^T row of tiles, once per workgroup ----
    const int nlast = (int)N - 8;
    V8 creg[KS];
    V8 cb[7][2];     // key tiles kt < rt
    V8 cbd[2];       // the diagonal tile
    if (active) {
        auto off = [&](int row, int ks) {
            return (uint32_t)min(row, qc - 1) * bcs + (uint32_t)min(ks * 16 + hf * 8, nlast);
        };
        const int jl = rt * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const V8 raw = ldg8(cbase + off(jl, ks));
            creg[ks] = (jl < qc && ks * 16 + hf * 8 < (int)N) ? raw : zero8<T>();
        }
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
                V8 lo, hi;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    lo[e] = from_f32<T>(acc[e]);
                    hi[e] = from_f32<T>(acc[8 + e]);
                }
                if (kt < rt) {
                    cb[kt < 7 ? kt : 6][0] = lo;
                    cb[kt < 7 ? kt : 6][1] = hi;
                } else {
                    cbd[0] = lo;
                    cbd[1] = hi;
                }
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

    if (nh > 0) store_vec(0);
    wait_vmem();
    __syncthreads();

    // ---- phase B: heads ----
    for (int hh = 0; hh < nh; ++hh) {
        const int buf = hh & 1;
        const int xbi = NBX == 2 ? buf : 0;
        const int hbi = NBH == 2 ? buf : 0;
        const bool more = hh + 1 < nh;
        if (more) {
            if (NBX == 2) issue_x(hh + 1, buf ^ 1);
            if (NBH == 2 && c > 0) issue_h(hh + 1, buf ^ 1);
            load_vec(hh + 1);
        }
        bool stored_all = true;
        if (active) {
            const unsigned char* xt = smem + xbi * XB;
            const unsigned char* ht = hb0 + hbi * Cfg::HBYTES;
            const float* c2v = vb0 + buf * (VB / 4);
            const float* dtv = c2v + Q;
            const float* ecs = c2v + 2 * Q;
            const float* uv = c2v + 3 * Q;
            int jl = rt * 32 + l32, qch = qc;
            asm volatile("" : "+v"(jl), "+v"(qch));    // keep per-element compares in the loop
            f32x16 acc[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) acc[pt] = zero16();

            if (c > 0) {   // (C . h_c), rows then scaled by exp(cs_j)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        const int row = pt * 32 + l32;
                        const int cbyte = (ks * 16 + hf * 8) * SSZ;   // 16 or 32 bytes
                        const unsigned char* rp = ht + row * HRC * 16;
                        typename Vec8<ST>::type hv;
                        if constexpr (SSZ == 2) {
                            hv = *reinterpret_cast<const bf16x8*>(rp + ((((cbyte >> 4)) ^ hsw) << 4));
                        } else {
                            const f32x4 lo = *reinterpret_cast<const f32x4*>(rp + (((cbyte >> 4) ^ hsw) << 4));
                            const f32x4 hi = *reinterpret_cast<const f32x4*>(rp + ((((cbyte >> 4) + 1) ^ hsw) << 4));
                            hv[0] = lo[0]; hv[1] = lo[1]; hv[2] = lo[2]; hv[3] = lo[3];
                            hv[4] = hi[0]; hv[5] = hi[1]; hv[6] = hi[2]; hv[7] = hi[3];
                        }
                        mma_k16(acc[pt], creg[ks], cvt8<T>(hv));
                    }
                }
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 e4 = *reinterpret_cast<const f32x4*>(ecs + rt * 32 + 8 * gq + 4 * hf);
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[pt][4 * gq + r] *= e4[r];
                }
            }

            const float c2j = c2v[jl];
            // key tiles off the diagonal: M = CB * exp(cs_j - cs_r) * u_i, no mask
#pragma unroll
            for (int kt = 0; kt < 7; ++kt) {
                if (kt < rt) {
                    const float vj = fast_exp2(c2j - c2v[kt * 32 + 31]);
                    V8 aop[2];
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const f32x4 u4 = *reinterpret_cast<const f32x4*>(uv + kt * 32 + 8 * gq + 4 * hf);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int idx = 4 * gq + r;
                            aop[idx >> 3][idx & 7] = from_f32<T>(to_f32(cb[kt][idx >> 3][idx & 7]) * vj * u4[r]);
                        }
                    }
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int pt = 0; pt < PT; ++pt)
                            mma_k16(acc[pt], aop[s], x_frag<T, XRC>(xt, 2 * kt + s, pt, xoa, xob, lane));
                }
            }
            // the diagonal tile: direct decay; the causal mask (i <= j) enters as a
            // -inf exponent for i > j, so exp2 gives exactly 0 with no lane masks
            V8 xd[PT][2];
            {
                V8 aop[2];
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int ib = rt * 32 + 8 * gq + 4 * hf;
                    const f32x4 ci = *reinterpret_cast<const f32x4*>(c2v + ib);
                    const f32x4 di = *reinterpret_cast<const f32x4*>(dtv + ib);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int idx = 4 * gq + r;
                        const float pen = __int_as_float(((jl - (ib + r)) >> 31) & (int)0xff800000u);
                        const float m = to_f32(cbd[idx >> 3][idx & 7]) * fast_exp2((c2j - ci[r]) + pen) * di[r];
                        aop[idx >> 3][idx & 7] = from_f32<T>(m);
                    }
                }
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int pt = 0; pt < PT; ++pt) {
                        xd[pt][s] = x_frag<T, XRC>(xt, 2 * rt + s, pt, xoa, xob, lane);
                        mma_k16(acc[pt], aop[s], xd[pt][s]);
                    }
            }

            // epilogue: y = acc + D x_j, staged through this wave's LDS slab
            // (8 rows at a time: accumulator quarter gq holds rows 8gq + 4hf + r)
            // and written as 16-byte row segments
            const float Dh = ldg(p.D + h0 + hh);
            unsigned char* yh = ybase + (int64_t)hh * P * ESZ;
            const uint32_t ystride = (uint32_t)(H * P * ESZ);
            constexpr int RB = PT * 32 * ESZ;                   // staged row bytes
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 4 * (gq & 1) + r;
                        *reinterpret_cast<T*>(yst + (4 * hf + r) * RB + (pt * 32 + l32) * ESZ) =
                            from_f32<T>(acc[pt][4 * gq + r] + Dh * to_f32(xd[pt][gq >> 1][e]));
                    }
                }
#pragma unroll
                for (int k = 0; k < Cfg::NSTORE; ++k) {
                    const int idx = k * 64 + lane;
                    const int jr = idx / (RB / 16), cb16 = idx % (RB / 16);
                    const u32x4 val = *reinterpret_cast<const u32x4*>(yst + (idx < Cfg::YCHUNKS ? idx : 0) * 16);
                    const int j = rt * 32 + 8 * gq + jr;
                    if (idx < Cfg::YCHUNKS && j < qch && cb16 * 16 < (int)(P * ESZ))
                        *(__attribute__((address_space(1))) u32x4*)(yh + (uint32_t)j * ystride + cb16 * 16) = val;
                    else if (idx < Cfg::YCHUNKS)
                        stored_all = false;
                }
            }
        }
        if (more) store_vec(buf ^ 1);
        // the next head's copies were issued before this head's stores: wait
        // for everything but the stores just issued (all lanes stored) or all
        if (__builtin_amdgcn_readfirstlane(__any(!stored_all) ? 1 : 0) == 0 && active)
            wait_vmem_le<4 * Cfg::NSTORE>();
        else
            wait_vmem();
        __syncthreads();
        if (more && (NBX == 1 || (NBH == 1 && c > 0))) {   // single-buffered tiles
            if (NBX == 1) issue_x(hh + 1, 0);
            if (NBH == 1 && c > 0) issue_h(hh + 1, 0);
            wait_vmem();
            __syncthreads();
        }
    }
}

template <typename T, int PT, int NT, typename ST, int NBX, int NBH>
static hipError_t launch_sc2(const Params& p, int hpw, int lds, hipStream_t s) {
    auto kern = ssd_chunk_scan_kernel<T, PT, NT, ST, NBX, NBH>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    const int64_t nhb = (p.heads_per_group + hpw - 1) / hpw;
    dim3 grid((unsigned)(p.nchunks * p.ngroups * nhb), (unsigned)p.batch);
    hipLaunchKernelGGL(kern, grid, dim3(kScanThreads), lds, s, p, hpw);
    return hipGetLastError();
}

// heads per workgroup: amortise phase A over up to 8 heads while keeping at
// least ~512 workgroups in flight.
static int scan_hpw(const Params& p) {
    const int64_t units = p.batch * p.nchunks * p.nheads;
    int64_t hpw = units / 512;
    if (hpw > 8) hpw = 8;
    if (hpw > p.heads_per_group) hpw = p.heads_per_group;
    if (hpw < 1) hpw = 1;
    return (int)hpw;
}

template <typename T, int PT, int NT, typename ST>
static hipError_t launch_sc(const Params& p, hipStream_t s) {
    using Cfg = ScanCfg<T, PT, NT, ST>;
    const int Q = (int)p.chunk;
    const int hpw = scan_hpw(p);
    if (Cfg::lds(Q, 2, 2) <= kScanMaxLds) return launch_sc2<T, PT, NT, ST, 2, 2>(p, hpw, Cfg::lds(Q, 2, 2), s);
    if (Cfg::lds(Q, 2, 1) <= kScanMaxLds) return launch_sc2<T, PT, NT, ST, 2, 1>(p, hpw, Cfg::lds(Q, 2, 1), s);
    if (Cfg::lds(Q, 1, 1) <= kScanMaxLds) return launch_sc2<T, PT, NT, ST, 1, 1>(p, hpw, Cfg::lds(Q, 1, 1), s);
    return hipErrorInvalidValue;
}

template <typename T, typename ST>
static hipError_t dispatch_sc(const Params& p, hipStream_t s) {
    const int pt = (int)((p.headdim + 31) / 32), nt = (int)((p.dstate + 31) / 32);
#define SSD_SC_CASE(PT_, NT_) \
    if (pt == PT_ && nt == NT_) return launch_sc<T, PT_, NT_, ST>(p, s);
#define SSD_SC_ROW(PT_) SSD_SC_CASE(PT_, 1) SSD_SC_CASE(PT_, 2) SSD_SC_CASE(PT_, 4) SSD_SC_CASE(PT_, 8)
    SSD_SC_ROW(1) SSD_SC_ROW(2) SSD_SC_ROW(4)
#undef SSD_SC_ROW
#undef SSD_SC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_scan(const Params& p, int dtype, int state_dtype, hipStream_t s) {
    if (dtype == 1 && state_dtype == 1) return dispatch_sc<bf16, bf16>(p, s);
    if (dtype == 1) return dispatch_sc<bf16, float>(p, s);
    return dispatch_sc<float, float>(p, s);
}

// Smallest LDS the chunk scan needs for (dtype, state dtype, P, N, Q): single
// x and h_c buffers; used by argument checking.
int chunk_scan_lds_bytes(int dtype, int state_dtype, int64_t P, int64_t N, int64_t Q) {
    const int esz = dtype == 1 ? 2 : 4, ssz = state_dtype == 1 ? 2 : 4;
    const int pp = (int)((P + 31) / 32) * 32, np = (int)((N + 31) / 32) * 32;
    return (int)Q * pp * esz + pp * np * ssz + 2 * 4 * (int)Q * 4 + kScanWaves * 8 * pp * esz;
}

}  // namespace ssd
