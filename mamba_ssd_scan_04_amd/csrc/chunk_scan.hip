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
// Matrix-core mapping. Row tiles of 32 tokens j; key tiles of 32 tokens i.
//  1. M^T tile = B_i-tile . C_j-tile^T over n (both operands read straight
//     from memory: B and C rows are n-contiguous). Its accumulator gives each
//     lane one column j and 16 rows i.
//  2. The lane scales its 16 values by exp(cs_j - cs_i) dt_i (masking i > j),
//     rounds them to the operand type, and uses them directly as the A operand
//     (row j, 8 values of k = i per lane half) of Y += M . X. The k order this
//     induces is matched by storing x^T in LDS in "fragment order"
//     (frag_token), so no data moves between lanes.
//  3. Y += (exp(cs_j) C_j) . h_c, with h_c staged in LDS ([P][N], k-major).
//  4. Epilogue adds D x_j (x read back from the LDS tile) and stores y.
// The accumulator of Y holds column p = lane%32 and 16 rows j per lane.
//
// Grid: (chunk, head, batch), 256 threads = 4 wavefronts. With 8 row tiles,
// wavefront w takes tiles w and 7 - w so the causal work (rt + 1 key tiles
// per row tile) is balanced.
#include "kernels.hpp"
#include "transpose.hpp"

namespace ssd {

constexpr int kScanMaxLds = 160 * 1024;

template <typename T> constexpr int pad_elems() { return 16 / (int)sizeof(T); }

template <typename T, int PT, int NT>
__host__ __device__ constexpr int scan_ldh() { return NT * 32 + pad_elems<T>(); }

// Dynamic LDS bytes of the chunk scan for chunk size Q.
template <typename T, int PT, int NT>
__host__ __device__ inline int scan_lds_bytes(int Q) {
    return PT * 32 * (Q + pad_elems<T>()) * (int)sizeof(T) + PT * 32 * scan_ldh<T, PT, NT>() * (int)sizeof(T) +
           2 * Q * (int)sizeof(float);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type scale8(const typename Vec8<T>::type& v, float s) {
    typename Vec8<T>::type o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(to_f32(v[e]) * s);
    return o;
}

template <typename T, int PT, int NT, typename ST>
__global__ __launch_bounds__(256) void ssd_chunk_scan_kernel(Params p) {
    constexpr int PP = PT * 32, NP = NT * 32, KS = NP / 16;
    constexpr int LDH = scan_ldh<T, PT, NT>();
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int Q = (int)p.chunk;
    const int LDX = Q + pad_elems<T>();
    T* xs = reinterpret_cast<T*>(smem);                 // [PP][LDX]  x^T, fragment order
    T* hs = xs + PP * LDX;                              // [PP][LDH]  h_c^T
    float* c2s = reinterpret_cast<float*>(hs + PP * LDH);  // [Q] cs * log2(e)
    float* dts = c2s + Q;                               // [Q] dt (0 past the end)

    const int c = blockIdx.x;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int64_t T_ = p.seqlen, H = p.nheads, P = p.headdim, N = p.dstate, G = p.ngroups;
    const int64_t g = h / p.heads_per_group;
    const int64_t t0 = (int64_t)c * Q;
    const T* xg = static_cast<const T*>(p.x);
    const T* bg = static_cast<const T*>(p.B);
    const T* cg = static_cast<const T*>(p.C);

    const float* csrow = p.cs + ((b * H + h) * p.nchunks + c) * Q;
    for (int j = threadIdx.x; j < Q; j += blockDim.x) {
        const int64_t t = t0 + j;
        c2s[j] = csrow[j] * kLog2e;
        dts[j] = (t < T_) ? p.dt[(b * T_ + t) * H + h] : 0.0f;
    }
    // x^T in fragment order: block m covers LDS positions [8m, 8m+8) of a row
    for (int sb = threadIdx.x; sb < (Q / 8) * (PP / 8); sb += blockDim.x) {
        const int col = (sb % (PP / 8)) * 8, m = sb / (PP / 8);
        float v[8][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int q = 8 * m + e;
            const int j = (q & ~15) + frag_token(q & 15);
            const int64_t t = t0 + j;
            load_row8<T>(v[e], xg + ((b * T_ + t) * H + h) * P + col, (t < T_) && (col < P));
        }
        store_transposed8<T>(xs + col * LDX + 8 * m, LDX, v);
    }
    if (c > 0) {
        const ST* sg = static_cast<const ST*>(p.states) + ((b * p.nchunks + c) * H + h) * P * N;
        for (int it = threadIdx.x; it < PP * (NP / 8); it += blockDim.x) {
            const int pr = it / (NP / 8), n0 = (it % (NP / 8)) * 8;
            float v[8];
            load_row8<ST>(v, sg + pr * N + n0, (pr < P) && (n0 < N));
            typename Vec8<T>::type o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e]);
            store8(hs + pr * LDH + n0, o);
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hf = lane >> 5, l32 = lane & 31;
    const int RT = Q / 32;
    int tiles[2] = {-1, -1};
    if (RT == 8) {
        tiles[0] = wave;
        tiles[1] = 7 - wave;
    } else if (wave < RT) {
        tiles[0] = wave;
    }
    const float Dh = p.D[h];
    T* yg = static_cast<T*>(p.y);

    for (int ti = 0; ti < 2; ++ti) {
        const int rt = tiles[ti];
        if (rt < 0) continue;
        const int jl = rt * 32 + l32;            // this lane's row j (as MFMA column / A row)
        const int64_t tj = t0 + jl;
        typename Vec8<T>::type creg[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int n0 = ks * 16 + hf * 8;
            creg[ks] = (tj < T_ && n0 < N) ? load8(cg + ((b * T_ + tj) * G + g) * N + n0) : zero8<T>();
        }
        f32x16 acc[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) acc[pt] = zero16();
        const float c2j = c2s[jl];

        if (c > 0) {  // off-diagonal term: (exp(cs_j) C_j) . h_c
            const float sj = exp2f(c2j);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const auto a = scale8<T>(creg[ks], sj);
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    mma_k16(acc[pt], a, load8(hs + (pt * 32 + l32) * LDH + ks * 16 + hf * 8));
            }
        }

        for (int kt = 0; kt <= rt; ++kt) {
            const int il = kt * 32 + l32;
            const int64_t ti_ = t0 + il;
            f32x16 cb = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int n0 = ks * 16 + hf * 8;
                const auto bop = (ti_ < T_ && n0 < N) ? load8(bg + ((b * T_ + ti_) * G + g) * N + n0) : zero8<T>();
                mma_k16(cb, bop, creg[ks]);
            }
            // cb[r]: row i = kt*32 + 8*(r/4) + 4*hf + r%4, column j = jl
            typename Vec8<T>::type aop[2];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int ib = kt * 32 + 8 * q4 + 4 * hf;
                const f32x4 ci = *reinterpret_cast<const f32x4*>(c2s + ib);
                const f32x4 di = *reinterpret_cast<const f32x4*>(dts + ib);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = cb[4 * q4 + r] * exp2f(c2j - ci[r]) * di[r];
                    v = (ib + r <= jl) ? v : 0.0f;
                    aop[q4 >> 1][4 * (q4 & 1) + r] = from_f32<T>(v);
                }
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int pt = 0; pt < PT; ++pt)
                    mma_k16(acc[pt], aop[s], load8(xs + (pt * 32 + l32) * LDX + (kt * 2 + s) * 16 + hf * 8));
            }
        }

        // epilogue: + D x_j, store y
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const int pc = pt * 32 + l32;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const auto xv = load8(xs + pc * LDX + (rt * 2 + s) * 16 + hf * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * s + e;
                    const int j = rt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    const int64_t t = t0 + j;
                    if (t < T_ && pc < P)
                        yg[((b * T_ + t) * H + h) * P + pc] = from_f32<T>(acc[pt][r] + Dh * to_f32(xv[e]));
                }
            }
        }
    }
}

template <typename T, int PT, int NT, typename ST>
static hipError_t launch_sc(const Params& p, hipStream_t s) {
    const int lds = scan_lds_bytes<T, PT, NT>((int)p.chunk);
    if (lds > kScanMaxLds) return hipErrorInvalidValue;
    auto kern = ssd_chunk_scan_kernel<T, PT, NT, ST>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)p.nchunks, (unsigned)p.nheads, (unsigned)p.batch);
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, p);
    return hipGetLastError();
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

// LDS the chunk scan needs for (dtype, P, N, Q); used by argument checking.
int chunk_scan_lds_bytes(int dtype, int64_t P, int64_t N, int64_t Q) {
    const int pt = (int)((P + 31) / 32), nt = (int)((N + 31) / 32);
    const int esz = dtype == 1 ? 2 : 4, pad = 16 / esz;
    return pt * 32 * ((int)Q + pad) * esz + pt * 32 * (nt * 32 + pad) * esz + 2 * (int)Q * 4;
}

}  // namespace ssd
