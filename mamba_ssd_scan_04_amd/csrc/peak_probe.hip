// Attainable-peak probes for the roofline: what the matrix cores and HBM
// deliver on this chip when nothing else limits them, to set beside the
// datasheet peaks the kernels are reported against. Built into its own
// library (libssd_peak.so); nothing on the SSD path calls it.
//
//   ssd_peak_mfma_bf16   every wave issues a long chain of
//                        v_mfma_f32_32x32x16_bf16 on register operands, four
//                        independent accumulators deep so that the matrix
//                        pipe never waits on a result; 32*32*16*2 = 32768
//                        flop per instruction.
//   ssd_peak_stream      y = x over n 16-byte vectors, grid-stride, four
//                        non-temporal loads in flight per thread, then their
//                        stores: a plain read + write stream (bytes moved =
//                        2 * 16 * n).
//   ssd_peak_stream_pieces
//                        the same copy, each workgroup one contiguous 4 KB
//                        piece (one non-temporal 16-byte vector per thread),
//                        ceil(n / 256) workgroups: the fastest of the copy
//                        patterns measured on this GPU (many short workgroups
//                        with little in flight each beat few long ones).
//   ssd_peak_scan_traffic
//                        the chunk scan's memory traffic with none of its
//                        arithmetic: the same grid, workgroup size, heads per
//                        workgroup and block order; per workgroup the chunk's
//                        B and C rows, then per head the copies of the next
//                        head's x tile and carried state into LDS (one head
//                        ahead, double-buffered, as buffer loads straight to
//                        LDS), its dt and cs values, and this head's y tile
//                        stored from LDS (y = x, so the copy can be checked);
//                        the copies are waited for and the stores are not.
//   ssd_peak_state_traffic
//                        the chunk state's memory traffic with none of its
//                        arithmetic: the same grid, heads per workgroup and
//                        block order, 4 wavefronts; per workgroup the chunk's
//                        B rows and its heads' x rows in blocks of 32 tokens
//                        through a 3-deep LDS ring (buffer loads straight to
//                        LDS, two blocks in flight), the heads' dt values into
//                        a side tile with the first block, then per head its
//                        Q cs values (= dt) and its P x N state, made of the
//                        last block's x rows repeated (so the copy can be
//                        checked).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 pk_bf16x8;
typedef __attribute__((ext_vector_type(16))) float pk_f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned pk_u32x4;

namespace {

constexpr int kAcc = 4;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* out) {
    pk_bf16x8 a, b;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(1.0f + 0.001f * (float)(lane + k));
        b[k] = (__bf16)(0.5f - 0.001f * (float)(lane - k));
    }
    pk_f32x16 acc[kAcc];
#pragma unroll
    for (int u = 0; u < kAcc; ++u)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[u][k] = 0.0f;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < kAcc; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kAcc; ++u)
#pragma unroll
        for (int k = 0; k < 16; ++k) s += acc[u][k];
    // one value per thread, so the chain cannot be dropped
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// grid-stride over groups of kUnroll vectors per thread: all of a group's
// loads are issued before its stores, so each wave keeps kUnroll loads in
// flight
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void stream_kernel(const pk_u32x4* __restrict__ x, pk_u32x4* __restrict__ y,
                                                     int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        pk_u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(x + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], y + i + u * stride);
    }
    for (; i < n; i += stride) y[i] = x[i];
}

// one 16-byte vector per thread, one contiguous 4 KB piece per workgroup
__global__ __launch_bounds__(256) void stream_piece_kernel(const pk_u32x4* __restrict__ x, pk_u32x4* __restrict__ y,
                                                           int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(x + i), y + i);
}

struct ScanTraffic {
    const unsigned char* x;
    const unsigned char* B;
    const unsigned char* C;
    const unsigned char* states;
    const float* dt;
    const float* cs;
    unsigned char* y;
    float* sink;
    int64_t T, H, P, N, G, Q, nc, hpw;
    int nt;   // x and state copies non-temporal
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t probe_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// 16-byte pieces: piece k of a rows x rb tile (rb bytes per row) is row k / (rb/16),
// bytes 16 (k % (rb/16)) of it; LDS holds the tile row-major, unswizzled.
// NT: the non-temporal policy (aux bit 1), as the kernels take it for data
// whose footprint exceeds the last-level cache.
template <bool NT>
__device__ __forceinline__ void probe_copy_tile(unsigned char* lds, const unsigned char* g, int rows, int rb,
                                                uint32_t stride) {
    const __amdgpu_buffer_rsrc_t rs = probe_rsrc(g);
    const int per_row = rb / 16, total = rows * per_row;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    for (int k0 = wave * 64; k0 < total; k0 += 512) {
        const int k = k0 + lane;
        const int kk = k < total ? k : total - 1;   // the last lanes of a partial group repeat a piece
        const uint32_t off = (uint32_t)(kk / per_row) * stride + 16u * (uint32_t)(kk % per_row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + k0 * 16), 16, off,
                                                 0, 0, NT ? 2 : 0);
    }
}

__global__ __launch_bounds__(512) void scan_traffic_kernel(ScanTraffic a) {
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    const int64_t H = a.H, P = a.P, N = a.N, G = a.G, Q = a.Q, nc = a.nc;
    const unsigned char* const xg = a.x;
    const unsigned char* const sg = a.states;
    const float* const csg = a.cs;
    const float* const dtg = a.dt;
    const int64_t hpg = H / G;
    const int nhb = (int)((hpg + a.hpw - 1) / a.hpw);
    const int total = (int)(gridDim.x * gridDim.y), id = (int)(blockIdx.x + gridDim.x * blockIdx.y);
    const int lin = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;   // XCD-aware, as the chunk scan
    int bx = lin % (int)gridDim.x;
    const int hb = bx % nhb;
    bx /= nhb;
    const int64_t g = bx % G;
    const int64_t c = bx / G;
    const int64_t b = lin / (int)gridDim.x;
    const int64_t h0 = g * hpg + hb;
    const int nh = (int)((hpg - hb + nhb - 1) / nhb);
    const int64_t tok0 = b * a.T + c * Q;
    const int xrb = (int)(P * 2), hrb = (int)(P * N * 2);
    const int XB = (int)(Q * xrb), HB = hrb;
    const uint32_t xstride = (uint32_t)(H * P * 2);
    float acc = 0.0f;
    // the chunk's B and C rows (group g), read into registers, every load
    // issued before any is used (at most 8 16-byte pieces of each per thread)
    {
        uint4 vb[8], vc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t k = threadIdx.x + 512 * u;
            const int64_t kk = k < Q * N / 8 ? k : Q * N / 8 - 1;
            const int64_t o = ((tok0 + kk / (N / 8)) * G + g) * N + 8 * (kk % (N / 8));
            vb[u] = *reinterpret_cast<const uint4*>(a.B + 2 * o);
            vc[u] = *reinterpret_cast<const uint4*>(a.C + 2 * o);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc += (float)(vb[u].x ^ vb[u].y ^ vb[u].z ^ vb[u].w ^ vc[u].x ^ vc[u].y ^ vc[u].z ^ vc[u].w);
    }
    // per head: the x tile, the carried state (none for chunk 0) and the
    // head's Q cs and Q dt values (waves 0-3: cs, 4-7: dt, 4 bytes per lane)
    unsigned char* const vl = smem + 2 * XB + 2 * HB;   // [2][2][256] floats
    auto issue_into = [&](int hh, unsigned char* xl, unsigned char* hl, unsigned char* vb) __attribute__((always_inline)) {
        const int64_t h = h0 + (int64_t)hh * nhb;
        if (a.nt) {
            probe_copy_tile<true>(xl, xg + (tok0 * H + h) * P * 2, (int)Q, xrb, xstride);
            if (c > 0) probe_copy_tile<true>(hl, sg + ((b * nc + c) * H + h) * P * N * 2, 1, hrb, 0);
        } else {
            probe_copy_tile<false>(xl, xg + (tok0 * H + h) * P * 2, (int)Q, xrb, xstride);
            if (c > 0) probe_copy_tile<false>(hl, sg + ((b * nc + c) * H + h) * P * N * 2, 1, hrb, 0);
        }
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
        const int i = (wave & 3) * 64 + lane, ic = i < Q ? i : (int)Q - 1;
        unsigned char* dst = vb + (wave >> 2) * 1024 + (wave & 3) * 256;
        const uint32_t off = wave < 4 ? 4u * (uint32_t)(((b * H + h) * nc + c) * Q + ic)
                                      : 4u * (uint32_t)((tok0 + ic) * H + h);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(probe_rsrc(wave < 4 ? (const void*)csg : (const void*)dtg),
                                                 (__attribute__((address_space(3))) void*)dst, 4, off, 0, 0, 0);
    };
    if (nh > 0) issue_into(0, smem, smem + 2 * XB, vl);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    unsigned char* const yb = a.y;
    // one head: copies of the next head into the other buffers, y from this
    // head's x tile; the buffers as non-aliasing pointers, so that the LDS
    // reads of this head do not wait for the copies in flight
    auto head = [&](int hh, const unsigned char* __restrict__ xl, unsigned char* __restrict__ xn,
                    unsigned char* __restrict__ hn, unsigned char* __restrict__ vn) __attribute__((always_inline)) {
        const int64_t h = h0 + (int64_t)hh * nhb;
        if (hh + 1 < nh) issue_into(hh + 1, xn, hn, vn);
        // y tile of this head = its x tile, 16 bytes per lane per store
        unsigned char* yg = yb + (tok0 * H + h) * P * 2;
        const int per_row = xrb / 16;
        int nst = 0;
        for (int k = threadIdx.x; k < Q * per_row; k += 512, ++nst) {
            const uint4 v = *reinterpret_cast<const uint4*>(xl + 16 * k);
            *reinterpret_cast<uint4*>(yg + (uint32_t)(k / per_row) * xstride + 16 * (k % per_row)) = v;
        }
        // the copies have landed: every memory operation of this wavefront
        // but its nst stores (vmcnt(nst), gfx9 encoding) has completed
        switch (nst) {
            case 1: __builtin_amdgcn_s_waitcnt(0x0f71); break;
            case 2: __builtin_amdgcn_s_waitcnt(0x0f72); break;
            case 3: __builtin_amdgcn_s_waitcnt(0x0f73); break;
            case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
            default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
        }
        __builtin_amdgcn_s_barrier();
    };
    for (int hh = 0; hh < nh; ++hh) {
        const int cur = hh & 1, nxt = cur ^ 1;
        head(hh, smem + cur * XB, smem + nxt * XB, smem + 2 * XB + nxt * HB, vl + nxt * 2048);
        acc += reinterpret_cast<const float*>(vl + nxt * 2048)[threadIdx.x & 255];
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x == 0) a.sink[lin] = acc;
}

struct StateTraffic {
    const unsigned char* x;
    const unsigned char* B;
    const float* dt;
    float* cs;
    unsigned char* states;
    int64_t T, H, P, N, G, Q, nc, hpw;
    int nt;   // x copies non-temporal
};

// Copies of a rows x rb tile (16-byte pieces, row-major in LDS) by 4
// wavefronts; rows * rb / 16 is a multiple of 256, so every wavefront issues
// rows * rb / 4096 instructions.
template <bool NT>
__device__ __forceinline__ void probe_copy_tile4(unsigned char* lds, const unsigned char* g, int rows, int rb,
                                                 uint32_t stride, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t rs = probe_rsrc(g);
    const int per_row = rb / 16, total = rows * per_row;
    for (int k0 = wave * 64; k0 < total; k0 += 256) {
        const int k = k0 + lane;
        const uint32_t off = (uint32_t)(k / per_row) * stride + 16u * (uint32_t)(k % per_row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + k0 * 16), 16, off,
                                                 0, 0, NT ? 2 : 0);
    }
}

constexpr int kStBlk = 32;   // tokens per ring block

// wait until at most n (0..8) of this wavefront's vector memory operations are
// outstanding (vmcnt(n), gfx9 encoding); larger n waits for all
__device__ __forceinline__ void probe_wait_le(int n) {
    switch (n) {
        case 1: __builtin_amdgcn_s_waitcnt(0x0f71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0f72); break;
        case 3: __builtin_amdgcn_s_waitcnt(0x0f73); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0f75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0f76); break;
        case 7: __builtin_amdgcn_s_waitcnt(0x0f77); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0f78); break;
        default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    }
}

__global__ __launch_bounds__(256) void state_traffic_kernel(StateTraffic a) {
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    const int64_t H = a.H, P = a.P, N = a.N, G = a.G, Q = a.Q, nc = a.nc, hpw = a.hpw;
    const int64_t hpg = H / G;
    const int nhb = (int)((hpg + hpw - 1) / hpw);
    const int total = (int)(gridDim.x * gridDim.y), id = (int)(blockIdx.x + gridDim.x * blockIdx.y);
    const int lin = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;   // XCD-aware, as the chunk state
    int bx = lin % (int)gridDim.x;
    const int hb = bx % nhb;
    bx /= nhb;
    const int64_t g = bx % G;
    const int64_t c = bx / G;
    const int64_t b = lin / (int)gridDim.x;
    const int64_t h0 = g * hpg + (int64_t)hb * hpw;
    const int nh = (int)(hpg - (int64_t)hb * hpw < hpw ? hpg - (int64_t)hb * hpw : hpw);
    const int64_t tok0 = b * a.T + c * Q;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int xrb = (int)(P * 2), brb = (int)(N * 2);
    const int XB = kStBlk * xrb, BB = kStBlk * brb, BUF = BB + (int)hpw * XB;
    const uint32_t xstride = (uint32_t)(H * P * 2), bstride = (uint32_t)(G * N * 2);
    const unsigned char* const xg = a.x + (tok0 * H + h0) * P * 2;
    const unsigned char* const bg = a.B + (tok0 * G + g) * N * 2;
    float* const side = reinterpret_cast<float*>(smem + 3 * BUF);   // [hpw][Q] dt, hpw * 256 floats
    const int nblk = (int)(Q / kStBlk);
    // copies per wavefront per block (every wavefront issues the same number)
    const int per_block = (int)(kStBlk * brb / 4096 + nh * (kStBlk * xrb / 4096));
    auto issue = [&](int blk, unsigned char* base) __attribute__((always_inline)) {
        const uint32_t r0 = (uint32_t)(blk * kStBlk);
        probe_copy_tile4<false>(base, bg + r0 * bstride, kStBlk, brb, bstride, wave, lane);
        if (a.nt) {
            for (int hq = 0; hq < nh; ++hq)
                probe_copy_tile4<true>(base + BB + hq * XB, xg + r0 * xstride + (int64_t)hq * P * 2, kStBlk, xrb,
                                       xstride, wave, lane);
        } else {
            for (int hq = 0; hq < nh; ++hq)
                probe_copy_tile4<false>(base + BB + hq * XB, xg + r0 * xstride + (int64_t)hq * P * 2, kStBlk, xrb,
                                        xstride, wave, lane);
        }
    };
    // the side tile: value i = (head i / Q, token i % Q), 4 bytes per lane
    const int sround = (int)((hpw * Q + 255) / 256);
    issue(0, smem);
    {
        const __amdgpu_buffer_rsrc_t rd = probe_rsrc(a.dt);
        for (int i = 0; i < sround; ++i) {
            const int fi = (wave + 4 * i) * 64 + lane, hq = fi / (int)Q, j = fi - hq * (int)Q;
            const bool ok = hq < nh;
            const uint32_t off = ok ? 4u * (uint32_t)((tok0 + j) * H + h0 + hq) : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)(side + fi), 4, off,
                                                     0, 0, 0);
        }
    }
    if (nblk > 1) issue(1, smem + BUF);
    probe_wait_le(nblk > 1 ? per_block : 0);   // block 0 and the side tile landed
    __builtin_amdgcn_s_barrier();
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 2 < nblk) issue(blk + 2, smem + ((blk + 2) % 3) * BUF);
        // block blk + 1 landed; block blk + 2 may still be in flight
        probe_wait_le(blk + 2 < nblk ? per_block : 0);
        __builtin_amdgcn_s_barrier();
    }
    // per head: cs (= its dt values) and the state, the last block's x rows of
    // the head repeated N / 32 times; the wavefronts of a head split the rows
    const int wph = (int)(4 / hpw), hh = wave / wph, part = wave % wph;
    if (hh < nh) {
        const int64_t h = h0 + hh;
        if (part == 0) {
            float* csr = a.cs + ((b * H + h) * nc + c) * Q;
            for (int j = lane; j < Q; j += 64) csr[j] = side[hh * Q + j];
        }
        const unsigned char* xt = smem + ((nblk - 1) % 3) * BUF + BB + hh * XB;
        unsigned char* sg = a.states + ((b * nc + c) * H + h) * P * N * 2;
        const int pieces = (int)(P * N * 2 / 16), xp = XB / 16;
        for (int k = part * 64 + lane; k < pieces; k += wph * 64)
            *reinterpret_cast<uint4*>(sg + 16 * (int64_t)k) = *reinterpret_cast<const uint4*>(xt + 16 * (k % xp));
    }
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 256 threads (4 waves), each wave issuing
// iters * 4 MFMAs; out holds blocks * 256 floats. Total flop =
// blocks * 4 * iters * 4 * 32768. Returns a hipError_t value (0 = success).
int ssd_peak_mfma_bf16(int64_t blocks, int64_t iters, float* out, hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, out);
    return (int)hipGetLastError();
}

// Copies n 16-byte vectors from x to y (both 16-byte aligned device buffers
// of at least 16 * n bytes) with `blocks` workgroups of 256 threads.
int ssd_peak_stream(const void* x, void* y, int64_t n, int64_t blocks, hipStream_t stream) {
    if (n <= 0 || blocks <= 0 || !x || !y) return (int)hipErrorInvalidValue;
    if (((uintptr_t)x | (uintptr_t)y) & 15) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const pk_u32x4*>(x), static_cast<pk_u32x4*>(y), n);
    return (int)hipGetLastError();
}

// Copies n 16-byte vectors from x to y (both 16-byte aligned device buffers
// of at least 16 * n bytes), one 4 KB piece per workgroup; n / 256 rounded up
// must fit a grid dimension.
int ssd_peak_stream_pieces(const void* x, void* y, int64_t n, hipStream_t stream) {
    if (n <= 0 || !x || !y) return (int)hipErrorInvalidValue;
    if (((uintptr_t)x | (uintptr_t)y) & 15) return (int)hipErrorInvalidValue;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_piece_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const pk_u32x4*>(x), static_cast<pk_u32x4*>(y), n);
    return (int)hipGetLastError();
}

// The chunk scan's traffic at one problem shape (bf16 x, B, C, states and y;
// fp32 dt and cs; every dimension as the chunk scan takes it; T a multiple of
// Q, Q <= 256, Q N <= 32768, whole 64-lane groups of 16-byte pieces in the x
// tile (Q P / 512) and the state (P N / 512), 4 Q P + 4 P N + 4096 bytes of
// LDS at most 160 KiB), with `hpw` heads per workgroup and `sink` holding one float per
// workgroup. nt != 0: the x and state copies take the non-temporal policy.
// y receives x. Returns a hipError_t value, or -1 for a shape it does not
// cover.
int ssd_peak_scan_traffic(const void* x, const void* B, const void* C, const void* states, const float* dt,
                          const float* cs, void* y, float* sink, int64_t batch, int64_t T, int64_t H, int64_t P,
                          int64_t N, int64_t G, int64_t Q, int64_t hpw, int64_t nt, hipStream_t stream) {
    if (!x || !B || !C || !states || !dt || !cs || !y || !sink) return (int)hipErrorInvalidValue;
    if (batch <= 0 || T <= 0 || Q <= 0 || Q > 256 || T % Q != 0 || G <= 0 || H % G != 0 || P % 8 != 0 ||
        N % 8 != 0 || hpw <= 0)
        return -1;
    const int64_t lds = 2 * Q * P * 2 + 2 * P * N * 2 + 4096;
    if (lds > 160 * 1024 || (Q * P * 2 / 16) % 64 != 0 || (P * N * 2 / 16) % 64 != 0 || Q * N > 32768) return -1;
    ScanTraffic a{static_cast<const unsigned char*>(x), static_cast<const unsigned char*>(B),
                  static_cast<const unsigned char*>(C), static_cast<const unsigned char*>(states), dt, cs,
                  static_cast<unsigned char*>(y), sink, T, H, P, N, G, Q, T / Q, hpw, nt != 0};
    const int64_t nhb = (H / G + hpw - 1) / hpw;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(scan_traffic_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(scan_traffic_kernel, dim3((unsigned)(a.nc * G * nhb), (unsigned)batch), dim3(512), (unsigned)lds,
                       stream, a);
    return (int)hipGetLastError();
}

// The chunk state's traffic at one problem shape (bf16 x, B and states; fp32
// dt and cs; every dimension as the chunk state takes it; T a multiple of Q,
// Q a multiple of 32 and at most 256, P and N multiples of 64, hpw 1, 2 or 4
// heads per workgroup), as the chunk state's launch: (T/Q) G ceil(H/G/hpw) x
// batch workgroups of 4 wavefronts. cs receives dt ([b][H][T/Q][Q] from
// [b][T][H]); the state of (b, chunk, head), [P][N], receives the head's x
// rows of the chunk's last 32 tokens ([32][P]) repeated N / 32 times. nt != 0:
// the x copies take the non-temporal policy. Returns a hipError_t value, or
// -1 for a shape it does not cover.
int ssd_peak_state_traffic(const void* x, const void* B, const float* dt, float* cs, void* states, int64_t batch,
                           int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q, int64_t hpw, int64_t nt,
                           hipStream_t stream) {
    if (!x || !B || !dt || !cs || !states) return (int)hipErrorInvalidValue;
    if (batch <= 0 || T <= 0 || Q <= 0 || Q > 256 || Q % 32 != 0 || T % Q != 0 || G <= 0 || H % G != 0 ||
        P % 64 != 0 || N % 64 != 0 || !(hpw == 1 || hpw == 2 || hpw == 4))
        return -1;
    const int64_t per_block = 32 * N * 2 / 4096 + hpw * (32 * P * 2 / 4096);
    // the side tile takes whole 256-value rounds of the dt copies: hpw * 1024 bytes
    const int64_t lds = 3 * (32 * N * 2 + hpw * 32 * P * 2) + hpw * 1024;
    if (lds > 160 * 1024 || per_block > 8) return -1;
    StateTraffic a{static_cast<const unsigned char*>(x), static_cast<const unsigned char*>(B), dt, cs,
                   static_cast<unsigned char*>(states), T, H, P, N, G, Q, T / Q, hpw, nt != 0};
    const int64_t nhb = (H / G + hpw - 1) / hpw;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(state_traffic_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(state_traffic_kernel, dim3((unsigned)(a.nc * G * nhb), (unsigned)batch), dim3(256),
                       (unsigned)lds, stream, a);
    return (int)hipGetLastError();
}

}  // extern "C"
