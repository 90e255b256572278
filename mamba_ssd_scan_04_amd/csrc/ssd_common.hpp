// Device-side building blocks shared by the four SSD kernels (gfx950 / CDNA4).
//
// Matrix core tiles are 32x32 with fp32 accumulation. A "k16 step" adds a
// 32x32x16 product: every lane supplies 8 consecutive-k elements of A (row
// lane%32) and 8 of B (column lane%32); lane half hf = lane/32 covers
// k = 8*hf .. 8*hf+7. For bf16 that is one v_mfma_f32_32x32x16_bf16; for fp32
// it is eight v_mfma_f32_32x32x2f32, instruction e taking k = e (half 0) and
// k = 8 + e (half 1), so both element types share one register layout.
// Accumulator element r (0..15) of a lane sits at row 8*(r/4) + 4*hf + r%4,
// column lane%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ssd {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;

struct Params {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk, nchunks;
    int64_t heads_per_group;
    const void* x;
    const float* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    float* cs;
    void* states;
    int fuse_cs;        // chunk_state also computes (and writes) cs from dt and A
    void* y;
    float* final_state;
    const float* init_state;   // state before the first token [b,H,N,P]; nullptr: zero
    int read_h0;               // chunk_scan applies states[., 0] (h_0) to the first chunk too
    const void* z;             // gate input [b,T,H,P] (x's type): y *= silu(z); nullptr: no gate
    const int* seq_idx;        // document ids [b,T], non-decreasing along T: the state is reset where
                               // the id changes; nullptr: one sequence per batch row
    int stream_x;              // copy x (chunk state, chunk scan) and the carried states (chunk
                               // scan) to LDS with the non-temporal policy: set when the data of a
                               // forward cannot stay in the last-level cache
};

// ---- element traits --------------------------------------------------------

template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// 8 consecutive elements from global or LDS memory (16-byte aligned for bf16,
// 32-byte aligned for fp32).
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load8(const float* p) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    f32x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    return v;
}
__device__ __forceinline__ void store8(bf16* p, const bf16x8& v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ void store8(float* p, const f32x8& v) {
    f32x4 lo, hi;
    lo[0] = v[0]; lo[1] = v[1]; lo[2] = v[2]; lo[3] = v[3];
    hi[0] = v[4]; hi[1] = v[5]; hi[2] = v[6]; hi[3] = v[7];
    *reinterpret_cast<f32x4*>(p) = lo;
    *reinterpret_cast<f32x4*>(p + 4) = hi;
}

template <typename T> __device__ __forceinline__ typename Vec8<T>::type zero8() {
    typename Vec8<T>::type v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(0.0f);
    return v;
}

// ---- matrix core -----------------------------------------------------------

__device__ __forceinline__ void mma_k16(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_k16(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 v;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = 0.0f;
    return v;
}

// ---- wavefront prefix sum --------------------------------------------------

// Inclusive prefix sum of v over the 64 lanes of a wavefront with DPP: a
// Hillis-Steele scan inside each 16-lane row (row_shr 1, 2, 4, 8; lanes
// shifted in from outside the row add 0), then row 0's total is added to row
// 1 and row 2's to row 3 (row_bcast:15), then the total of rows 0-1 to rows 2
// and 3 (row_bcast:31).
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, BOUND));
}
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
    (void)lane;
    v += dpp_f32<0x111, 0xF, true>(v);    // row_shr:1
    v += dpp_f32<0x112, 0xF, true>(v);    // row_shr:2
    v += dpp_f32<0x114, 0xF, true>(v);    // row_shr:4
    v += dpp_f32<0x118, 0xF, true>(v);    // row_shr:8
    v += dpp_f32<0x142, 0xA, false>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f32<0x143, 0xC, false>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// In-chunk inclusive prefix sum over one wavefront (the parallel scan of
// "Transformers are SSMs", appendix B.2.2): lane l holds the `per` consecutive
// values l*per .. l*per+per-1 in v[0..per) (per <= 4, lanes >= active hold
// nothing); each lane sums its values serially, a wavefront scan of the lane
// totals gives the offsets. Positions at or past qc then take the exact value
// at qc - 1, so a short last chunk repeats its final value.
__device__ __forceinline__ void chunk_prefix(float (&v)[4], int per, int active, int qc, int lane) {
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (k < per && lane < active) run += v[k];
        v[k] = run;
    }
    const float incl = wave_inclusive_scan(run, lane);
    const float base = incl - run;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] += base;
    const int qa = qc < per * active ? qc : per * active;
    if (qa < per * active) {
        const int src = (qa - 1) / per, ks = (qa - 1) % per;
        float mine = v[0];
#pragma unroll
        for (int k = 1; k < 4; ++k)
            if (k == ks) mine = v[k];
        const float lastv = __shfl(mine, src, 64);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (lane * per + k >= qa) v[k] = lastv;
    }
}

// Position of token i_local (0..15) of a 16-token group in the "fragment
// order" used for the x^T tile of the chunk scan: the middle two quads are
// swapped so that an MFMA accumulator's rows (8*g + 4*hf + r) can feed the
// next MFMA's k operand without moving data between lanes.
__device__ __forceinline__ int frag_token(int q) {
    // q = 8*hf + e  ->  token 8*(e/4) + 4*hf + e%4
    const int hf = q >> 3, e = q & 7;
    return ((e >> 2) << 3) + (hf << 2) + (e & 3);
}

}  // namespace ssd

// ---- LDS tiles ---------------------------------------------------------------
//
// Row-major tiles in LDS are addressed in 16-byte chunks with an XOR swizzle
// of the chunk index by the row, so that the two access patterns the kernels
// use are (nearly) free of bank conflicts:
//  (a) transpose reads: 4 consecutive rows x 64 contiguous bytes per half wave;
//  (b) row reads: 32 consecutive rows, the same 16-byte chunk of each.
// RC is the number of 16-byte chunks per row (a power of two >= 4).
namespace ssd {

template <int RC>
__device__ __forceinline__ int swz(int r) {
    if constexpr (RC >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (RC == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
}

// byte offset of (row r, byte b within the row) in a swizzled tile
template <int RC>
__device__ __forceinline__ int tile_byte(int r, int b) {
    return r * RC * 16 + (((b >> 4) ^ swz<RC>(r)) << 4) + (b & 15);
}

// Buffer resource (V#) for raw byte-addressed loads from a wave-uniform base:
// no stride, 32-bit data format, offsets up to 2^31 - 1.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// One 16-byte global -> LDS copy per lane, straight into LDS (no registers):
// lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16) from rs + voff. The
// buffer form (not the global one) lets the compiler keep exact counts of
// the LDS reads in flight around it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, unsigned char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
// The same copy with the cache policy picked at run time (nt uniform across
// the wavefront): nt = non-temporal (the line is not kept in the caches on
// the way), for data read once whose footprint exceeds the caches.
__device__ __forceinline__ void dma16p(__amdgpu_buffer_rsrc_t rs, uint32_t voff, unsigned char* lds, bool nt) {
    if (nt)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 2);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Asynchronous global -> LDS copy of a rows x RC-chunk tile. Every lane of a
// wavefront copies one 16-byte chunk per instruction; instruction k of the
// tile writes LDS bytes [1024 k, 1024 k + 1024). The source of physical chunk
// (r, pc) is logical chunk c = pc ^ swz(r) of row r: gbase + r * row_stride +
// 16 c, with r clamped to valid_rows - 1 and c to valid_chunks - 1 (rows or
// columns past the data are filled with copies of real data: the kernels only
// ever give them zero weight or leave their outputs unstored). gbase is
// uniform; offsets are 32-bit.
template <int RC>
__device__ __forceinline__ void dma_tile(unsigned char* lds, int rows, int valid_rows, int valid_chunks,
                                         const unsigned char* gbase, uint32_t row_stride, int wave,
                                         int nwaves, int lane, bool nt = false) {
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(gbase);
    const int total = rows * RC;   // a multiple of 64
    for (int k = wave; k * 64 < total; k += nwaves) {
        const int P = k * 64 + lane;
        const int r = P / RC;
        int c = (P % RC) ^ swz<RC>(r);
        c = c < valid_chunks ? c : valid_chunks - 1;
        const int rr = r < valid_rows ? r : valid_rows - 1;
        dma16p(rs, (uint32_t)rr * row_stride + 16u * (uint32_t)c, lds + k * 1024, nt);
    }
}

// The same copies as dma_tile, planned once: lane offsets of the at most NI
// instructions a wavefront issues (instruction i is tile instruction
// wave + nwaves * i; -1 = none), then issued for any source base.
template <int RC, int NI>
__device__ __forceinline__ void dma_tile_plan(int (&off)[NI], int rows, int valid_rows, int valid_chunks,
                                              uint32_t row_stride, int wave, int nwaves, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k = wave + nwaves * i;
        if (k * 64 < rows * RC) {
            const int P = k * 64 + lane;
            const int r = P / RC;
            int c = (P % RC) ^ swz<RC>(r);
            c = c < valid_chunks ? c : valid_chunks - 1;
            const int rr = r < valid_rows ? r : valid_rows - 1;
            off[i] = (int)((uint32_t)rr * row_stride + 16u * (uint32_t)c);
        } else {
            off[i] = -1;
        }
    }
}
// NT: the non-temporal policy (see dma16p).
template <int NI, bool NT = false>
__device__ __forceinline__ void dma_tile_issue(unsigned char* lds, const unsigned char* gbase, const int (&off)[NI],
                                               int wave, int nwaves) {
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(gbase);
#pragma unroll
    for (int i = 0; i < NI; ++i)
        if (off[i] >= 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + (wave + nwaves * i) * 1024),
                                                     16, (uint32_t)off[i], 0, 0, NT ? 2 : 0);
}

// Loads through explicit global-address-space pointers (not flat).
__device__ __forceinline__ bf16x8 ldg8(const bf16* p) {
    return *(const __attribute__((address_space(1))) bf16x8*)p;
}
__device__ __forceinline__ f32x8 ldg8(const float* p) {
    const f32x4 lo = *(const __attribute__((address_space(1))) f32x4*)p;
    const f32x4 hi = *(const __attribute__((address_space(1))) f32x4*)(p + 4);
    f32x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    return v;
}
__device__ __forceinline__ float ldg(const float* p) { return *(const __attribute__((address_space(1))) float*)p; }
template <typename T> __device__ __forceinline__ void stg(T* p, T v) { *(__attribute__((address_space(1))) T*)p = v; }

// Wait until this wavefront's outstanding vector memory operations (including
// the LDS copies above) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef __attribute__((ext_vector_type(4))) short s16x4;

// 8 k-elements of a matrix-core operand from a row-major swizzled LDS tile
// whose rows are the k index: lane (l32, hf) receives rows rowk(hf, e),
// e = 0..7, of column col0 + l32. bf16 uses two ds_read_b64_tr_b16: within a
// group of 16 lanes, result lane i slot s is element i%4 of the 8 bytes at the
// address of lane 4s + i/4, so lane 16q + 4s + j points at row rowk(hf, s)
// (s + 4 for the second read), columns col0 + 16(q%2) + 4j .. +3.
template <int RC, typename RowK>
__device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int col0, RowK rowk, int lane) {
    const int q = lane >> 4, s = (lane >> 2) & 3, j = lane & 3, hf = lane >> 5;
    const int cb = (col0 + 16 * (q & 1) + 4 * j) * 2;   // byte within the row
    const unsigned char* base = reinterpret_cast<const unsigned char*>(tile);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    lds_s16x4* pa = (lds_s16x4*)(base + tile_byte<RC>(rowk(hf, s), cb));
    lds_s16x4* pb = (lds_s16x4*)(base + tile_byte<RC>(rowk(hf, s + 4), cb));
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pa);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(pb);
    // whole-vector bit casts (casting single ext-vector elements miscompiles)
    const bf16x4 av = __builtin_bit_cast(bf16x4, a);
    const bf16x4 bv = __builtin_bit_cast(bf16x4, b);
    return __builtin_shufflevector(av, bv, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int RC, typename RowK>
__device__ __forceinline__ f32x8 frag_tr(const float* tile, int col0, RowK rowk, int lane) {
    const int hf = lane >> 5, l32 = lane & 31;
    const unsigned char* base = reinterpret_cast<const unsigned char*>(tile);
    f32x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        out[e] = *reinterpret_cast<const float*>(base + tile_byte<RC>(rowk(hf, e), (col0 + l32) * 4));
    return out;
}

// 8 consecutive elements (one or two 16-byte chunks) of row r starting at
// element col (a multiple of 8) from a swizzled LDS tile.
template <int RC>
__device__ __forceinline__ bf16x8 row8(const bf16* tile, int r, int col) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const unsigned char*>(tile) +
                                            tile_byte<RC>(r, col * 2));
}
template <int RC>
__device__ __forceinline__ f32x8 row8(const float* tile, int r, int col) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(tile);
    const f32x4 lo = *reinterpret_cast<const f32x4*>(base + tile_byte<RC>(r, col * 4));
    const f32x4 hi = *reinterpret_cast<const f32x4*>(base + tile_byte<RC>(r, col * 4 + 16));
    f32x8 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    return v;
}

template <typename T> __device__ __forceinline__ typename Vec8<T>::type cvt8(const bf16x8& v) {
    if constexpr (sizeof(T) == 2) return v;
    else {
        f32x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = to_f32(v[e]);
        return o;
    }
}
template <typename T> __device__ __forceinline__ typename Vec8<T>::type cvt8(const f32x8& v) {
    typename Vec8<T>::type o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = from_f32<T>(v[e]);
    return o;
}


// Two transpose reads at precomputed per-lane byte offsets (see frag_tr): the
// k rows of a fragment step by whole 16-row groups, which leaves the swizzle
// unchanged, so a fragment at row offset R is base + off + R * row_bytes.
__device__ __forceinline__ bf16x8 frag_tr_at(const unsigned char* base, int off_a, int off_b) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off_a));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off_b));
    const bf16x4 av = __builtin_bit_cast(bf16x4, a);
    const bf16x4 bv = __builtin_bit_cast(bf16x4, b);
    return __builtin_shufflevector(av, bv, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane byte offsets of the two transpose reads of frag_tr for rows
// rowk(hf, e) (evaluated at the first 16-row group) and column tile col0.
template <int RC, typename RowK>
__device__ __forceinline__ void frag_tr_offsets(int col0, RowK rowk, int lane, int& off_a, int& off_b) {
    const int q = lane >> 4, s = (lane >> 2) & 3, j = lane & 3, hf = lane >> 5;
    const int cb = (col0 + 16 * (q & 1) + 4 * j) * 2;
    off_a = tile_byte<RC>(rowk(hf, s), cb);
    off_b = tile_byte<RC>(rowk(hf, s + 4), cb);
}

// Wait until at most N of this wavefront's vector memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for pipelines of global -> LDS copies. __syncthreads()
// makes this wavefront's LDS writes visible with a release fence, and a copy
// into LDS still in flight counts as such a write, so it waits for every
// outstanding copy (vmcnt(0)) and no copy ever stays in flight across it.
// Here the caller first waits for the copies the other wavefronts will read
// (wait_vmem_le); the barrier completes this wavefront's LDS reads and writes
// (lgkmcnt(0)) and the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most n (runtime, wave-uniform) vector memory operations of
// this wavefront are outstanding; n above the counter's range (63) waits for
// at most 63, i.e. for more than asked.
__device__ __forceinline__ void wait_vmem_le_rt(int n) {
    switch (n) {
#define SSD_WAIT_CASE(K) case K: wait_vmem_le<K>(); break;
#define SSD_WAIT_8(K) SSD_WAIT_CASE(K) SSD_WAIT_CASE(K + 1) SSD_WAIT_CASE(K + 2) SSD_WAIT_CASE(K + 3) \
    SSD_WAIT_CASE(K + 4) SSD_WAIT_CASE(K + 5) SSD_WAIT_CASE(K + 6) SSD_WAIT_CASE(K + 7)
        SSD_WAIT_8(0) SSD_WAIT_8(8) SSD_WAIT_8(16) SSD_WAIT_8(24)
        SSD_WAIT_8(32) SSD_WAIT_8(40) SSD_WAIT_8(48) SSD_WAIT_8(56)
#undef SSD_WAIT_8
#undef SSD_WAIT_CASE
        default: wait_vmem_le<63>(); break;
    }
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each with
// its own L2. Remap the linear id so that a contiguous range of logical
// indices runs on one XCD: neighbouring logical blocks (same chunk, other
// heads) then share B and C through the same L2.
__device__ __forceinline__ int xcd_logical_block() {
    const int total = (int)(gridDim.x * gridDim.y);
    const int id = (int)(blockIdx.x + gridDim.x * blockIdx.y);
    return (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
}

// 2^x on the hardware transcendental unit (v_exp_f32): results below the
// smallest normal flush to 0, 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane n of this lane's 16-lane row (DPP row_newbcast); folded by
// the compiler into the consuming VALU instruction as a DPP source operand.
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
    static_assert(N >= 0 && N < 16, "row lane");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
}  // namespace ssd
