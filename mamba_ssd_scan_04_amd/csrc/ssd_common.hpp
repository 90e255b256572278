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

namespace ssd {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

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
    void* y;
    float* final_state;
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

// Inclusive prefix sum of v over the 64 lanes of a wavefront (Hillis-Steele).
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float n = __shfl_up(v, off, 64);
        if (lane >= off) v += n;
    }
    return v;
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
