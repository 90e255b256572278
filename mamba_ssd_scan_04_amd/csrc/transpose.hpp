// Token-major to k-major staging: matrix-core operands want 8 consecutive
// elements of the contraction index per lane, but x and B are stored with the
// token index outermost. A thread reads an 8 (token) x 8 (column) block as 8
// row segments (16 B for bf16, 32 B for fp32; adjacent threads read adjacent
// segments of the same token row, so a wavefront reads whole 128-byte rows),
// optionally scales each token row in fp32, and writes the block transposed
// into LDS as 8 column runs of 8 tokens.
#pragma once

#include "ssd_common.hpp"

namespace ssd {

template <typename T>
__device__ __forceinline__ void load_row8(float (&v)[8], const T* src, bool ok) {
    if (ok) {
        const typename Vec8<T>::type r = load8(src);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = to_f32(r[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
}

// dst points at LDS element [col0][tok0]; ld is the LDS row length in elements.
// v[r][e] is token r, column e.
template <typename T>
__device__ __forceinline__ void store_transposed8(T* dst, int ld, const float (&v)[8][8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        typename Vec8<T>::type o;
#pragma unroll
        for (int r = 0; r < 8; ++r) o[r] = from_f32<T>(v[r][e]);
        store8(dst + e * ld, o);
    }
}

}  // namespace ssd
