// ssd_gated_rmsnorm: the normalisation after the gate in the Mamba-2 block.
//
// "Transformers are SSMs" (chapterpal summary), Knowl 6: the SSD output Y is
// gated by SiLU(z) and then normalised (a group norm or an RMS norm) before the
// output projection; Knowl 8 takes the norm in groups whose count divides the
// tensor-parallel degree. Per token, the H*P channels of y are cut into
// `groups` equal contiguous groups and each is divided by its root mean
// square:
//
//   g = y * silu(z)   (y itself without z),   out = g / sqrt(mean(g^2) + eps) * w
//
// One pass over HBM per tensor: a wavefront takes one (token, group), reads
// its channels in 16-byte pieces (the sum of squares), reduces across lanes in
// a fixed order, and reads them again (from cache) to scale and store. out
// may be y itself: every element is read by the lane that writes it, before
// it writes it.
#include "kernels.hpp"

namespace ssd {

template <typename T> struct Pk8;
template <> struct Pk8<bf16> {
    static __device__ __forceinline__ void load(const bf16* p, float (&v)[8]) {
        const bf16x8 r = ldg8(p);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = to_f32(r[k]);
    }
    static __device__ __forceinline__ void store(bf16* p, const float (&v)[8]) {
        bf16x8 r;
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] = from_f32<bf16>(v[k]);
        stg(reinterpret_cast<bf16x8*>(p), r);
    }
};
template <> struct Pk8<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
        const f32x8 r = ldg8(p);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = r[k];
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
        f32x4 lo, hi;
        lo[0] = v[0]; lo[1] = v[1]; lo[2] = v[2]; lo[3] = v[3];
        hi[0] = v[4]; hi[1] = v[5]; hi[2] = v[6]; hi[3] = v[7];
        stg(reinterpret_cast<f32x4*>(p), lo);
        stg(reinterpret_cast<f32x4*>(p + 4), hi);
    }
};

constexpr int kNormWaves = 4;

template <typename T, bool GATE>
__global__ __launch_bounds__(64 * kNormWaves) void ssd_gated_rmsnorm_kernel(const T* y, const T* __restrict__ z,
                                                                            const float* __restrict__ w, float eps,
                                                                            int64_t rows, int64_t groups, int64_t cg,
                                                                            T* out) {
    const int64_t item = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    if (item >= rows) return;   // uniform per wavefront
    const int lane = threadIdx.x & 63;
    const int64_t base = item * cg;                 // the group's first element ([b,T,H*P], groups contiguous)
    const float* wg = w + (item % groups) * cg;
    auto gated = [&](int64_t c, float (&v)[8]) {
        Pk8<T>::load(y + base + c, v);
        if constexpr (GATE) {
            float zv[8];
            Pk8<T>::load(z + base + c, zv);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = v[k] * (zv[k] / (1.0f + expf(-zv[k])));
        }
    };
    float ss = 0.0f;
    for (int64_t c = (int64_t)lane * 8; c < cg; c += 64 * 8) {
        float v[8];
        gated(c, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += v[k] * v[k];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / (float)cg + eps);
    for (int64_t c = (int64_t)lane * 8; c < cg; c += 64 * 8) {
        float v[8];
        gated(c, v);
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wg + c);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wg + c + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = v[k] * r * w0[k];
            v[4 + k] = v[4 + k] * r * w1[k];
        }
        Pk8<T>::store(out + base + c, v);
    }
}

template <typename T>
static hipError_t launch_norm_t(const void* y, const void* z, const float* w, float eps, int64_t rows, int64_t groups,
                                int64_t cg, void* out, hipStream_t s) {
    dim3 grid((unsigned)((rows + kNormWaves - 1) / kNormWaves));
    if (z)
        hipLaunchKernelGGL((ssd_gated_rmsnorm_kernel<T, true>), grid, dim3(64 * kNormWaves), 0, s,
                           static_cast<const T*>(y), static_cast<const T*>(z), w, eps, rows, groups, cg,
                           static_cast<T*>(out));
    else
        hipLaunchKernelGGL((ssd_gated_rmsnorm_kernel<T, false>), grid, dim3(64 * kNormWaves), 0, s,
                           static_cast<const T*>(y), static_cast<const T*>(nullptr), w, eps, rows, groups, cg,
                           static_cast<T*>(out));
    return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const void* y, const void* z, const float* w, float eps, int64_t rows, int64_t groups,
                                int64_t cg, void* out, int dtype, hipStream_t s) {
    return dtype == 1 ? launch_norm_t<bf16>(y, z, w, eps, rows, groups, cg, out, s)
                      : launch_norm_t<float>(y, z, w, eps, rows, groups, cg, out, s);
}

}  // namespace ssd
