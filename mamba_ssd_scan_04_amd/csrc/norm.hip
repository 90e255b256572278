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
// One pass over HBM per tensor: a wavefront takes one (token, group) and its
// channels in 16-byte pieces, lane l pieces l, l + 64, ... When a group has
// at most MAXP pieces per lane the pieces are all loaded at once into
// registers, the sum of squares reduced across lanes in a fixed order, and
// the scaled values stored from the registers; larger groups read their
// pieces twice (the second time from cache). out may be y itself: every
// element is read by the lane that writes it, before it writes it.
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

// A global load / store of one vector, NT: with the non-temporal policy (the
// line is not kept in the caches), for passes whose data exceeds the
// last-level cache.
template <bool NT, typename V>
__device__ __forceinline__ V gload(const V* p) {
    const __attribute__((address_space(1))) V* q = (const __attribute__((address_space(1))) V*)p;
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}
template <bool NT, typename V>
__device__ __forceinline__ void gstore(V* p, const V& v) {
    __attribute__((address_space(1))) V* q = (__attribute__((address_space(1))) V*)p;
    if constexpr (NT) __builtin_nontemporal_store(v, q);
    else *q = v;
}

// y * silu(z) of one 16-byte piece (y alone without the gate), in fp32
template <typename T, bool GATE>
__device__ __forceinline__ void gate8(const typename Vec8<T>::type& ry, const typename Vec8<T>::type& rz, float (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        v[k] = to_f32(ry[k]);
        if constexpr (GATE) {
            const float zk = to_f32(rz[k]);
            v[k] = v[k] * (zk / (1.0f + expf(-zk)));
        }
    }
}

// Groups of at most 64 MAXP pieces: every piece read once, all of a lane's
// loads issued before any is used. NT: y, z and out with the non-temporal
// policy.
template <typename T, bool GATE, int MAXP, bool NT>
__global__ __launch_bounds__(64 * kNormWaves) void ssd_gated_rmsnorm_reg_kernel(const T* y, const T* __restrict__ z,
                                                                                const float* __restrict__ w, float eps,
                                                                                int64_t rows, int64_t groups,
                                                                                int64_t cg, T* out) {
    using V8 = typename Vec8<T>::type;
    const int64_t item = (int64_t)blockIdx.x * kNormWaves + (threadIdx.x >> 6);
    if (item >= rows) return;   // uniform per wavefront
    const int lane = threadIdx.x & 63;
    const int64_t base = item * cg;
    const float* wg = w + (item % groups) * cg;
    const int np = (int)((cg / 8 + 63) / 64);   // pieces per lane, at most MAXP
    V8 ry[MAXP], rz[GATE ? MAXP : 1];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        if (j < np) {
            // lanes past the group's end load its last piece and add nothing
            const int64_t c = min<int64_t>((int64_t)(lane + 64 * j) * 8, cg - 8);
            ry[j] = gload<NT>(reinterpret_cast<const V8*>(y + base + c));
            if constexpr (GATE) rz[j] = gload<NT>(reinterpret_cast<const V8*>(z + base + c));
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        if (j < np && (int64_t)(lane + 64 * j) * 8 < cg) {
            float v[8];
            gate8<T, GATE>(ry[j], rz[GATE ? j : 0], v);
#pragma unroll
            for (int k = 0; k < 8; ++k) ss += v[k] * v[k];
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / (float)cg + eps);
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        const int64_t c = (int64_t)(lane + 64 * j) * 8;
        if (j < np && c < cg) {
            float v[8];
            gate8<T, GATE>(ry[j], rz[GATE ? j : 0], v);
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(wg + c);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(wg + c + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[k] = v[k] * r * w0[k];
                v[4 + k] = v[4 + k] * r * w1[k];
            }
            V8 o;
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = from_f32<T>(v[k]);
            gstore<NT>(reinterpret_cast<V8*>(out + base + c), o);
        }
    }
}

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

template <typename T, int MAXP, bool NT>
static void launch_norm_reg(dim3 grid, const void* y, const void* z, const float* w, float eps, int64_t rows,
                            int64_t groups, int64_t cg, void* out, hipStream_t s) {
    if (z)
        hipLaunchKernelGGL((ssd_gated_rmsnorm_reg_kernel<T, true, MAXP, NT>), grid, dim3(64 * kNormWaves), 0, s,
                           static_cast<const T*>(y), static_cast<const T*>(z), w, eps, rows, groups, cg,
                           static_cast<T*>(out));
    else
        hipLaunchKernelGGL((ssd_gated_rmsnorm_reg_kernel<T, false, MAXP, NT>), grid, dim3(64 * kNormWaves), 0, s,
                           static_cast<const T*>(y), static_cast<const T*>(nullptr), w, eps, rows, groups, cg,
                           static_cast<T*>(out));
}

// The last-level cache of an MI355X (AMD Infinity Cache) holds 256 MiB: a
// pass over more data than that streams it with the non-temporal policy.
constexpr double kNormCacheBytes = 256.0 * 1024 * 1024;

template <typename T>
static hipError_t launch_norm_t(const void* y, const void* z, const float* w, float eps, int64_t rows, int64_t groups,
                                int64_t cg, void* out, hipStream_t s) {
    dim3 grid((unsigned)((rows + kNormWaves - 1) / kNormWaves));
    // register-resident up to 16 (bf16) or 8 (fp32) pieces per lane, in the
    // smallest instantiation that holds the group
    const int64_t np = (cg / 8 + 63) / 64;
    const bool nt = (double)(z ? 3 : 2) * (double)rows * (double)cg * (double)sizeof(T) > kNormCacheBytes;
#define SSD_NORM_REG(MAXP_)                                                                      \
    if (np <= MAXP_) {                                                                           \
        if (nt)                                                                                  \
            launch_norm_reg<T, MAXP_, true>(grid, y, z, w, eps, rows, groups, cg, out, s);       \
        else                                                                                     \
            launch_norm_reg<T, MAXP_, false>(grid, y, z, w, eps, rows, groups, cg, out, s);      \
        return hipGetLastError();                                                                \
    }
    SSD_NORM_REG(4)
    SSD_NORM_REG(8)
    if constexpr (sizeof(T) == 2) {
        SSD_NORM_REG(12)
        SSD_NORM_REG(16)
    }
#undef SSD_NORM_REG
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
