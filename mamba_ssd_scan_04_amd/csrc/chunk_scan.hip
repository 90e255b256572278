// ssd_chunk_scan: dispatch over the instantiations of the chunk-scan kernel
// (chunk_scan_impl.hpp). Each (input type, state type, variant) is compiled in
// a translation unit of its own (chunk_scan_inst.hip, built once per
// combination), so that the many template instantiations build in parallel.
#include "kernels.hpp"

namespace ssd {

#define SSD_SC_DECL(X, S, V) hipError_t launch_chunk_scan_##X##_##S##_##V(const Params& p, hipStream_t s);
#define SSD_SC_DECL3(X, S) SSD_SC_DECL(X, S, 0) SSD_SC_DECL(X, S, 1) SSD_SC_DECL(X, S, 2) SSD_SC_DECL(X, S, 3)
SSD_SC_DECL3(bf16, bf16)
SSD_SC_DECL3(bf16, f32)
SSD_SC_DECL3(f32, f32)
#undef SSD_SC_DECL3
#undef SSD_SC_DECL

hipError_t launch_chunk_scan(const Params& p, int dtype, int state_dtype, hipStream_t s) {
    // 0 plain, 1 gated, 2 packed documents, 3 both
    const int v = (p.z ? 1 : 0) + (p.seq_idx ? 2 : 0);
#define SSD_SC_PICK(X, S)                                         \
    return v == 1 ? launch_chunk_scan_##X##_##S##_1(p, s)         \
         : v == 2 ? launch_chunk_scan_##X##_##S##_2(p, s)         \
         : v == 3 ? launch_chunk_scan_##X##_##S##_3(p, s)         \
                  : launch_chunk_scan_##X##_##S##_0(p, s);
    if (dtype == 1 && state_dtype == 1) { SSD_SC_PICK(bf16, bf16) }
    if (dtype == 1) { SSD_SC_PICK(bf16, f32) }
    SSD_SC_PICK(f32, f32)
#undef SSD_SC_PICK
}

// Smallest LDS the chunk scan needs for (dtype, state dtype, P, N, Q): single
// x and h_c buffers; used by argument checking.
int chunk_scan_lds_bytes(int dtype, int state_dtype, int64_t P, int64_t N, int64_t Q) {
    const int esz = dtype == 1 ? 2 : 4, ssz = state_dtype == 1 ? 2 : 4;
    if (Q < 32) Q = 32;   // rows as tiled: whole 32-token tiles
    const int pp = (int)((P + 31) / 32) * 32, np = (int)((N + 31) / 32) * 32;
    return (int)Q * pp * esz + pp * np * ssz + 2 * 3 * (int)Q * 4;
}

}  // namespace ssd
