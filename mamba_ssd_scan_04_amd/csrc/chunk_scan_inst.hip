// One (input type, state type, variant) of the chunk-scan kernel; the build
// compiles this file once per combination with SSD_SC_X (bf16 | f32),
// SSD_SC_S (bf16 | f32) and SSD_SC_V (0 plain, 1 gated, 2 packed documents, 3 gated
// packed documents).
#include "chunk_scan_impl.hpp"

#if !defined(SSD_SC_X) || !defined(SSD_SC_S) || !defined(SSD_SC_V)
#error "chunk_scan_inst.hip is built with -DSSD_SC_X=.. -DSSD_SC_S=.. -DSSD_SC_V=.."
#endif

namespace ssd {
typedef float f32;

#define SSD_SC_NAME2(X, S, V) launch_chunk_scan_##X##_##S##_##V
#define SSD_SC_NAME(X, S, V) SSD_SC_NAME2(X, S, V)

hipError_t SSD_SC_NAME(SSD_SC_X, SSD_SC_S, SSD_SC_V)(const Params& p, hipStream_t s) {
    return dispatch_sc<SSD_SC_X, SSD_SC_S, SSD_SC_V>(p, s);
}

}  // namespace ssd
