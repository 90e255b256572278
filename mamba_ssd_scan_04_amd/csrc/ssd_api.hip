// The C ABI of libssd (declared in include/ssd.h): argument checks, workspace
// layout and the launch order of the four kernels. No allocation, no state.
#include <stdint.h>

#include <atomic>

#include "ssd.h"
#include "kernels.hpp"

namespace ssd {
int chunk_scan_lds_bytes(int dtype, int state_dtype, int64_t P, int64_t N, int64_t Q);
}

namespace ssd {
int device_cus() {
    // per-device cache; threads that race on a first call store the same value
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace ssd

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxLds = 160 * 1024;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool in_list(int64_t v, const int64_t* list, int n) {
    for (int i = 0; i < n; ++i)
        if (list[i] == v) return true;
    return false;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t nchunks_of(const ssd_dims* d) { return (d->seqlen + d->chunk_size - 1) / d->chunk_size; }

size_t cs_bytes_of(const ssd_dims* d) {
    return (size_t)d->batch * d->nheads * nchunks_of(d) * d->chunk_size * sizeof(float);
}

size_t states_bytes_of(const ssd_dims* d) {
    const size_t esz = d->state_dtype == SSD_BF16 ? 2 : 4;
    return (size_t)d->batch * nchunks_of(d) * d->nheads * d->headdim * d->dstate * esz;
}

// The last-level cache of an MI355X (AMD Infinity Cache) holds 256 MiB. When
// the data of one forward (x, y, B, C, dt, cs and the inter-chunk states)
// exceeds it, x cannot stay cached between its two reads (chunk state, chunk
// scan) anyway: the copies of x, and the chunk scan's copies of the carried
// states, then take the non-temporal policy, which leaves the cache to the
// states that the next launch reads. Below the cache's size, streaming would
// give up the hits of data still cached from an earlier call.
constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;

bool stream_x_of(const ssd_dims* d) {
    const double esz = d->dtype == SSD_BF16 ? 2.0 : 4.0;
    const double bt = (double)d->batch * (double)d->seqlen;
    const double bytes = esz * bt * (2.0 * d->nheads * d->headdim + 2.0 * d->ngroups * d->dstate) +
                         8.0 * bt * d->nheads + (double)states_bytes_of(d);
    return bytes > kLastLevelCacheBytes;
}

ssd::Params make_params(const ssd_dims* d) {
    ssd::Params p{};
    p.stream_x = stream_x_of(d) ? 1 : 0;
    p.batch = d->batch;
    p.seqlen = d->seqlen;
    p.nheads = d->nheads;
    p.headdim = d->headdim;
    p.dstate = d->dstate;
    p.ngroups = d->ngroups;
    p.chunk = d->chunk_size;
    p.nchunks = nchunks_of(d);
    p.heads_per_group = d->nheads / d->ngroups;
    return p;
}

ssd_status to_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_LAUNCH; }

bool empty(const ssd_dims* d) { return d->batch == 0 || d->seqlen == 0; }

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(ssd_status s) {
    switch (s) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL_POINTER: return "a required pointer is NULL";
        case SSD_ERR_BAD_SHAPE: return "bad shape: negative or zero size, or nheads not divisible by ngroups";
        case SSD_ERR_UNSUPPORTED:
            return "unsupported configuration: headdim in {16,32,64,128}, dstate in {16,32,64,128,256}, "
                   "chunk_size in {16,32,64,128,256}, dtype fp32/bf16, bf16 states only with bf16 inputs, "
                   "the chunk scan's x and state tiles must fit in LDS (Q*P*esize + P*N*ssize <= ~156 KB), "
                   "and one chunk's rows must span less than 2^31 bytes (Q*H*P*esize, Q*G*N*esize)";
        case SSD_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
        case SSD_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than ssd_workspace_size()";
        case SSD_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case SSD_ERR_TOO_LARGE:
            return "the workspace this problem needs exceeds the library's fixed device scratch "
                   "(ssd_forward_noalloc handles up to ssd_noalloc_scratch_bytes() of workspace)";
    }
    return "unknown status";
}

ssd_status ssd_check_dims(const ssd_dims* d) {
    static const int64_t kP[] = {16, 32, 64, 128};
    static const int64_t kN[] = {16, 32, 64, 128, 256};
    static const int64_t kQ[] = {16, 32, 64, 128, 256};
    if (!d) return SSD_ERR_NULL_POINTER;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 ||
        d->ngroups <= 0 || d->chunk_size <= 0)
        return SSD_ERR_BAD_SHAPE;
    if (d->nheads % d->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (!in_list(d->headdim, kP, 4) || !in_list(d->dstate, kN, 5) || !in_list(d->chunk_size, kQ, 5))
        return SSD_ERR_UNSUPPORTED;
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (d->state_dtype != SSD_F32 && d->state_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (d->state_dtype == SSD_BF16 && d->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (ssd::chunk_scan_lds_bytes(d->dtype, d->state_dtype, d->headdim, d->dstate, d->chunk_size) > kMaxLds)
        return SSD_ERR_UNSUPPORTED;
    // grid limits: nchunks and nheads go in grid.x / grid.y, batch in grid.z
    if (nchunks_of(d) > INT32_MAX || d->nheads > 65535 || d->batch > 65535) return SSD_ERR_UNSUPPORTED;
    // the kernels address one chunk's token rows of x, y, z, B and C with
    // 32-bit offsets from the chunk's first row (buffer loads reach at most
    // 2^31 - 1 bytes): a chunk's span of those rows must stay below 2^31 bytes
    const int64_t esz = d->dtype == SSD_BF16 ? 2 : 4;
    const int64_t span_x = d->chunk_size * d->nheads * d->headdim * esz;
    const int64_t span_b = d->chunk_size * d->ngroups * d->dstate * esz;
    if (span_x >= ((int64_t)1 << 31) || span_b >= ((int64_t)1 << 31)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status ssd_stage_sizes(const ssd_dims* d, size_t* cs_bytes, size_t* states_bytes) {
    const ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (cs_bytes) *cs_bytes = cs_bytes_of(d);
    if (states_bytes) *states_bytes = states_bytes_of(d);
    return SSD_OK;
}

size_t ssd_workspace_size(const ssd_dims* d) {
    if (ssd_check_dims(d) != SSD_OK || empty(d)) return 0;
    return round_up(cs_bytes_of(d)) + round_up(states_bytes_of(d));
}

ssd_status ssd_chunk_cumsum(const ssd_dims* d, const float* dt, const float* A, float* cs,
                            hipStream_t stream) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (empty(d)) return SSD_OK;
    if (!dt || !A || !cs) return SSD_ERR_NULL_POINTER;
    if (!aligned16(dt) || !aligned16(A) || !aligned16(cs)) return SSD_ERR_MISALIGNED;
    ssd::Params p = make_params(d);
    p.dt = dt;
    p.A = A;
    p.cs = cs;
    return to_status(ssd::launch_chunk_cumsum(p, stream));
}

ssd_status ssd_chunk_state(const ssd_dims* d, const void* x, const float* dt, const void* B,
                           const float* cs, void* states, hipStream_t stream) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (empty(d)) return SSD_OK;
    if (!x || !dt || !B || !cs || !states) return SSD_ERR_NULL_POINTER;
    if (!aligned16(x) || !aligned16(dt) || !aligned16(B) || !aligned16(cs) || !aligned16(states))
        return SSD_ERR_MISALIGNED;
    ssd::Params p = make_params(d);
    p.x = x;
    p.dt = dt;
    p.B = B;
    p.cs = const_cast<float*>(cs);
    p.states = states;
    return to_status(ssd::launch_chunk_state(p, d->dtype, d->state_dtype, stream));
}

ssd_status ssd_chunk_cumsum_state(const ssd_dims* d, const void* x, const float* dt, const float* A,
                                  const void* B, float* cs, void* states, hipStream_t stream) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (empty(d)) return SSD_OK;
    if (!x || !dt || !A || !B || !cs || !states) return SSD_ERR_NULL_POINTER;
    if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(cs) || !aligned16(states))
        return SSD_ERR_MISALIGNED;
    ssd::Params p = make_params(d);
    p.x = x;
    p.dt = dt;
    p.A = A;
    p.B = B;
    p.cs = cs;
    p.states = states;
    p.fuse_cs = 1;
    return to_status(ssd::launch_chunk_state(p, d->dtype, d->state_dtype, stream));
}

}  // extern "C"

namespace {

ssd_status state_passing_impl(const ssd_dims* d, const float* cs, void* states, const float* init,
                              float* final_state, hipStream_t stream, const int* seq = nullptr) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (!final_state) return SSD_ERR_NULL_POINTER;
    if (!aligned16(final_state) || (init && !aligned16(init))) return SSD_ERR_MISALIGNED;
    ssd::Params p = make_params(d);
    p.final_state = final_state;
    p.init_state = init;
    if (d->batch == 0) return SSD_OK;
    const int64_t nstate = d->batch * d->nheads * d->dstate * d->headdim;
    if (d->seqlen == 0)
        return init ? to_status(hipMemcpyAsync(final_state, init, (size_t)nstate * sizeof(float),
                                               hipMemcpyDeviceToDevice, stream))
                    : to_status(ssd::launch_zero_fill(final_state, nstate, stream));
    if (!cs || !states) return SSD_ERR_NULL_POINTER;
    if (!aligned16(cs) || !aligned16(states)) return SSD_ERR_MISALIGNED;
    p.cs = const_cast<float*>(cs);
    p.states = states;
    p.seq_idx = seq;
    return to_status(ssd::launch_state_passing(p, d->state_dtype, stream));
}

ssd_status chunk_scan_impl(const ssd_dims* d, const void* x, const float* dt, const void* B, const void* C,
                           const float* D, const float* cs, const void* states, int read_h0, const void* z,
                           void* y, hipStream_t stream, const int* seq = nullptr) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (empty(d)) return SSD_OK;
    if (!x || !dt || !B || !C || !D || !cs || !states || !y) return SSD_ERR_NULL_POINTER;
    if (!aligned16(x) || !aligned16(dt) || !aligned16(B) || !aligned16(C) || !aligned16(D) ||
        !aligned16(cs) || !aligned16(states) || !aligned16(y))
        return SSD_ERR_MISALIGNED;
    ssd::Params p = make_params(d);
    p.x = x;
    p.dt = dt;
    p.B = B;
    p.C = C;
    p.D = D;
    p.cs = const_cast<float*>(cs);
    p.states = const_cast<void*>(states);
    p.y = y;
    p.read_h0 = read_h0;
    if (z && !aligned16(z)) return SSD_ERR_MISALIGNED;
    p.z = z;
    p.seq_idx = seq;
    return to_status(ssd::launch_chunk_scan(p, d->dtype, d->state_dtype, stream));
}

ssd_status forward_impl(const ssd_dims* d, const void* x, const float* dt, const float* A, const void* B,
                        const void* C, const float* D, const float* init, const void* z, void* y,
                        float* final_state, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const int* seq = nullptr) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (d->batch == 0) return SSD_OK;
    if (d->seqlen == 0) return state_passing_impl(d, nullptr, nullptr, init, final_state, stream);
    if (!final_state) return SSD_ERR_NULL_POINTER;
    if (!x || !dt || !A || !B || !C || !D || !y || !workspace) return SSD_ERR_NULL_POINTER;
    if (!aligned16(final_state) || !aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) ||
        !aligned16(C) || !aligned16(D) || !aligned16(y) || !aligned16(workspace) || (init && !aligned16(init)) ||
        (z && !aligned16(z)))
        return SSD_ERR_MISALIGNED;
    if (workspace_bytes < ssd_workspace_size(d)) return SSD_ERR_WORKSPACE_TOO_SMALL;
    float* cs = static_cast<float*>(workspace);
    void* states = static_cast<unsigned char*>(workspace) + round_up(cs_bytes_of(d));
    if (seq) {   // the fused chunk-state launch, with the document masks
        ssd::Params p = make_params(d);
        p.x = x;
        p.dt = dt;
        p.A = A;
        p.B = B;
        p.cs = cs;
        p.states = states;
        p.fuse_cs = 1;
        p.seq_idx = seq;
        st = to_status(ssd::launch_chunk_state(p, d->dtype, d->state_dtype, stream));
    } else {
        st = ssd_chunk_cumsum_state(d, x, dt, A, B, cs, states, stream);
    }
    if (st == SSD_OK) st = state_passing_impl(d, cs, states, init, final_state, stream, seq);
    if (st == SSD_OK) st = chunk_scan_impl(d, x, dt, B, C, D, cs, states, init ? 1 : 0, z, y, stream, seq);
    return st;
}


// packed documents, with the output gate when z is given
ssd_status varlen_impl(const ssd_dims* d, const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, const float* initial_state, const int32_t* seq_idx,
                       const void* z, void* y, float* final_state, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    if (empty(d)) return forward_impl(d, x, dt, A, B, C, D, initial_state, nullptr, y, final_state, workspace,
                                      workspace_bytes, stream);
    if (!seq_idx) return SSD_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(seq_idx) & 3) return SSD_ERR_MISALIGNED;
    // the chunk scan keeps the chunk's document ids in LDS beside its tiles
    if (ssd::chunk_scan_lds_bytes(d->dtype, d->state_dtype, d->headdim, d->dstate, d->chunk_size) +
            4 * (d->chunk_size < 32 ? 32 : d->chunk_size) > kMaxLds)
        return SSD_ERR_UNSUPPORTED;
    return forward_impl(d, x, dt, A, B, C, D, initial_state, z, y, final_state, workspace, workspace_bytes,
                        stream, seq_idx);
}

}  // namespace

extern "C" {

ssd_status ssd_state_passing(const ssd_dims* d, const float* cs, void* states, float* final_state,
                             hipStream_t stream) {
    return state_passing_impl(d, cs, states, nullptr, final_state, stream);
}

ssd_status ssd_state_passing_init(const ssd_dims* d, const float* cs, void* states, const float* initial_state,
                                  float* final_state, hipStream_t stream) {
    return state_passing_impl(d, cs, states, initial_state, final_state, stream);
}

ssd_status ssd_chunk_scan(const ssd_dims* d, const void* x, const float* dt, const void* B,
                          const void* C, const float* D, const float* cs, const void* states,
                          void* y, hipStream_t stream) {
    return chunk_scan_impl(d, x, dt, B, C, D, cs, states, 0, nullptr, y, stream);
}

ssd_status ssd_chunk_scan_init(const ssd_dims* d, const void* x, const float* dt, const void* B,
                               const void* C, const float* D, const float* cs, const void* states,
                               void* y, hipStream_t stream) {
    return chunk_scan_impl(d, x, dt, B, C, D, cs, states, 1, nullptr, y, stream);
}

ssd_status ssd_forward(const ssd_dims* d, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, void* y,
                       float* final_state, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    return forward_impl(d, x, dt, A, B, C, D, nullptr, nullptr, y, final_state, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the allocation-free forward -------------------------------------------
//
// The workspace of ssd_forward (cs and the inter-chunk states) in a fixed
// device array instead of a caller buffer. Each device holds its own copy
// from the first call on it until the process ends. In host code the array's
// name is only a stand-in: its device address is looked up once per device
// (hipGetSymbolAddress) and that address is what the kernels receive.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// this device's address of `scratch`, looked up on its first use (racing
// first calls look up the same address); nullptr on failure
void* device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace

extern "C" {

size_t ssd_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

ssd_status ssd_forward_noalloc(const ssd_dims* d, const void* x, const float* dt, const float* A, const void* B,
                               const void* C, const float* D, void* y, float* final_state, hipStream_t stream) {
    const ssd_status st = ssd_check_dims(d);
    if (st != SSD_OK) return st;
    const size_t need = ssd_workspace_size(d);
    if (need > kNoallocScratchBytes) return SSD_ERR_TOO_LARGE;
    if (d->batch == 0) return SSD_OK;
    if (d->seqlen == 0) return forward_impl(d, x, dt, A, B, C, D, nullptr, nullptr, y, final_state, nullptr, 0, stream);
    if (!x || !dt || !A || !B || !C || !D || !y || !final_state) return SSD_ERR_NULL_POINTER;
    void* ws = device_scratch();
    if (!ws) return SSD_ERR_LAUNCH;
    return forward_impl(d, x, dt, A, B, C, D, nullptr, nullptr, y, final_state, ws, kNoallocScratchBytes, stream);
}

ssd_status ssd_step(const ssd_dims* d, const void* x, const float* dt, const float* A, const void* B,
                    const void* C, const float* D, float* state, void* y, hipStream_t stream) {
    // one token: only the shapes and the input type matter (seqlen, chunk_size
    // and state_dtype are ignored)
    static const int64_t kP[] = {16, 32, 64, 128};
    static const int64_t kN[] = {16, 32, 64, 128, 256};
    if (!d) return SSD_ERR_NULL_POINTER;
    if (d->batch < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0 ||
        d->nheads % d->ngroups != 0)
        return SSD_ERR_BAD_SHAPE;
    if (!in_list(d->headdim, kP, 4) || !in_list(d->dstate, kN, 5)) return SSD_ERR_UNSUPPORTED;
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if (d->nheads > 0x7FFFFFFF || d->batch > 65535) return SSD_ERR_UNSUPPORTED;
    if (d->batch == 0) return SSD_OK;
    ssd_dims one = *d;
    one.seqlen = 1;
    one.chunk_size = 32;
    if (!x || !dt || !A || !B || !C || !D || !state || !y) return SSD_ERR_NULL_POINTER;
    if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(C) || !aligned16(D) ||
        !aligned16(state) || !aligned16(y))
        return SSD_ERR_MISALIGNED;
    ssd::Params p = make_params(&one);
    p.x = x;
    p.dt = dt;
    p.A = A;
    p.B = B;
    p.C = C;
    p.D = D;
    p.final_state = state;
    p.y = y;
    return to_status(ssd::launch_step(p, d->dtype, stream));
}

ssd_status ssd_forward_init(const ssd_dims* d, const void* x, const float* dt, const float* A,
                            const void* B, const void* C, const float* D, const float* initial_state,
                            void* y, float* final_state, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    return forward_impl(d, x, dt, A, B, C, D, initial_state, nullptr, y, final_state, workspace,
                        workspace_bytes, stream);
}

ssd_status ssd_forward_gated(const ssd_dims* d, const void* x, const float* dt, const float* A,
                             const void* B, const void* C, const float* D, const float* initial_state,
                             const void* z, void* y, float* final_state, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    if (d && d->batch > 0 && d->seqlen > 0 && !z) return SSD_ERR_NULL_POINTER;
    return forward_impl(d, x, dt, A, B, C, D, initial_state, z, y, final_state, workspace, workspace_bytes,
                        stream);
}

ssd_status ssd_forward_varlen(const ssd_dims* d, const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* D, const float* initial_state,
                              const int32_t* seq_idx, void* y, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    return varlen_impl(d, x, dt, A, B, C, D, initial_state, seq_idx, nullptr, y, final_state, workspace,
                       workspace_bytes, stream);
}

ssd_status ssd_forward_varlen_gated(const ssd_dims* d, const void* x, const float* dt, const float* A,
                                    const void* B, const void* C, const float* D, const float* initial_state,
                                    const int32_t* seq_idx, const void* z, void* y, float* final_state,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (d && d->batch > 0 && d->seqlen > 0 && !z) return SSD_ERR_NULL_POINTER;
    return varlen_impl(d, x, dt, A, B, C, D, initial_state, seq_idx, z, y, final_state, workspace,
                       workspace_bytes, stream);
}

// shapes of a per-head state: b >= 0, H, N, P in the supported lists
static ssd_status check_state_dims(const ssd_dims* d) {
    static const int64_t kP[] = {16, 32, 64, 128};
    static const int64_t kN[] = {16, 32, 64, 128, 256};
    if (!d) return SSD_ERR_NULL_POINTER;
    if (d->batch < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0) return SSD_ERR_BAD_SHAPE;
    if (!in_list(d->headdim, kP, 4) || !in_list(d->dstate, kN, 5)) return SSD_ERR_UNSUPPORTED;
    if (d->nheads > 65535 * 64 || d->batch > 65535) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

ssd_status ssd_total_decay(const ssd_dims* d, const float* dt, const float* A, float* total, hipStream_t stream) {
    ssd_status st = check_state_dims(d);
    if (st != SSD_OK) return st;
    if (d->seqlen < 0) return SSD_ERR_BAD_SHAPE;
    if (d->batch == 0) return SSD_OK;
    if (!A || !total || (d->seqlen > 0 && !dt)) return SSD_ERR_NULL_POINTER;
    if (!aligned16(A) || !aligned16(total) || (dt && !aligned16(dt))) return SSD_ERR_MISALIGNED;
    if (d->seqlen == 0) return to_status(ssd::launch_zero_fill(total, d->batch * d->nheads, stream));
    return to_status(ssd::launch_total_decay(dt, A, total, d->batch, d->seqlen, d->nheads, stream));
}

ssd_status ssd_fold_states(const ssd_dims* d, int64_t nshards, const float* totals, const float* shard_finals,
                           const float* initial_state, float* entering, hipStream_t stream) {
    ssd_status st = check_state_dims(d);
    if (st != SSD_OK) return st;
    if (nshards < 0) return SSD_ERR_BAD_SHAPE;
    if (d->batch == 0) return SSD_OK;
    if (!entering || (nshards > 0 && (!totals || !shard_finals))) return SSD_ERR_NULL_POINTER;
    if (!aligned16(entering) || (totals && !aligned16(totals)) || (shard_finals && !aligned16(shard_finals)) ||
        (initial_state && !aligned16(initial_state)))
        return SSD_ERR_MISALIGNED;
    const int64_t bh = d->batch * d->nheads, np = d->dstate * d->headdim;
    if (bh * np / 4 / 256 >= (int64_t)INT32_MAX) return SSD_ERR_UNSUPPORTED;
    return to_status(ssd::launch_fold(nshards, bh, np, totals, shard_finals, initial_state, entering, stream));
}

ssd_status ssd_gated_rmsnorm(const ssd_dims* d, const void* y, const void* z, const float* weight, float eps,
                             int64_t groups, void* out, hipStream_t stream) {
    if (!d) return SSD_ERR_NULL_POINTER;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || groups <= 0)
        return SSD_ERR_BAD_SHAPE;
    const int64_t C = d->nheads * d->headdim;
    if (C % groups != 0) return SSD_ERR_BAD_SHAPE;
    if (d->dtype != SSD_F32 && d->dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
    if ((C / groups) % 8 != 0) return SSD_ERR_UNSUPPORTED;   // whole 8-channel pieces per group
    const int64_t rows = d->batch * d->seqlen * groups;
    if (rows == 0) return SSD_OK;
    if (!y || !weight || !out) return SSD_ERR_NULL_POINTER;
    if (!aligned16(y) || !aligned16(weight) || !aligned16(out) || (z && !aligned16(z))) return SSD_ERR_MISALIGNED;
    if ((rows + 3) / 4 > (int64_t)INT32_MAX) return SSD_ERR_UNSUPPORTED;
    return to_status(ssd::launch_gated_rmsnorm(y, z, weight, eps, rows, groups, C / groups, out, d->dtype, stream));
}

}  // extern "C"
