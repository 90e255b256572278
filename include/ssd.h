/*
 * libssd: the SSD (state space duality) chunked sequence transform on MI355X.
 *
 * The operation ("Transformers are SSMs", Dao & Gu; Knowl 1 of the chapterpal
 * summary) maps, per batch element and head h (group g = h / (H / G)):
 *
 *   h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * B_t x_t^T,  h_{-1} = 0   (N x P)
 *   y_t = C_t^T h_t + D_h * x_t
 *
 * and is evaluated by the block decomposition of Knowl 2: chunks of Q tokens,
 * the masked quadratic form (L o C B^T) X inside each chunk, a scalar linear
 * recurrence on N x P chunk states between chunks. Heads of one group share
 * B and C (Knowl 7, the multi-input / grouped-input patterns).
 *
 * Entry points: ssd_forward (the whole transform) and its stages
 * (ssd_chunk_cumsum, ssd_chunk_state, ssd_chunk_cumsum_state,
 * ssd_state_passing, ssd_chunk_scan); from a given initial state
 * (ssd_forward_init, ssd_state_passing_init, ssd_chunk_scan_init); with the
 * block's output gate (ssd_forward_gated) and the norm after it
 * (ssd_gated_rmsnorm); over rows packing several documents
 * (ssd_forward_varlen, and with the gate ssd_forward_varlen_gated); one
 * decoding token (ssd_step); the shard chain of
 * sequence parallelism (ssd_total_decay, ssd_fold_states); and sizing,
 * checking and status helpers.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *    16-byte aligned. The caller owns every buffer; the library never
 *    allocates, frees or keeps a pointer, holds no state between calls, and is
 *    safe to call from several threads.
 *  - Arguments are checked synchronously. On any error the call returns a
 *    status and launches nothing. On success the kernels are enqueued on
 *    `stream` (0 = the null stream) and the call returns without waiting;
 *    device faults surface at the caller's stream synchronisation.
 *  - Data values are never inspected: NaN and Inf propagate. A_h > 0 is
 *    computed as written (the pages take a_t in [0, 1]).
 *  - Sizes: batch >= 0, seqlen >= 0 (0 gives a zero final state), nheads,
 *    ngroups >= 1 with nheads % ngroups == 0; headdim P in {16, 32, 64, 128};
 *    dstate N in {16, 32, 64, 128, 256}; chunk_size Q in {16, 32, 64, 128, 256}.
 *    seqlen need not be a multiple of Q: the last chunk may be shorter.
 *
 * Tensor layouts (b = batch, T = seqlen, H = nheads, P = headdim, N = dstate,
 * G = ngroups, nc = ceil(T / Q)):
 *    x, y        [b, T, H, P]   dtype (fp32 or bf16)
 *    dt          [b, T, H]      fp32, the step size (softplus already applied)
 *    A, D        [H]            fp32
 *    B, C        [b, T, G, N]   dtype
 *    final_state [b, H, N, P]   fp32
 *    cs          [b, H, nc, Q]  fp32  (stage buffer, see ssd_chunk_cumsum)
 *    states      [b, nc, H, P, N] state dtype (stage buffer; note P before N)
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 1

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    SSD_ERR_BAD_SHAPE = 2,           /* negative or zero size, or nheads % ngroups != 0 */
    SSD_ERR_UNSUPPORTED = 3,         /* headdim/dstate/chunk_size/dtype outside the lists above */
    SSD_ERR_MISALIGNED = 4,          /* a tensor pointer is not 16-byte aligned */
    SSD_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < ssd_workspace_size() */
    SSD_ERR_LAUNCH = 6,              /* the HIP runtime rejected a launch */
    SSD_ERR_TOO_LARGE = 7            /* ssd_forward_noalloc: the workspace would exceed its fixed scratch */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
    int64_t batch;       /* b */
    int64_t seqlen;      /* T */
    int64_t nheads;      /* H */
    int64_t headdim;     /* P */
    int64_t dstate;      /* N */
    int64_t ngroups;     /* G: heads [g*H/G, (g+1)*H/G) share B[..., g, :] and C[..., g, :] */
    int64_t chunk_size;  /* Q */
    int32_t dtype;       /* ssd_dtype of x, B, C and y */
    int32_t state_dtype; /* ssd_dtype of the inter-chunk states in the workspace; SSD_BF16
                            only with dtype == SSD_BF16. The final state is always fp32. */
} ssd_dims;

/* Version of this interface (SSD_ABI_VERSION). */
int ssd_abi_version(void);

/* Text for a status code (static storage; never NULL). */
const char* ssd_status_string(ssd_status s);

/* Checks `d` alone (no pointers): SSD_OK or the error ssd_forward would give. */
ssd_status ssd_check_dims(const ssd_dims* d);

/* Bytes of device workspace ssd_forward needs for `d`; 0 when `d` is invalid
 * (and for batch == 0 or seqlen == 0, which need none). The workspace holds
 * the cs buffer and the states buffer below, each at a 256-byte aligned offset. */
size_t ssd_workspace_size(const ssd_dims* d);

/* Bytes of the two stage buffers for the stage entry points: cs [b,H,nc,Q] fp32
 * and states [b,nc,H,P,N] in d->state_dtype. Either output pointer may be NULL.
 * Returns ssd_check_dims(d). */
ssd_status ssd_stage_sizes(const ssd_dims* d, size_t* cs_bytes, size_t* states_bytes);

/*
 * Full forward: Knowl 2's inputs X, A, B, C and chunk size Q, its outputs Y and
 * h_final (the algorithm's inputs and outputs), with the per-head
 * discretisation dt, A and the skip term D. Enqueues, in order,
 * ssd_chunk_cumsum_state (stages 1 and 2 in one launch), ssd_state_passing
 * and ssd_chunk_scan; the result is bitwise that of the four stage entry
 * points run one after another.
 *   x [b,T,H,P], dt [b,T,H], A [H], B [b,T,G,N], C [b,T,G,N], D [H]: inputs
 *   y [b,T,H,P] (out, dtype), final_state [b,H,N,P] (out, fp32)
 *   workspace: device buffer of at least ssd_workspace_size(d) bytes; its
 *   contents on entry do not matter and are garbage on return.
 * y must not overlap any input. */
ssd_status ssd_forward(const ssd_dims* d, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, void* y,
                       float* final_state, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * ssd_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches and results as ssd_forward, with the workspace kept in a
 * fixed device array inside the library (ssd_noalloc_scratch_bytes() bytes,
 * 64 MiB) instead of a caller buffer. Each GPU the call runs on holds its own
 * copy of that array until the process ends; its address is looked up once per
 * device on the first call there. The call itself allocates nothing. Every
 * call on one GPU shares that GPU's array, so calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller; the array's contents on entry do not matter (nothing is read before
 * it is written). Errors: as ssd_forward (without the workspace ones), plus
 * SSD_ERR_TOO_LARGE when ssd_workspace_size(d) exceeds the array, and
 * SSD_ERR_LAUNCH when the array's device address cannot be found.
 */
ssd_status ssd_forward_noalloc(const ssd_dims* d, const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D, void* y,
                               float* final_state, hipStream_t stream);

/* Bytes of the fixed device scratch of ssd_forward_noalloc (the largest
 * ssd_workspace_size it accepts). */
size_t ssd_noalloc_scratch_bytes(void);

/*
 * Full forward from a given initial state: the recurrence of Knowl 1 started
 * at h_{-1} = initial_state instead of zero (so that a sequence can be resumed
 * from the final state of its prefix). initial_state [b,H,N,P] fp32 (device,
 * caller-owned, read only; 16-byte aligned), or NULL for a zero state, which
 * gives exactly ssd_forward. Enqueues ssd_chunk_cumsum_state,
 * ssd_state_passing_init and ssd_chunk_scan_init. With T = 0, final_state
 * receives a copy of initial_state. Other arguments and errors as ssd_forward.
 */
ssd_status ssd_forward_init(const ssd_dims* d, const void* x, const float* dt, const float* A,
                            const void* B, const void* C, const float* D, const float* initial_state,
                            void* y, float* final_state, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Full forward with the output gate of the Mamba-2 block fused into the chunk
 * scan's epilogue ("Transformers are SSMs", Knowl 6: the SSD output is gated
 * by SiLU of the block's z branch before the norm and the output projection):
 *   y = SSD(x, dt, A, B, C, D; initial_state) * silu(z),  silu(z) = z / (1 + e^{-z})
 * elementwise, z [b,T,H,P] in d->dtype (device, caller-owned, 16-byte aligned,
 * read only, required when b > 0 and T > 0). final_state is the ungated
 * state; initial_state as for ssd_forward_init (NULL: zero). Other arguments
 * and errors as ssd_forward_init.
 */
ssd_status ssd_forward_gated(const ssd_dims* d, const void* x, const float* dt, const float* A,
                             const void* B, const void* C, const float* D, const float* initial_state,
                             const void* z, void* y, float* final_state, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * The normalisation after the gate in the Mamba-2 block ("Transformers are
 * SSMs", Knowl 6: Y * SiLU(z), then a group or RMS norm before the output
 * projection; Knowl 8: the norm in groups whose count divides the
 * tensor-parallel degree). Per token, the H*P channels of y [b,T,H,P] are cut
 * into `groups` equal contiguous groups (1: RMSNorm over all channels):
 *   g = y * silu(z)  (y itself when z is NULL),
 *   out = g / sqrt(mean over the group of g^2 + eps) * weight[channel].
 * y, z and out are in d->dtype, [b,T,H,P]; weight [H*P] fp32; all device,
 * caller-owned, 16-byte aligned. out may be y (in place) but must not
 * otherwise overlap the inputs. eps is used as given. d gives batch, seqlen,
 * nheads, headdim and dtype (dstate, ngroups, chunk_size and state_dtype are
 * ignored). After ssd_forward_gated, a call with z = NULL and out = y
 * normalises the gated output in place. Errors: SSD_ERR_NULL_POINTER,
 * SSD_ERR_BAD_SHAPE (negative sizes, H or P < 1, groups < 1 or not dividing
 * H*P), SSD_ERR_UNSUPPORTED (unknown dtype, or a group size not a multiple
 * of 8 channels), SSD_ERR_MISALIGNED.
 */
ssd_status ssd_gated_rmsnorm(const ssd_dims* d, const void* y, const void* z, const float* weight, float eps,
                             int64_t groups, void* out, hipStream_t stream);

/*
 * Full forward over rows that pack several documents ("Transformers are SSMs",
 * Knowl 8: variable-length sequences concatenated, the state reset between
 * them by a zero decay at each document start). seq_idx [b,T] int32 (device,
 * caller-owned, read only, 4-byte aligned, required when b > 0 and T > 0)
 * gives each token's document id; ids must not decrease along T (the values
 * are not checked; with decreasing ids the result is undefined). At every
 * t > 0 whose id differs from that of t - 1 the decay exp(dt_t A_h) is taken
 * as 0, so no state crosses into a new document. initial_state (NULL: zero)
 * enters the row's first document; final_state is the state after token T - 1,
 * i.e. that of the last document. Enqueues the chunk-state, state-passing and
 * chunk-scan kernels in their document-masked instantiations. Errors as
 * ssd_forward_init, plus SSD_ERR_NULL_POINTER for a missing seq_idx,
 * SSD_ERR_MISALIGNED for one not 4-byte aligned, and SSD_ERR_UNSUPPORTED when
 * the chunk scan's LDS has no room for the chunk's ids (4 * chunk_size bytes
 * beyond the smallest tile set).
 */
ssd_status ssd_forward_varlen(const ssd_dims* d, const void* x, const float* dt, const float* A,
                              const void* B, const void* C, const float* D, const float* initial_state,
                              const int32_t* seq_idx, void* y, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Packed documents with the output gate: the block of "Transformers are
 * SSMs", Knowl 6 (y gated by SiLU(z) before the norm) over rows that pack
 * several documents as in Knowl 8. The same as ssd_forward_varlen, then
 *   y = y * silu(z),  silu(z) = z / (1 + e^{-z})
 * elementwise in the chunk scan's epilogue, z [b,T,H,P] in d->dtype (device,
 * caller-owned, 16-byte aligned, read only, required when b > 0 and T > 0).
 * final_state is the ungated state. Errors as ssd_forward_varlen, plus
 * SSD_ERR_NULL_POINTER for a missing z.
 */
ssd_status ssd_forward_varlen_gated(const ssd_dims* d, const void* x, const float* dt, const float* A,
                                    const void* B, const void* C, const float* D, const float* initial_state,
                                    const int32_t* seq_idx, const void* z, void* y, float* final_state,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Sequence (context) parallelism ("Transformers are SSMs", Knowl 8): a long
 * sequence cut along T into K shards, each run on its own tokens, with only
 * the boundary state passed from one shard to the next. The shard-level chain
 * is the state passing of Knowl 2 one level up:
 *   H_0 = initial state (or 0),  H_{k+1} = exp(Lambda_k) H_k + F_k,
 * where F_k is shard k's final state when run from a zero state
 * (ssd_forward) and Lambda_k = sum over its tokens of dt_t A_h, the log of
 * the product of its decays. Running shard k from H_k (ssd_forward_init)
 * then gives its exact output; H_K is the final state of the whole sequence.
 */

/*
 * Lambda for one shard: total[b,h] = A[h] * sum_t dt[b,t,h] (fp32, the sum
 * in a fixed order). d gives batch, seqlen (the shard's T), nheads, headdim
 * and dstate (the last two only checked); dt [b,T,H] fp32, A [H] fp32,
 * total [b,H] fp32 (device, 16-byte aligned). T = 0 writes zeros. Errors:
 * SSD_ERR_NULL_POINTER, SSD_ERR_BAD_SHAPE (negative sizes, H, N or P < 1),
 * SSD_ERR_UNSUPPORTED (P or N outside the supported lists),
 * SSD_ERR_MISALIGNED.
 */
ssd_status ssd_total_decay(const ssd_dims* d, const float* dt, const float* A, float* total,
                           hipStream_t stream);

/*
 * The shard chain for nshards = K >= 0 shards: totals [K,b,H] (Lambda_k, as
 * from ssd_total_decay), shard_finals [K,b,H,N,P] (F_k), initial_state
 * [b,H,N,P] or NULL for zero; entering [K+1,b,H,N,P] receives H_0 .. H_K
 * (H_k enters shard k; H_K is the final state). All fp32 device buffers,
 * 16-byte aligned, caller-owned; entering must not overlap the inputs. d gives
 * batch, nheads, headdim and dstate (seqlen, chunk_size and the dtypes are
 * ignored). Errors as ssd_total_decay, plus SSD_ERR_BAD_SHAPE for K < 0.
 */
ssd_status ssd_fold_states(const ssd_dims* d, int64_t nshards, const float* totals, const float* shard_finals,
                           const float* initial_state, float* entering, hipStream_t stream);

/*
 * One token of the recurrence, for decoding ("Transformers are SSMs", Knowl 1,
 * the recurrent form one step at a time: the inference mode with O(N P) state
 * per head):
 *   state[b,h] <- exp(dt[b,h] A[h]) state[b,h] + dt[b,h] B[b,g] x[b,h]^T
 *   y[b,h]      = C[b,g]^T state[b,h] + D[h] x[b,h],   g = h / (H / G)
 *   x [b,H,P] (d->dtype), dt [b,H] fp32, A [H], B [b,G,N], C [b,G,N] (d->dtype),
 *   D [H]: inputs; state [b,H,N,P] fp32, updated in place (the layout of
 *   ssd_forward's final_state, which can be passed straight in); y [b,H,P]
 *   (d->dtype) out. d->seqlen, d->chunk_size and d->state_dtype are ignored.
 * All pointers device, caller-owned, 16-byte aligned; y must not overlap the
 * inputs or the state. Errors: SSD_ERR_NULL_POINTER, SSD_ERR_MISALIGNED,
 * SSD_ERR_BAD_SHAPE, SSD_ERR_UNSUPPORTED (P or N outside the supported sets),
 * SSD_ERR_LAUNCH. batch = 0 is a no-op.
 */
ssd_status ssd_step(const ssd_dims* d, const void* x, const float* dt, const float* A, const void* B,
                    const void* C, const float* D, float* state, void* y, hipStream_t stream);

/*
 * Stage 1 (Knowl 2, first step: the running products of the decays inside
 * each chunk, taken in log space): cs[b,h,c,j] = sum_{s=0..j} dt[b,cQ+s,h] * A[h],
 * an inclusive prefix sum per chunk, so exp(cs) is the cumulative product of a. Positions past the
 * end of a short last chunk repeat its last value (padding tokens have dt = 0).
 *   dt [b,T,H], A [H] in; cs [b,H,nc,Q] fp32 out.
 */
ssd_status ssd_chunk_cumsum(const ssd_dims* d, const float* dt, const float* A, float* cs,
                            hipStream_t stream);

/*
 * Stage 2 (Knowl 2, second step: the chunk state S, B^T times the inputs
 * decayed to the chunk's end):
 *   states[b,c,h,p,n] = sum_j B[b,cQ+j,g,n] * exp(cs_last - cs_j) * dt[b,cQ+j,h] * x[b,cQ+j,h,p]
 * where cs_last is the chunk's last cs value: each token is decayed to the end
 * of its chunk. bf16 MFMA (fp32 MFMA for fp32 inputs), fp32 accumulation.
 *   x, dt, B, cs in; states [b,nc,H,P,N] out (transposed N x P matrices).
 */
ssd_status ssd_chunk_state(const ssd_dims* d, const void* x, const float* dt, const void* B,
                           const float* cs, void* states, hipStream_t stream);

/*
 * Stages 1 and 2 in one launch: each chunk-state workgroup first forms the
 * in-chunk prefix sums of its heads (the arithmetic of ssd_chunk_cumsum,
 * bitwise the same), writes them to cs and uses them for the chunk states.
 *   x, dt, A, B in; cs [b,H,nc,Q] fp32 out; states [b,nc,H,P,N] out.
 */
ssd_status ssd_chunk_cumsum_state(const ssd_dims* d, const void* x, const float* dt, const float* A,
                                  const void* B, float* cs, void* states, hipStream_t stream);

/*
 * Stage 3 (Knowl 2, the sequential loop over chunks h_{c+1} = (prod a) h_c + S_c,
 * h_0 = 0, h_final = h_{T/Q}): in place, states[c] (S_c on entry) is replaced by
 * the state entering chunk c (h_c; zero for c = 0), and final_state [b,H,N,P]
 * receives h_{nc} in fp32. The running state is kept in fp32.
 */
ssd_status ssd_state_passing(const ssd_dims* d, const float* cs, void* states,
                             float* final_state, hipStream_t stream);

/*
 * Stage 3 from a given initial state: as ssd_state_passing with h_0 =
 * initial_state [b,H,N,P] fp32 (NULL: zero), so states[c = 0] receives h_0.
 */
ssd_status ssd_state_passing_init(const ssd_dims* d, const float* cs, void* states,
                                  const float* initial_state, float* final_state, hipStream_t stream);

/*
 * Stage 4 (Knowl 2, diagonal-block outputs (L o C B^T) X, the off-diagonal
 * output C (decayed h_c) and their sum; plus D * x):
 *   y[t=cQ+j] = sum_{i<=j} (C_j . B_i) exp(cs_j - cs_i) dt_i x_i
 *             + exp(cs_j) C_j^T h_c + D_h x_j
 * with states holding h_c as written by ssd_state_passing.
 */
ssd_status ssd_chunk_scan(const ssd_dims* d, const void* x, const float* dt, const void* B,
                          const void* C, const float* D, const float* cs, const void* states,
                          void* y, hipStream_t stream);

/*
 * Stage 4 for a nonzero initial state: as ssd_chunk_scan, but the first
 * chunk's carried-state term exp(cs_j) C_j^T h_0 is applied as well, with h_0
 * read from states[c = 0] as ssd_state_passing_init wrote it. (ssd_chunk_scan
 * takes h_0 = 0 and does not read it.)
 */
ssd_status ssd_chunk_scan_init(const ssd_dims* d, const void* x, const float* dt, const void* B,
                               const void* C, const float* D, const float* cs, const void* states,
                               void* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
