/*
 * fp64 CPU oracle for the SSD (state space duality) sequence transform.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load, call or
 * link this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes ("Transformers are SSMs", Knowl 1, the linear (recurrent)
 * form, with the per-head discretisation a_t = exp(dt_t * A_h), an input term
 * scaled by dt_t, and a skip term D_h * x_t):
 *
 *   for every batch element b and head h, with group g = h / (H / G):
 *     state_{-1} = init[b,h] (zero when no initial state is given)   (N x P)
 *     state_t    = exp(dt[b,t,h] * A[h]) * state_{t-1}
 *                  + dt[b,t,h] * B[b,t,g,:] (outer) x[b,t,h,:]
 *     y[b,t,h,:] = C[b,t,g,:]^T state_t + D[h] * x[b,t,h,:]
 *   final[b,h]   = state_{T-1}
 *
 * Variable-length packing (Knowl 8: documents concatenated into one sequence,
 * the state reset at each document start by a zero decay there): with sequence
 * ids seq [b,T] (int32, non-decreasing along t), the decay
 * exp(dt[b,t,h] * A[h]) is replaced by 0 at every t > 0 whose id differs from
 * that of t - 1, so the state entering a document's first token is dropped.
 * The initial state, if given, enters the first document.
 *
 * This is the plain definition: the block-decomposition algorithm (Knowl 2)
 * reaches exactly this result, so the oracle is the recurrence itself and not
 * the algorithm. Heads of one group share B and C (Knowl 7, the grouped
 * pattern), assigned contiguously.
 *
 * Layouts (row-major, contiguous): x, y [b,T,H,P]; dt [b,T,H]; A, D [H];
 * B, C [b,T,G,N]; final and init [b,H,N,P]. Optional boundary snapshots
 * snaps [b,nc,H,N,P], nc = ceil(T / every): snaps[c] is the state after token
 * c*every - 1, i.e. the state entering chunk c (the initial state for c = 0).
 *
 * Parallelism: a pool of POSIX threads takes (b, h) items from a shared
 * counter. Each item is independent; results do not depend on the thread
 * count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, every;
    const double *x, *dt, *A, *B, *C, *D, *init;
    const int32_t* seq;  /* [b,T] sequence ids, or NULL */
    double *y, *final_state, *snaps;
    int64_t next;      /* shared work counter */
    int failed;
} job_t;

static void run_item(job_t* j, int64_t item, double* st) {
    const int64_t T = j->seqlen, H = j->nheads, P = j->headdim, N = j->dstate;
    const int64_t G = j->ngroups;
    const int64_t b = item / H, h = item % H;
    const int64_t g = h / (H / G);
    const double Ah = j->A[h], Dh = j->D[h];
    if (j->init)
        memcpy(st, j->init + ((b * H + h) * N) * P, sizeof(double) * (size_t)(N * P));
    else
        memset(st, 0, sizeof(double) * (size_t)(N * P));
    for (int64_t t = 0; t < T; ++t) {
        if (j->snaps && t % j->every == 0) {
            const int64_t nc = (T + j->every - 1) / j->every;
            double* dst = j->snaps + (((b * nc + t / j->every) * H + h) * N) * P;
            memcpy(dst, st, sizeof(double) * (size_t)(N * P));
        }
        const double dtv = j->dt[(b * T + t) * H + h];
        const int starts = j->seq && t > 0 && j->seq[b * T + t] != j->seq[b * T + t - 1];
        const double a = starts ? 0.0 : exp(dtv * Ah);
        const double* xt = j->x + ((b * T + t) * H + h) * P;
        const double* Bt = j->B + ((b * T + t) * G + g) * N;
        const double* Ct = j->C + ((b * T + t) * G + g) * N;
        double* yt = j->y + ((b * T + t) * H + h) * P;
        for (int64_t n = 0; n < N; ++n) {
            const double u = dtv * Bt[n];
            double* row = st + n * P;
            for (int64_t p = 0; p < P; ++p) row[p] = a * row[p] + u * xt[p];
        }
        for (int64_t p = 0; p < P; ++p) yt[p] = Dh * xt[p];
        for (int64_t n = 0; n < N; ++n) {
            const double c = Ct[n];
            const double* row = st + n * P;
            for (int64_t p = 0; p < P; ++p) yt[p] += c * row[p];
        }
    }
    if (j->final_state)
        memcpy(j->final_state + ((b * H + h) * N) * P, st, sizeof(double) * (size_t)(N * P));
}

static void* worker(void* arg) {
    job_t* j = (job_t*)arg;
    double* st = (double*)malloc(sizeof(double) * (size_t)(j->dstate * j->headdim));
    if (!st) {
        __atomic_store_n(&j->failed, 1, __ATOMIC_RELAXED);
        return NULL;
    }
    const int64_t items = j->batch * j->nheads;
    for (;;) {
        int64_t it = __atomic_fetch_add(&j->next, 1, __ATOMIC_RELAXED);
        if (it >= items) break;
        run_item(j, it, st);
    }
    free(st);
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation/thread failure.
 * y and x may not alias. init, final_state, snaps and seq may be NULL (init
 * NULL: zero initial state; seq NULL: one sequence per batch row). every <= 0
 * turns the snapshots off. nthreads < 1 means 1. */
int ssd_oracle_forward_varlen(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                              int64_t dstate, int64_t ngroups, const double* x, const double* dt,
                              const double* A, const double* B, const double* C, const double* D,
                              const double* init, const int32_t* seq, double* y, double* final_state,
                              int64_t every, double* snaps, int nthreads) {
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    if (!x || !dt || !A || !B || !C || !D || !y) return -1;
    if (batch == 0 || seqlen == 0) {
        if (final_state && batch > 0) {
            const size_t n = (size_t)(batch * nheads * dstate * headdim);
            if (init)
                memcpy(final_state, init, sizeof(double) * n);
            else
                memset(final_state, 0, sizeof(double) * n);
        }
        return 0;
    }
    job_t j;
    j.batch = batch; j.seqlen = seqlen; j.nheads = nheads; j.headdim = headdim;
    j.dstate = dstate; j.ngroups = ngroups; j.every = every;
    j.x = x; j.dt = dt; j.A = A; j.B = B; j.C = C; j.D = D; j.init = init; j.seq = seq;
    j.y = y; j.final_state = final_state; j.snaps = (every > 0) ? snaps : NULL;
    j.next = 0; j.failed = 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > batch * nheads) nthreads = (int)(batch * nheads);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &j) != 0) break;
        ++started;
    }
    if (started == 0) worker(&j);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    return j.failed ? -2 : 0;
}

/* The same with one sequence per batch row. */
int ssd_oracle_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups, const double* x, const double* dt,
                       const double* A, const double* B, const double* C, const double* D,
                       const double* init, double* y, double* final_state, int64_t every,
                       double* snaps, int nthreads) {
    return ssd_oracle_forward_varlen(batch, seqlen, nheads, headdim, dstate, ngroups, x, dt, A, B, C,
                                     D, init, NULL, y, final_state, every, snaps, nthreads);
}
