/*
 * gdn_oracle.c -- fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the HIP
 * library under gated_deltanet_scan_amd/.
 *
 * What it computes (no chunks, no blocking, no fusion): the gated delta rule
 * in the closed form of the Qwen3.5-9B architecture page (section Gated
 * DeltaNet), one token at a time, for every value head independently.  With
 * the forget gate a_t = exp(g_t) and the correction rate b_t, the state
 * S (dk x dv) moves from S_{t-1} to
 *     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T.
 * Expanded, this is one read of the old state along k_t and one rank-one
 * write: with r = S_{t-1}^T k_t (the value the state returns for k_t),
 *     e   = b_t (v_t - a_t r)          (the part of v_t the decayed state misses)
 *     S_t = a_t S_{t-1} + k_t e^T
 * and the token's output is the new state read along q_t, o_t = scale S_t^T q_t.
 * The NPU page ("Qwen3.5-9B -- every component on the Intel NPU", section
 * "How it works") runs the same rule as a per-token loop on the NPU.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of this repository):
 *   - the output is multiplied by `scale` (1/sqrt(dk) in every workload),
 *     i.e. o_t = scale * S_t^T q_t;
 *   - value head h reads query/key head floor(h * HQK / HV) (contiguous
 *     grouped-query blocks);
 *   - layouts: q, k [T, HQK, dk]; v, o [T, HV, dv]; g, beta [T, HV];
 *     state [N, HV, dk, dv] with S[i][j], i over dk, j over dv (S^T k
 *     contracts the key index);
 *   - packed variable-length batches: sequence n owns tokens
 *     cu_seqlens[n] .. cu_seqlens[n+1]-1 and starts from its own state.
 *
 * Precision: every operand is taken as fp64 and every operation is done in
 * fp64, in the order of the expanded form above.  Inputs are expected to be the exact
 * values the device receives (bf16 or fp32 widened without rounding).
 *
 * Parity pins: see the CPU tests (brute-force product of the closed-form
 * factors, pure decay with beta = 0, exact recall with alpha = 1, beta = 1,
 * unit keys, one-hot key overwrite, padding tokens, composition, the
 * chunkwise-parallel form).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t total_tokens;
    int32_t num_seqs, hqk, hv, dk, dv;
    const int64_t *cu_seqlens;
    const double *q, *k, *v, *g, *beta, *s0;
    double scale;
    double *o, *s_out;
    int64_t num_items;
    int64_t next_item; /* guarded by lock */
    pthread_mutex_t lock;
} job_t;

/* One (sequence, value head) recurrence, token by token. */
static void run_item(const job_t *J, int64_t item, double *S, double *r)
{
    const int32_t hv = J->hv, dk = J->dk, dv = J->dv, hqk = J->hqk;
    const int32_t n = (int32_t)(item / hv);
    const int32_t h = (int32_t)(item % hv);
    const int32_t hq = (int32_t)(((int64_t)h * hqk) / hv); /* grouped query/key head */
    const size_t state_elems = (size_t)dk * dv;
    const size_t state_off = ((size_t)n * hv + h) * state_elems;

    if (J->s0)
        memcpy(S, J->s0 + state_off, state_elems * sizeof(double));
    else
        memset(S, 0, state_elems * sizeof(double));

    for (int64_t t = J->cu_seqlens[n]; t < J->cu_seqlens[n + 1]; ++t) {
        const double *qt = J->q + ((size_t)t * hqk + hq) * dk;
        const double *kt = J->k + ((size_t)t * hqk + hq) * dk;
        const double *vt = J->v + ((size_t)t * hv + h) * dv;
        const double alpha = exp(J->g[(size_t)t * hv + h]);
        const double b = J->beta[(size_t)t * hv + h];
        double *ot = J->o + ((size_t)t * hv + h) * dv;

        /* r = S_{t-1}^T k_t */
        for (int32_t j = 0; j < dv; ++j)
            r[j] = 0.0;
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j)
                r[j] += kt[i] * S[(size_t)i * dv + j];
        /* e = b_t (v_t - a_t r), kept in r */
        for (int32_t j = 0; j < dv; ++j)
            r[j] = b * (vt[j] - alpha * r[j]);
        /* S_t = a_t S_{t-1} + k_t e^T */
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = alpha * S[(size_t)i * dv + j] + kt[i] * r[j];
        /* o_t = scale S_t^T q_t */
        for (int32_t j = 0; j < dv; ++j)
            ot[j] = 0.0;
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t j = 0; j < dv; ++j)
                ot[j] += qt[i] * S[(size_t)i * dv + j];
        for (int32_t j = 0; j < dv; ++j)
            ot[j] *= J->scale;
    }
    memcpy(J->s_out + state_off, S, state_elems * sizeof(double));
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc((size_t)J->dk * J->dv * sizeof(double));
    double *r = (double *)malloc((size_t)J->dv * sizeof(double));
    if (!S || !r) {
        free(S);
        free(r);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t item = J->next_item++;
        pthread_mutex_unlock(&J->lock);
        if (item >= J->num_items)
            break;
        run_item(J, item, S, r);
    }
    free(S);
    free(r);
    return NULL;
}

/*
 * Runs the recurrence for every (sequence, value head) pair.
 * Returns 0 on success, a negative value on bad arguments or when a worker
 * could not allocate its scratch.  `o` must be zero-length-safe: tokens of
 * the packed batch are written exactly once each.
 */
int gdn_oracle_forward(int64_t total_tokens, int32_t num_seqs, const int64_t *cu_seqlens,
                       int32_t hqk, int32_t hv, int32_t dk, int32_t dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta,
                       const double *initial_state, double scale,
                       double *o, double *final_state, int32_t num_threads)
{
    if (num_seqs < 0 || hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0)
        return -1;
    if (!cu_seqlens || !final_state)
        return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != total_tokens)
        return -2;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -2;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o))
        return -1;

    job_t J;
    J.total_tokens = total_tokens;
    J.num_seqs = num_seqs;
    J.hqk = hqk;
    J.hv = hv;
    J.dk = dk;
    J.dv = dv;
    J.cu_seqlens = cu_seqlens;
    J.q = q;
    J.k = k;
    J.v = v;
    J.g = g;
    J.beta = beta;
    J.s0 = initial_state;
    J.scale = scale;
    J.o = o;
    J.s_out = final_state;
    J.num_items = (int64_t)num_seqs * hv;
    J.next_item = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (num_threads < 1)
        num_threads = 1;
    if (num_threads > J.num_items)
        num_threads = (int32_t)(J.num_items > 0 ? J.num_items : 1);

    int rc = 0;
    pthread_t *tids = (pthread_t *)calloc((size_t)num_threads, sizeof(pthread_t));
    if (!tids) {
        pthread_mutex_destroy(&J.lock);
        return -3;
    }
    int32_t started = 0;
    for (int32_t i = 1; i < num_threads; ++i) {
        if (pthread_create(&tids[i], NULL, worker, &J) != 0)
            break;
        ++started;
    }
    if (worker(&J) != NULL)
        rc = -3;
    for (int32_t i = 1; i <= started; ++i) {
        void *ret = NULL;
        pthread_join(tids[i], &ret);
        if (ret != NULL)
            rc = -3;
    }
    free(tids);
    pthread_mutex_destroy(&J.lock);
    return rc;
}
