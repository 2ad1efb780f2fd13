/*
 * gqa_oracle.c -- plain float64 CPU oracle for grouped-query attention at
 * decode time.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library.
 * It shares no code, header, table or helper with the HIP path: it is the
 * slow, obviously correct definition the HIP kernels are checked against.
 *
 * What it computes (sources, cited by page title and section):
 *
 *  - "GQA (Grouped-Query Attention) 분석", section "Grouped broadcast":
 *    query head h reads KV head g(h) = floor(h / (H/G)); the head's scores
 *    are softmax(Q[h] . K[g(h)]^T / sqrt(D)) and its output is those scores
 *    times V[g(h)].  Logically the same as repeating K/V H/G times.
 *  - same page, section "동작 원리 / 3. Incremental decode": at each step
 *    the new token's query attends over the whole cache of its group, after
 *    the new K/V were appended to the cache.
 *  - "Same GQA, Different Execution Cost Across Backends", section 1 (the
 *    one mapping every implementation shares): kv = h // group_size, with
 *    contiguous blocks of query heads per KV head.
 *
 * Readings where the pages leave a step open (each one also listed in the
 * design notes of the repository):
 *  - scale is an explicit argument (the pages use 1/sqrt(D));
 *  - seq_lens[b] counts the valid cache rows of sequence b, including the
 *    sq new tokens, which sit at the end of the valid range; values are
 *    clamped to [0, T]; a NULL seq_lens means every sequence holds T rows;
 *  - with sq > 1 new tokens, query s sees cache rows 0 .. L - sq + s
 *    (causal, aligned to the end of the valid range);
 *  - a query row that sees no cache row at all outputs zeros.
 *
 * The softmax is computed in two passes (max, then exp/sum) in float64, in a
 * fixed loop order.  No blocking, no chunking, no online rescaling.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* g(h) = floor(h / (H / G)).  Requires H % G == 0. */
int gqa_oracle_kv_head(int h, int H, int G) { return h / (H / G); }

typedef struct {
    int B, H, G, sq, T, D;
    const double *q, *k, *v;
    const int32_t *seq_lens;
    double scale;
    double *out;   /* [B,H,sq,D] */
    double *probs; /* optional [B,H,sq,T]; NULL when not wanted */
    long first, last; /* half-open range of (b,h,s) units for this worker */
} oracle_job;

/*
 * One output row.  qrow: [D]; kb, vb: the [T,D] cache slab of the row's KV
 * head; L: valid rows of the sequence (already clamped to [0, T]);
 * s: index of this query among the sq new tokens.  z: scratch of T doubles.
 */
static void oracle_row_core(const double *qrow, const double *kb, const double *vb,
                            long L, int sq, int s, int T, int D, double scale,
                            double *orow, double *prow, double *z)
{
    const long last = L - sq + s; /* last visible cache row for this query */

    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (prow)
        for (long j = 0; j < T; ++j) prow[j] = 0.0;
    if (last < 0) return; /* sees nothing: zeros */

    /* scores z_j = scale * <q, k_j>, j = 0..last */
    for (long j = 0; j <= last; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * kb[(size_t)j * D + d];
        z[j] = scale * acc;
    }
    /* softmax: max, exponentials, sum, normalise */
    double m = z[0];
    for (long j = 1; j <= last; ++j)
        if (z[j] > m) m = z[j];
    double Z = 0.0;
    for (long j = 0; j <= last; ++j) {
        z[j] = exp(z[j] - m);
        Z += z[j];
    }
    for (long j = 0; j <= last; ++j) z[j] /= Z;
    if (prow)
        for (long j = 0; j <= last; ++j) prow[j] = z[j];
    /* output = sum_j p_j * v_j */
    for (long j = 0; j <= last; ++j) {
        const double p = z[j];
        for (int d = 0; d < D; ++d) orow[d] += p * vb[(size_t)j * D + d];
    }
}

static long clamp_len(long L, int T)
{
    if (L < 0) return 0;
    if (L > T) return T;
    return L;
}

/* Row (b, h, s) of a full problem: picks the KV head g(h) and the slabs. */
static void oracle_row(const oracle_job *J, int b, int h, int s, double *z)
{
    const int H = J->H, G = J->G, sq = J->sq, T = J->T, D = J->D;
    const int g = gqa_oracle_kv_head(h, H, G);
    const long L = clamp_len(J->seq_lens ? (long)J->seq_lens[b] : (long)T, T);
    const size_t row = ((size_t)b * H + h) * sq + s;
    oracle_row_core(J->q + row * D,
                    J->k + ((size_t)b * G + g) * (size_t)T * D,
                    J->v + ((size_t)b * G + g) * (size_t)T * D,
                    L, sq, s, T, D, J->scale, J->out + row * D,
                    J->probs ? J->probs + row * (size_t)T : NULL, z);
}

static void *oracle_worker(void *arg)
{
    const oracle_job *J = (const oracle_job *)arg;
    double *z = (double *)malloc(sizeof(double) * (size_t)(J->T > 0 ? J->T : 1));
    if (!z) return (void *)1;
    for (long u = J->first; u < J->last; ++u) {
        const int s = (int)(u % J->sq);
        const int h = (int)((u / J->sq) % J->H);
        const int b = (int)(u / ((long)J->sq * J->H));
        oracle_row(J, b, h, s, z);
    }
    free(z);
    return NULL;
}

/*
 * out[b,h,s,:] for every (b,h,s).  q: [B,H,sq,D], k,v: [B,G,T,D], all
 * float64, row-major, contiguous.  seq_lens: [B] int32 or NULL.
 * probs: NULL, or [B,H,sq,T] receiving each row's softmax (zeros on
 * invisible rows).  nthreads >= 1 splits the rows over POSIX threads; the
 * arithmetic of each row does not depend on nthreads.
 * Returns 0, or 1 on a bad argument.
 */
int gqa_oracle_decode_f64(int B, int H, int G, int sq, int T, int D,
                          const double *q, const double *k, const double *v,
                          const int32_t *seq_lens, double scale, double *out,
                          double *probs, int nthreads)
{
    if (B < 0 || H <= 0 || G <= 0 || sq <= 0 || T <= 0 || D <= 0) return ORACLE_BAD_ARG;
    if (H % G != 0) return ORACLE_BAD_ARG;
    if (!q || !k || !v || !out) return ORACLE_BAD_ARG;
    if (nthreads < 1) nthreads = 1;
    const long units = (long)B * H * sq;
    if (units == 0) return ORACLE_OK;
    if (nthreads > units) nthreads = (int)units;

    oracle_job *jobs = (oracle_job *)calloc((size_t)nthreads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    char *started = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !tids || !started) {
        free(jobs);
        free(tids);
        free(started);
        return ORACLE_BAD_ARG;
    }
    int rc = ORACLE_OK;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *J = &jobs[t];
        J->B = B; J->H = H; J->G = G; J->sq = sq; J->T = T; J->D = D;
        J->q = q; J->k = k; J->v = v; J->seq_lens = seq_lens;
        J->scale = scale; J->out = out; J->probs = probs;
        J->first = units * t / nthreads;
        J->last = units * (t + 1) / nthreads;
    }
    if (nthreads == 1) {
        if (oracle_worker(&jobs[0]) != NULL) rc = ORACLE_BAD_ARG;
    } else {
        for (int t = 0; t < nthreads; ++t) {
            if (pthread_create(&tids[t], NULL, oracle_worker, &jobs[t]) == 0) {
                started[t] = 1;
            } else if (oracle_worker(&jobs[t]) != NULL) { /* run it inline */
                rc = ORACLE_BAD_ARG;
            }
        }
        for (int t = 0; t < nthreads; ++t) {
            if (!started[t]) continue;
            void *ret = NULL;
            pthread_join(tids[t], &ret);
            if (ret != NULL) rc = ORACLE_BAD_ARG;
        }
    }
    free(jobs);
    free(tids);
    free(started);
    return rc;
}

/*
 * One row only: out_row[D] for query head h, new-token index s of one
 * sequence.  Lets tests check sampled rows of a problem too large to
 * evaluate whole.  q_row: that row's [D] query; k_b, v_b: the sequence's
 * [G,T,D] cache slabs; seq_len_b: its valid length (negative means T).
 */
int gqa_oracle_decode_row_f64(int H, int G, int sq, int T, int D,
                              const double *q_row, const double *k_b,
                              const double *v_b, int h, int s, int seq_len_b,
                              double scale, double *out_row)
{
    if (H <= 0 || G <= 0 || sq <= 0 || T <= 0 || D <= 0 || H % G != 0) return ORACLE_BAD_ARG;
    if (h < 0 || h >= H || s < 0 || s >= sq) return ORACLE_BAD_ARG;
    if (!q_row || !k_b || !v_b || !out_row) return ORACLE_BAD_ARG;
    double *z = (double *)malloc(sizeof(double) * (size_t)T);
    if (!z) return ORACLE_BAD_ARG;
    const int g = gqa_oracle_kv_head(h, H, G);
    const long L = clamp_len(seq_len_b < 0 ? (long)T : (long)seq_len_b, T);
    oracle_row_core(q_row, k_b + (size_t)g * T * D, v_b + (size_t)g * T * D,
                    L, sq, s, T, D, scale, out_row, NULL, z);
    free(z);
    return ORACLE_OK;
}
