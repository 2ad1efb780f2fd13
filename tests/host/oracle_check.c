/* Drives the float64 oracle (oracle/gqa_oracle.c) over small shapes,
 * including empty, clamped and fully masked sequences, on one and several
 * threads.  Built with AddressSanitizer and UndefinedBehaviorSanitizer by the
 * test that runs it; any report aborts the run.  Checks two closed forms
 * (a constant V returns the constant; one visible row returns that row) and
 * that the thread count does not change a bit.  Exits 0 when all hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gqa_oracle_decode_f64(int B, int H, int G, int sq, int T, int D, const double *q, const double *k,
                          const double *v, const int32_t *seq_lens, double scale, double *out, double *probs,
                          int nthreads);
int gqa_oracle_decode_row_f64(int H, int G, int sq, int T, int D, const double *q_row, const double *k_b,
                              const double *v_b, int h, int s, int seq_len_b, double scale, double *out_row);

static double urand(unsigned *st)
{
    *st = *st * 1664525u + 1013904223u;
    return ((*st >> 8) / 16777216.0) * 2.0 - 1.0;
}

int main(void)
{
    int fails = 0;
    const int shapes[][6] = {{1, 4, 2, 1, 5, 3}, {3, 6, 3, 2, 7, 4}, {2, 8, 1, 3, 9, 2}, {4, 4, 4, 1, 1, 5}};
    for (unsigned si = 0; si < sizeof(shapes) / sizeof(shapes[0]); ++si) {
        const int B = shapes[si][0], H = shapes[si][1], G = shapes[si][2], sq = shapes[si][3], T = shapes[si][4],
                  D = shapes[si][5];
        const size_t nq = (size_t)B * H * sq * D, nk = (size_t)B * G * T * D;
        double *q = malloc(nq * sizeof(double)), *k = malloc(nk * sizeof(double)), *v = malloc(nk * sizeof(double));
        double *o1 = malloc(nq * sizeof(double)), *o3 = malloc(nq * sizeof(double));
        double *pr = malloc((size_t)B * H * sq * T * sizeof(double));
        int32_t *lens = malloc((size_t)B * sizeof(int32_t));
        unsigned st = 7 + si;
        for (size_t i = 0; i < nq; ++i) q[i] = urand(&st);
        for (size_t i = 0; i < nk; ++i) k[i] = urand(&st);
        for (size_t i = 0; i < nk; ++i) v[i] = urand(&st);
        for (int b = 0; b < B; ++b) lens[b] = (b % 4 == 0) ? T : (b % 4 == 1) ? 0 : (b % 4 == 2) ? T + 5 : 1;
        if (gqa_oracle_decode_f64(B, H, G, sq, T, D, q, k, v, lens, 0.5, o1, pr, 1) != 0) ++fails;
        if (gqa_oracle_decode_f64(B, H, G, sq, T, D, q, k, v, lens, 0.5, o3, NULL, 3) != 0) ++fails;
        if (memcmp(o1, o3, nq * sizeof(double)) != 0) {
            printf("thread count changed the result (shape %u)\n", si);
            ++fails;
        }
        /* row entry point agrees bit for bit */
        double *row = malloc((size_t)D * sizeof(double));
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < H; ++h)
                for (int s = 0; s < sq; ++s) {
                    const size_t r = ((size_t)(b * H + h) * sq + s) * D;
                    if (gqa_oracle_decode_row_f64(H, G, sq, T, D, q + r, k + (size_t)b * G * T * D,
                                                  v + (size_t)b * G * T * D, h, s, lens[b], 0.5, row) != 0)
                        ++fails;
                    if (memcmp(row, o1 + r, (size_t)D * sizeof(double)) != 0) {
                        printf("row entry point differs (shape %u, b %d h %d s %d)\n", si, b, h, s);
                        ++fails;
                    }
                }
        /* constant V per KV head returns that constant wherever a row is visible */
        for (int b = 0; b < B; ++b)
            for (int g = 0; g < G; ++g)
                for (int t = 0; t < T; ++t)
                    for (int d = 0; d < D; ++d) v[(((size_t)b * G + g) * T + t) * D + d] = 0.25 * (g + 1) - 0.1 * d;
        gqa_oracle_decode_f64(B, H, G, sq, T, D, q, k, v, lens, 0.5, o1, NULL, 2);
        for (int b = 0; b < B; ++b) {
            const int L = lens[b] < 0 ? 0 : (lens[b] > T ? T : lens[b]);
            for (int h = 0; h < H; ++h)
                for (int s = 0; s < sq; ++s)
                    for (int d = 0; d < D; ++d) {
                        const int g = h / (H / G);
                        const double want = (L - sq + s >= 0) ? 0.25 * (g + 1) - 0.1 * d : 0.0;
                        const double got = o1[((size_t)(b * H + h) * sq + s) * D + d];
                        if (fabs(got - want) > 1e-12) {
                            printf("constant V: shape %u b %d h %d s %d d %d got %g want %g\n", si, b, h, s, d,
                                   got, want);
                            ++fails;
                        }
                    }
        }
        free(q); free(k); free(v); free(o1); free(o3); free(pr); free(lens); free(row);
    }
    /* bad arguments are refused, never read */
    double x = 0;
    if (gqa_oracle_decode_f64(1, 3, 2, 1, 1, 1, &x, &x, &x, NULL, 1.0, &x, NULL, 1) == 0) ++fails;
    if (gqa_oracle_decode_f64(1, 4, 2, 0, 1, 1, &x, &x, &x, NULL, 1.0, &x, NULL, 1) == 0) ++fails;
    if (gqa_oracle_decode_row_f64(4, 2, 1, 1, 1, &x, &x, &x, 4, 0, 1, 1.0, &x) == 0) ++fails;
    printf("oracle checks done, %d failures\n", fails);
    return fails == 0 ? 0 : 1;
}
