/* Runs every function of oracle/hetattn_oracle.h on small inputs under the
 * host sanitizers and checks a few invariants of each result (counts, sorted
 * index lists, weights summing to one, the listed-key gradients equal to the
 * full backward's rows, argument rejection).  Exits non-zero on the first
 * failed check. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hetattn_oracle.h"

static int failures = 0;
#define CHECK(c)                                                             \
    do {                                                                     \
        if (!(c)) {                                                          \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c);     \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static unsigned int lcg = 12345u;
static float frand(void) {
    lcg = lcg * 1664525u + 1013904223u;
    return (float)((lcg >> 8) & 0xffff) / 32768.0f - 1.0f;
}

static void check_route(const unsigned char *mask, const int *di, const int *li, const int *counts, int B, int N) {
    for (int b = 0; b < B; b++) {
        const int nd = counts[2 * b], nl = counts[2 * b + 1];
        CHECK(nd + nl == N && nd >= 0 && nl >= 0);
        for (int i = 0; i < N; i++) {
            if (i < nd) CHECK(mask[b * N + di[b * N + i]] == 0 && (i == 0 || di[b * N + i] > di[b * N + i - 1]));
            else CHECK(di[b * N + i] == -1);
            if (i < nl) CHECK(mask[b * N + li[b * N + i]] == 1 && (i == 0 || li[b * N + i] > li[b * N + i - 1]));
            else CHECK(li[b * N + i] == -1);
        }
    }
}

int main(void) {
    enum { B = 2, H = 2, D = 8, T = 3, Hg = 4, Wg = 5, N = T * Hg * Wg };
    const long E = (long)B * N * H * D;
    float *q = malloc(sizeof(float) * E), *k = malloc(sizeof(float) * E), *v = malloc(sizeof(float) * E),
          *dout = malloc(sizeof(float) * E), *u = malloc(sizeof(float) * B * N);
    for (long e = 0; e < E; e++) { q[e] = frand(); k[e] = frand(); v[e] = frand(); dout[e] = frand(); }
    for (int i = 0; i < B * N; i++) u[i] = (i % 7 == 0) ? 0.5f : fabsf(frand());
    u[3] = NAN;
    u[5] = -0.0f;
    unsigned char mask[B * N], mask2[B * N];
    int di[B * N], li[B * N], counts[2 * B];
    double thresh[B];

    CHECK(oracle_route_top_rho(u, B, N, 0.25, mask, di, li, counts, thresh) == 0);
    check_route(mask, di, li, counts, B, N);
    CHECK(counts[0] == (int)floor(0.25 * N + 0.5));
    CHECK(oracle_route_top_rho(u, B, N, 1.5, mask, di, li, counts, thresh) < 0);
    CHECK(oracle_route_mean_std(u, B, N, 0.9, mask, di, li, counts, thresh) == 0);
    check_route(mask, di, li, counts, B, N);
    CHECK(oracle_route_uniform(B, N, 0.3, mask, di, li, counts) == 0);
    check_route(mask, di, li, counts, B, N);
    CHECK(oracle_route_random(B, N, 0.3, 77ull, 1u, 2u, mask, di, li, counts) == 0);
    check_route(mask, di, li, counts, B, N);
    memcpy(mask2, mask, sizeof(mask));
    CHECK(oracle_route_swap(mask2, B, N, 0.1, 5ull, 0u, 3u, mask, di, li, counts) == 0);
    check_route(mask, di, li, counts, B, N);
    unsigned int draws[N], ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out4[4];
    oracle_swap_draws(N, 1u, 9ull, 2u, 3u, draws);
    oracle_philox4x32_10(ctr, key, out4);
    int start, len;
    CHECK(oracle_window_axis(5, 3, 0, &start, &len) == 0 && start == 0 && len == 3);
    CHECK(oracle_window_axis_cut(5, 3, 0, &start, &len) == 0 && start == 0 && len == 2);
    CHECK(oracle_window_axis(5, 4, 0, &start, &len) < 0);

    CHECK(oracle_route_top_rho(u, B, N, 0.25, mask, di, li, counts, thresh) == 0);
    long rows[B * N];
    for (int i = 0; i < B * N; i++) rows[i] = i;
    double *o = malloc(sizeof(double) * E), *lse = malloc(sizeof(double) * B * N * H);
    double *w = malloc(sizeof(double) * N);
    for (int border = 0; border < 2; border++) {
        CHECK(oracle_attend_rows(q, k, v, B, H, D, T, Hg, Wg, 3, 3, 3, border, 0.3, mask, rows, B * N, o, 2) == 0);
        CHECK(oracle_row_lse(q, k, B, H, D, T, Hg, Wg, 3, 3, 3, border, 0.3, mask, rows, B * N, lse, 2) == 0);
        for (long row = 0; row < B * N; row += 7) {
            CHECK(oracle_attention_weights(q, k, B, H, D, T, Hg, Wg, 3, 3, 3, border, 0.3, mask, row, 1, w) == 0);
            double sw = 0.0;
            for (int j = 0; j < N; j++) sw += w[j];
            CHECK(fabs(sw - 1.0) < 1e-12);
        }
    }
    CHECK(oracle_attend_rows(q, k, v, B, H, D, T, Hg, Wg, 3, 2, 3, 0, 0.3, mask, rows, B * N, o, 2) < 0);
    rows[0] = -1;
    CHECK(oracle_attend_rows(q, k, v, B, H, D, T, Hg, Wg, 3, 3, 3, 0, 0.3, mask, rows, 1, o, 2) < 0);
    rows[0] = 0;

    double *dq = malloc(sizeof(double) * E), *dk = malloc(sizeof(double) * E), *dv = malloc(sizeof(double) * E);
    CHECK(oracle_attend_backward(q, k, v, dout, B, H, D, T, Hg, Wg, 3, 3, 3, 0, 0.3, mask, dq, dk, dv, 2) == 0);
    double *dqr = malloc(sizeof(double) * 4 * H * D);
    long some[4] = {0, 17, N, 2 * N - 1};
    CHECK(oracle_attend_backward_dq_rows(q, k, v, dout, B, H, D, T, Hg, Wg, 3, 3, 3, 0, 0.3, mask, some, 4, dqr,
                                         2) == 0);
    for (int r = 0; r < 4; r++)
        for (int e = 0; e < H * D; e++) CHECK(fabs(dqr[r * H * D + e] - dq[some[r] * H * D + e]) < 1e-12);
    int hsel[1] = {1};
    double *dkr = malloc(sizeof(double) * 4 * D), *dvr = malloc(sizeof(double) * 4 * D);
    CHECK(oracle_attend_backward_kv_rows(q, k, v, dout, B, H, D, T, Hg, Wg, 3, 3, 3, 0, 0.3, mask, some, 4, hsel, 1,
                                         dkr, dvr, 2) == 0);
    for (int r = 0; r < 4; r++)
        for (int d = 0; d < D; d++) {
            CHECK(fabs(dkr[r * D + d] - dk[(some[r] * H + 1) * D + d]) < 1e-12);
            CHECK(fabs(dvr[r * D + d] - dv[(some[r] * H + 1) * D + d]) < 1e-12);
        }
    long dup[2] = {3, 3};
    CHECK(oracle_attend_backward_kv_rows(q, k, v, dout, B, H, D, T, Hg, Wg, 3, 3, 3, 0, 0.3, mask, dup, 2, hsel, 1,
                                         dkr, dvr, 2) < 0);

    free(q); free(k); free(v); free(dout); free(u); free(o); free(lse); free(w);
    free(dq); free(dk); free(dv); free(dqr); free(dkr); free(dvr);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver ok\n");
    return 0;
}
