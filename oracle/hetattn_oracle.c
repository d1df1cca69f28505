/*
 * hetattn_oracle.c -- plain fp64 CPU oracle for uncertainty-routed
 * heterogeneous attention.  TEST INFRASTRUCTURE ONLY (see the header).
 *
 * [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
 * Video Diffusion" (HetA-DiT, arXiv 2609.31050), full text.
 *
 * Each function writes the definition out directly: a library sort for the
 * ranking, explicit loops for every sum.  Nothing is blocked, fused or
 * reordered beyond what the definitions state.
 */
#include "hetattn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* u as used for ranking: u_i >= 0 on the pages ([HetA §3.2.1 Eq. 7]); a -0
 * is the same value as +0 and a NaN is read as the most uncertain value. */
static double mapped_u(float x)
{
    if (isnan(x)) return INFINITY;
    if (x == 0.0f) return 0.0;
    return (double)x;
}

typedef struct {
    double u;
    int idx;
} ranked_token;

/* Larger u first; equal u -> smaller token index first. */
static int rank_cmp(const void *pa, const void *pb)
{
    const ranked_token *a = (const ranked_token *)pa;
    const ranked_token *b = (const ranked_token *)pb;
    if (a->u > b->u) return -1;
    if (a->u < b->u) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx) ? 1 : 0;
}

/* From a per-token dense flag, write the mask (1 = local, [HetA §3.2.2
 * Eq. 12]) and the two ascending index lists with their counts. */
static void write_route(const unsigned char *dense, int N, unsigned char *mask,
                        int *dense_idx, int *local_idx, int *counts)
{
    int nd = 0, nl = 0;
    for (int i = 0; i < N; i++) {
        if (dense[i]) {
            mask[i] = 0;
            dense_idx[nd++] = i;
        } else {
            mask[i] = 1;
            local_idx[nl++] = i;
        }
    }
    for (int i = nd; i < N; i++) dense_idx[i] = -1;
    for (int i = nl; i < N; i++) local_idx[i] = -1;
    counts[0] = nd;
    counts[1] = nl;
}

int oracle_route_top_rho(const float *u, int B, int N, double rho,
                         unsigned char *mask, int *dense_idx, int *local_idx,
                         int *counts, double *thresh)
{
    if (!u || !mask || !dense_idx || !local_idx || !counts || !thresh) return -1;
    if (B <= 0 || N <= 0) return -1;
    if (!(rho >= 0.0 && rho <= 1.0)) return -1;

    long K = (long)floor(rho * (double)N + 0.5);
    if (K < 0) K = 0;
    if (K > N) K = N;

    ranked_token *order = (ranked_token *)malloc(sizeof(ranked_token) * (size_t)N);
    unsigned char *dense = (unsigned char *)malloc((size_t)N);
    if (!order || !dense) {
        free(order);
        free(dense);
        return -2;
    }
    for (int b = 0; b < B; b++) {
        const float *ub = u + (size_t)b * N;
        for (int i = 0; i < N; i++) {
            order[i].u = mapped_u(ub[i]);
            order[i].idx = i;
        }
        qsort(order, (size_t)N, sizeof(ranked_token), rank_cmp);
        memset(dense, 0, (size_t)N);
        for (long r = 0; r < K; r++) dense[order[r].idx] = 1;
        thresh[b] = (K == 0) ? INFINITY : order[K - 1].u;
        write_route(dense, N, mask + (size_t)b * N, dense_idx + (size_t)b * N,
                    local_idx + (size_t)b * N, counts + 2 * b);
    }
    free(order);
    free(dense);
    return 0;
}

int oracle_route_mean_std(const float *u, int B, int N, double c,
                          unsigned char *mask, int *dense_idx, int *local_idx,
                          int *counts, double *thresh)
{
    if (!u || !mask || !dense_idx || !local_idx || !counts || !thresh) return -1;
    if (B <= 0 || N <= 0) return -1;
    if (!isfinite(c)) return -1;

    unsigned char *dense = (unsigned char *)malloc((size_t)N);
    if (!dense) return -2;
    for (int b = 0; b < B; b++) {
        const float *ub = u + (size_t)b * N;
        /* Eq. 11: mean and (population) standard deviation over the sample. */
        double sum = 0.0;
        for (int i = 0; i < N; i++) sum += mapped_u(ub[i]);
        double mu = sum / (double)N;
        double ss = 0.0;
        for (int i = 0; i < N; i++) {
            double dlt = mapped_u(ub[i]) - mu;
            ss += dlt * dlt;
        }
        double sigma = sqrt(ss / (double)N);
        double T = mu + c * sigma;
        /* Eq. 12: m_i = 1[u_i < T]; the dense tokens are those with m_i = 0. */
        for (int i = 0; i < N; i++) dense[i] = (mapped_u(ub[i]) < T) ? 0 : 1;
        thresh[b] = T;
        write_route(dense, N, mask + (size_t)b * N, dense_idx + (size_t)b * N,
                    local_idx + (size_t)b * N, counts + 2 * b);
    }
    free(dense);
    return 0;
}

/* Philox4x32 (Salmon et al., SC'11): one round multiplies two of the four
 * words by the Philox constants, takes the high and low halves of the 64-bit
 * products and mixes the high halves with the other two words and the key;
 * the key is advanced by the two Weyl increments between rounds. */
void oracle_philox4x32_10(const unsigned int ctr[4], const unsigned int key[2], unsigned int out[4])
{
    const unsigned long long M0 = 0xD2511F53ull, M1 = 0xCD9E8D57ull;
    const unsigned int W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    unsigned int x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    unsigned int k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; round++) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        unsigned long long p0 = M0 * (unsigned long long)x0;
        unsigned long long p1 = M1 * (unsigned long long)x2;
        unsigned int hi0 = (unsigned int)(p0 >> 32), lo0 = (unsigned int)p0;
        unsigned int hi1 = (unsigned int)(p1 >> 32), lo1 = (unsigned int)p1;
        unsigned int y0 = hi1 ^ x1 ^ k0;
        unsigned int y2 = hi0 ^ x3 ^ k1;
        x0 = y0;
        x1 = lo1;
        x2 = y2;
        x3 = lo0;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

typedef struct {
    unsigned int key;
    int idx;
} keyed_token;

/* Smaller key first; equal keys -> smaller token index first. */
static int key_cmp(const void *pa, const void *pb)
{
    const keyed_token *a = (const keyed_token *)pa;
    const keyed_token *b = (const keyed_token *)pb;
    if (a->key < b->key) return -1;
    if (a->key > b->key) return 1;
    if (a->idx == b->idx) return 0;
    return (a->idx < b->idx) ? -1 : 1;
}

int oracle_route_swap(const unsigned char *mask_in, int B, int N, double r,
                      unsigned long long seed, unsigned int step, unsigned int block,
                      unsigned char *mask, int *dense_idx, int *local_idx, int *counts)
{
    if (!mask_in || !mask || !dense_idx || !local_idx || !counts) return -1;
    if (B <= 0 || N <= 0) return -1;
    if (!(r >= 0.0 && r <= 1.0)) return -1;
    const long S0 = (long)floor(r * (double)N + 0.5);
    const unsigned int key[2] = {(unsigned int)(seed & 0xffffffffull), (unsigned int)(seed >> 32)};

    keyed_token *dset = (keyed_token *)malloc(sizeof(keyed_token) * (size_t)N);
    keyed_token *lset = (keyed_token *)malloc(sizeof(keyed_token) * (size_t)N);
    unsigned char *dense = (unsigned char *)malloc((size_t)N);
    if (!dset || !lset || !dense) {
        free(dset);
        free(lset);
        free(dense);
        return -2;
    }
    for (int b = 0; b < B; b++) {
        const unsigned char *mb = mask_in + (size_t)b * N;
        int nd = 0, nl = 0;
        for (int i = 0; i < N; i++) {
            const unsigned int ctr[4] = {(unsigned int)i, (unsigned int)b, block, step};
            unsigned int out[4];
            oracle_philox4x32_10(ctr, key, out);
            if (mb[i] == 0) {
                dset[nd].key = out[0];
                dset[nd].idx = i;
                nd++;
            } else {
                lset[nl].key = out[0];
                lset[nl].idx = i;
                nl++;
            }
        }
        long S = S0;
        if (S > nd) S = nd;
        if (S > nl) S = nl;
        qsort(dset, (size_t)nd, sizeof(keyed_token), key_cmp);
        qsort(lset, (size_t)nl, sizeof(keyed_token), key_cmp);
        for (int i = 0; i < N; i++) dense[i] = (mb[i] == 0);
        for (long s = 0; s < S; s++) {
            dense[dset[s].idx] = 0;
            dense[lset[s].idx] = 1;
        }
        write_route(dense, N, mask + (size_t)b * N, dense_idx + (size_t)b * N,
                    local_idx + (size_t)b * N, counts + 2 * b);
    }
    free(dset);
    free(lset);
    free(dense);
    return 0;
}

void oracle_swap_draws(int N, unsigned int b, unsigned long long seed, unsigned int step,
                       unsigned int block, unsigned int *out)
{
    const unsigned int key[2] = {(unsigned int)(seed & 0xffffffffull), (unsigned int)(seed >> 32)};
    for (int i = 0; i < N; i++) {
        const unsigned int ctr[4] = {(unsigned int)i, b, block, step};
        unsigned int w[4];
        oracle_philox4x32_10(ctr, key, w);
        out[i] = w[0];
    }
}

/* Dense count of the rho-based routers: floor(rho*N + 1/2), clamped. */
static long rho_count(double rho, int N)
{
    double k = floor((double)N * rho + 0.5);
    if (k < 0.0) k = 0.0;
    if (k > (double)N) k = (double)N;
    return (long)k;
}

int oracle_route_uniform(int B, int N, double rho, unsigned char *mask, int *dense_idx,
                         int *local_idx, int *counts)
{
    if (!mask || !dense_idx || !local_idx || !counts || B <= 0 || N <= 0) return -1;
    if (!(rho >= 0.0 && rho <= 1.0)) return -1;
    const long K = rho_count(rho, N);
    unsigned char *dense = (unsigned char *)calloc((size_t)N, 1);
    if (!dense) return -2;
    /* K lattice points over the flattened volume, starting at token 0. */
    for (long j = 0; j < K; j++) dense[j * (long)N / K] = 1;
    for (int b = 0; b < B; b++)
        write_route(dense, N, mask + (size_t)b * N, dense_idx + (size_t)b * N,
                    local_idx + (size_t)b * N, counts + 2 * b);
    free(dense);
    return 0;
}

int oracle_route_random(int B, int N, double rho, unsigned long long seed, unsigned int step,
                        unsigned int block, unsigned char *mask, int *dense_idx, int *local_idx,
                        int *counts)
{
    if (!mask || !dense_idx || !local_idx || !counts || B <= 0 || N <= 0) return -1;
    if (!(rho >= 0.0 && rho <= 1.0)) return -1;
    const long K = rho_count(rho, N);
    keyed_token *tok = (keyed_token *)malloc(sizeof(keyed_token) * (size_t)N);
    unsigned int *x = (unsigned int *)malloc(sizeof(unsigned int) * (size_t)N);
    unsigned char *dense = (unsigned char *)malloc((size_t)N);
    if (!tok || !x || !dense) {
        free(tok);
        free(x);
        free(dense);
        return -2;
    }
    for (int b = 0; b < B; b++) {
        oracle_swap_draws(N, (unsigned int)b, seed, step, block, x);
        for (int i = 0; i < N; i++) {
            tok[i].key = x[i];
            tok[i].idx = i;
            dense[i] = 0;
        }
        qsort(tok, (size_t)N, sizeof(keyed_token), key_cmp);
        for (long j = 0; j < K; j++) dense[tok[j].idx] = 1;
        write_route(dense, N, mask + (size_t)b * N, dense_idx + (size_t)b * N,
                    local_idx + (size_t)b * N, counts + 2 * b);
    }
    free(tok);
    free(x);
    free(dense);
    return 0;
}

int oracle_window_axis(int S, int k, int pos, int *start, int *len)
{
    if (S <= 0 || k <= 0 || (k % 2) == 0 || pos < 0 || pos >= S || !start || !len)
        return -1;
    int L = (k < S) ? k : S;
    int s = pos - (k - 1) / 2; /* window centred on pos ... */
    if (s > S - L) s = S - L;  /* ... moved back inside the grid */
    if (s < 0) s = 0;
    *start = s;
    *len = L;
    return 0;
}

int oracle_window_axis_cut(int S, int k, int pos, int *start, int *len)
{
    if (S <= 0 || k <= 0 || (k % 2) == 0 || pos < 0 || pos >= S || !start || !len)
        return -1;
    const int h = (k - 1) / 2;
    int lo = pos - h, hi = pos + h + 1; /* centred on pos ... */
    if (lo < 0) lo = 0;                 /* ... and cut at the grid border */
    if (hi > S) hi = S;
    *start = lo;
    *len = hi - lo;
    return 0;
}

/* Softmax attention of one query over an explicit key list, in double:
 * s_j = scale * q.k_j, a_j = exp(s_j - max s) / sum exp(s - max s),
 * o = sum_j a_j v_j ([HetA §3.1.1 Eqs. 2-3]).  Subtracting the maximum only
 * keeps exp() in range; it does not change a_j.  lse_out, if given, gets
 * log sum_j exp(s_j) = max s + log sum exp(s - max s), the log of the
 * softmax's normaliser. */
static void attend_one(const float *qrow, const float *kbase, const float *vbase,
                       long key_stride, int D, const int *keys, int nkeys,
                       double scale, double *s, double *o, double *w_out, double *lse_out)
{
    double smax = -INFINITY;
    for (int j = 0; j < nkeys; j++) {
        const float *kr = kbase + (long)keys[j] * key_stride;
        double dot = 0.0;
        for (int d = 0; d < D; d++) dot += (double)qrow[d] * (double)kr[d];
        s[j] = scale * dot;
        if (s[j] > smax) smax = s[j];
    }
    double denom = 0.0;
    for (int j = 0; j < nkeys; j++) {
        s[j] = exp(s[j] - smax);
        denom += s[j];
    }
    if (lse_out) *lse_out = smax + log(denom);
    for (int d = 0; d < D; d++) o[d] = 0.0;
    for (int j = 0; j < nkeys; j++) {
        double a = s[j] / denom;
        if (w_out) w_out[j] = a;
        if (vbase) {
            const float *vr = vbase + (long)keys[j] * key_stride;
            for (int d = 0; d < D; d++) o[d] += a * (double)vr[d];
        }
    }
}

/* The key set of token n: every token of the sample when dense (mask 0),
 * else the 3D box of [HetA §3.1.1 Eq. 3] in t-major order, shifted inside
 * the grid (border 0) or cut at its border (border 1). */
static int key_set(int n, unsigned char is_local, int T, int Hg, int Wg,
                   int wt, int wh, int ww, int border, int *keys)
{
    int N = T * Hg * Wg;
    if (!is_local) {
        for (int j = 0; j < N; j++) keys[j] = j;
        return N;
    }
    int t = n / (Hg * Wg), y = (n / Wg) % Hg, x = n % Wg;
    int t0, lt, y0, ly, x0, lx;
    if (border == 0) {
        oracle_window_axis(T, wt, t, &t0, &lt);
        oracle_window_axis(Hg, wh, y, &y0, &ly);
        oracle_window_axis(Wg, ww, x, &x0, &lx);
    } else {
        oracle_window_axis_cut(T, wt, t, &t0, &lt);
        oracle_window_axis_cut(Hg, wh, y, &y0, &ly);
        oracle_window_axis_cut(Wg, ww, x, &x0, &lx);
    }
    int m = 0;
    for (int a = t0; a < t0 + lt; a++)
        for (int bb = y0; bb < y0 + ly; bb++)
            for (int c = x0; c < x0 + lx; c++) keys[m++] = (a * Hg + bb) * Wg + c;
    return m;
}

static int check_shape(int B, int heads, int D, int T, int Hg, int Wg, int wt,
                       int wh, int ww, int border)
{
    if (border != 0 && border != 1) return -1;
    if (B <= 0 || heads <= 0 || D <= 0 || T <= 0 || Hg <= 0 || Wg <= 0) return -1;
    if (wt <= 0 || wh <= 0 || ww <= 0) return -1;
    if (wt % 2 == 0 || wh % 2 == 0 || ww % 2 == 0) return -1;
    return 0;
}

int oracle_attend_rows(const float *q, const float *k, const float *v,
                       int B, int heads, int D,
                       int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                       double scale, const unsigned char *mask,
                       const long *rows, long nrows, double *out, int nthreads)
{
    if (!q || !k || !v || !mask || !rows || !out) return -1;
    if (check_shape(B, heads, D, T, Hg, Wg, wt, wh, ww, border)) return -1;
    const long N = (long)T * Hg * Wg;
    for (long r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= (long)B * N) return -1;
    const long tok_stride = (long)heads * D; /* [B, N, heads, D] */
    int err = 0;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : err)
    {
        int *keys = (int *)malloc(sizeof(int) * (size_t)N);
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        if (!keys || !s) {
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < nrows; r++) {
                long b = rows[r] / N, n = rows[r] % N;
                int nk = key_set((int)n, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border, keys);
                for (int h = 0; h < heads; h++) {
                    const float *qrow = q + (b * N + n) * tok_stride + (long)h * D;
                    const float *kb = k + b * N * tok_stride + (long)h * D;
                    const float *vb = v + b * N * tok_stride + (long)h * D;
                    attend_one(qrow, kb, vb, tok_stride, D, keys, nk, scale, s,
                               out + (r * heads + h) * (long)D, NULL, NULL);
                }
            }
        }
        free(keys);
        free(s);
    }
    return err ? -2 : 0;
}

int oracle_row_lse(const float *q, const float *k,
                   int B, int heads, int D,
                   int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                   double scale, const unsigned char *mask,
                   const long *rows, long nrows, double *out, int nthreads)
{
    if (!q || !k || !mask || !rows || !out) return -1;
    if (check_shape(B, heads, D, T, Hg, Wg, wt, wh, ww, border)) return -1;
    const long N = (long)T * Hg * Wg;
    for (long r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= (long)B * N) return -1;
    const long tok_stride = (long)heads * D;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : err)
    {
        int *keys = (int *)malloc(sizeof(int) * (size_t)N);
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        if (!keys || !s || !o) {
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < nrows; r++) {
                long b = rows[r] / N, n = rows[r] % N;
                int nk = key_set((int)n, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border, keys);
                for (int h = 0; h < heads; h++) {
                    const float *qrow = q + (b * N + n) * tok_stride + (long)h * D;
                    const float *kb = k + b * N * tok_stride + (long)h * D;
                    attend_one(qrow, kb, NULL, tok_stride, D, keys, nk, scale, s, o, NULL,
                               out + r * heads + h);
                }
            }
        }
        free(keys);
        free(s);
        free(o);
    }
    return err ? -2 : 0;
}

int oracle_attention_weights(const float *q, const float *k,
                             int B, int heads, int D,
                             int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                             double scale, const unsigned char *mask,
                             long row, int head, double *weights)
{
    if (!q || !k || !mask || !weights) return -1;
    if (check_shape(B, heads, D, T, Hg, Wg, wt, wh, ww, border)) return -1;
    const long N = (long)T * Hg * Wg;
    if (row < 0 || row >= (long)B * N || head < 0 || head >= heads) return -1;
    const long tok_stride = (long)heads * D;
    long b = row / N, n = row % N;
    int *keys = (int *)malloc(sizeof(int) * (size_t)N);
    double *s = (double *)malloc(sizeof(double) * (size_t)N);
    double *w = (double *)malloc(sizeof(double) * (size_t)N);
    double *o = (double *)malloc(sizeof(double) * (size_t)D);
    if (!keys || !s || !w || !o) {
        free(keys); free(s); free(w); free(o);
        return -2;
    }
    int nk = key_set((int)n, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border, keys);
    const float *qrow = q + (b * N + n) * tok_stride + (long)head * D;
    const float *kb = k + b * N * tok_stride + (long)head * D;
    attend_one(qrow, kb, NULL, tok_stride, D, keys, nk, scale, s, o, w, NULL);
    for (long j = 0; j < N; j++) weights[j] = 0.0;
    for (int j = 0; j < nk; j++) weights[keys[j]] = w[j];
    free(keys); free(s); free(w); free(o);
    return 0;
}

/* Backward of one query row over its key list, in double ([HetA §3.1.1
 * Eqs. 2-3] differentiated): with p the softmax weights, dP_j = dO.v_j,
 * D = sum_j p_j dP_j and dS_j = p_j (dP_j - D), the row adds
 * scale * sum_j dS_j k_j to dq, scale * dS_j q to dk_j and p_j dO to dv_j
 * (dk, dv may be NULL).  s and w are scratch of nkeys doubles. */
static void backward_one(const float *qrow, const float *dorow, const float *kbase,
                         const float *vbase, long key_stride, int D, const int *keys, int nkeys,
                         double scale, double *s, double *w, double *dq, double *dkbase,
                         double *dvbase)
{
    double smax = -INFINITY;
    for (int j = 0; j < nkeys; j++) {
        const float *krow = kbase + keys[j] * key_stride;
        double qk = 0.0;
        for (int d = 0; d < D; d++) qk += (double)qrow[d] * (double)krow[d];
        s[j] = qk * scale;
        if (s[j] > smax) smax = s[j];
    }
    double denom = 0.0;
    for (int j = 0; j < nkeys; j++) {
        s[j] = exp(s[j] - smax);
        denom += s[j];
    }
    double Dsum = 0.0;
    for (int j = 0; j < nkeys; j++) {
        s[j] /= denom; /* p_j */
        const float *vrow = vbase + keys[j] * key_stride;
        double dp = 0.0;
        for (int d = 0; d < D; d++) dp += (double)dorow[d] * (double)vrow[d];
        w[j] = dp; /* dP_j */
        Dsum += s[j] * dp;
    }
    for (int d = 0; d < D; d++) dq[d] = 0.0;
    for (int j = 0; j < nkeys; j++) {
        const double ds = s[j] * (w[j] - Dsum);
        const float *krow = kbase + keys[j] * key_stride;
        for (int d = 0; d < D; d++) dq[d] += scale * ds * (double)krow[d];
        if (dkbase) {
            double *dkr = dkbase + (long)keys[j] * key_stride;
            double *dvr = dvbase + (long)keys[j] * key_stride;
            for (int d = 0; d < D; d++) {
                dkr[d] += scale * ds * (double)qrow[d];
                dvr[d] += s[j] * (double)dorow[d];
            }
        }
    }
}

int oracle_attend_backward(const float *q, const float *k, const float *v, const float *dout,
                           int B, int heads, int D,
                           int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                           double scale, const unsigned char *mask,
                           double *dq, double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !dout || !mask || !dq || !dk || !dv) return -1;
    if (check_shape(B, heads, D, T, Hg, Wg, wt, wh, ww, border)) return -1;
    const long N = (long)T * Hg * Wg;
    const long tok_stride = (long)heads * D;
    for (long e = 0; e < (long)B * N * tok_stride; e++) {
        dk[e] = 0.0;
        dv[e] = 0.0;
    }
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    /* One (sample, head) per task: the dk, dv rows it adds to are its own. */
#pragma omp parallel reduction(| : err)
    {
        int *keys = (int *)malloc(sizeof(int) * (size_t)N);
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *w = (double *)malloc(sizeof(double) * (size_t)N);
        if (!keys || !s || !w) {
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < (long)B * heads; bh++) {
                const long b = bh / heads, h = bh % heads;
                const long base = b * N * tok_stride + h * D;
                for (long n = 0; n < N; n++) {
                    int nk = key_set((int)n, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border, keys);
                    backward_one(q + base + n * tok_stride, dout + base + n * tok_stride, k + base,
                                 v + base, tok_stride, D, keys, nk, scale, s, w,
                                 dq + base + n * tok_stride, dk + base, dv + base);
                }
            }
        }
        free(keys);
        free(s);
        free(w);
    }
    return err ? -2 : 0;
}

int oracle_attend_backward_dq_rows(const float *q, const float *k, const float *v,
                                   const float *dout, int B, int heads, int D,
                                   int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                                   double scale, const unsigned char *mask,
                                   const long *rows, long nrows, double *dq, int nthreads)
{
    if (!q || !k || !v || !dout || !mask || !rows || !dq) return -1;
    if (check_shape(B, heads, D, T, Hg, Wg, wt, wh, ww, border)) return -1;
    const long N = (long)T * Hg * Wg;
    for (long r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= (long)B * N) return -1;
    const long tok_stride = (long)heads * D;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel reduction(| : err)
    {
        int *keys = (int *)malloc(sizeof(int) * (size_t)N);
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *w = (double *)malloc(sizeof(double) * (size_t)N);
        if (!keys || !s || !w) {
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < nrows; r++) {
                const long b = rows[r] / N, n = rows[r] % N;
                int nk = key_set((int)n, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border, keys);
                for (int h = 0; h < heads; h++) {
                    const long base = b * N * tok_stride + (long)h * D;
                    backward_one(q + base + n * tok_stride, dout + base + n * tok_stride, k + base,
                                 v + base, tok_stride, D, keys, nk, scale, s, w,
                                 dq + (r * heads + h) * (long)D, NULL, NULL);
                }
            }
        }
        free(keys);
        free(s);
        free(w);
    }
    return err ? -2 : 0;
}


/* Whether token j lies in the key set of token n of the same sample: every
 * token for a dense row (mask 0), else the 3D window of n along each axis,
 * shifted (border 0) or cut (border 1) exactly as key_set builds it. */
static int key_in_set(int n, int j, unsigned char is_local, int T, int Hg, int Wg,
                      int wt, int wh, int ww, int border)
{
    if (!is_local) return 1;
    const int pos_n[3] = {n / (Hg * Wg), (n / Wg) % Hg, n % Wg};
    const int pos_j[3] = {j / (Hg * Wg), (j / Wg) % Hg, j % Wg};
    const int ext[3] = {T, Hg, Wg}, win[3] = {wt, wh, ww};
    for (int ax = 0; ax < 3; ax++) {
        int start, len;
        if (border == 0) oracle_window_axis(ext[ax], win[ax], pos_n[ax], &start, &len);
        else oracle_window_axis_cut(ext[ax], win[ax], pos_n[ax], &start, &len);
        if (pos_j[ax] < start || pos_j[ax] >= start + len) return 0;
    }
    return 1;
}

/* The two statistics of one row that its key gradients need, over its key
 * list: lse = log sum_j exp(s_j) with s_j = scale * q.k_j, and
 * dsum = sum_j p_j dP_j with p_j = exp(s_j - lse) and dP_j = dout.v_j.
 * s is scratch of nkeys doubles. */
static void row_grad_stats(const float *qrow, const float *dorow, const float *kbase,
                           const float *vbase, long key_stride, int D, const int *keys, int nkeys,
                           double scale, double *s, double *lse, double *dsum)
{
    double smax = -INFINITY;
    for (int j = 0; j < nkeys; j++) {
        const float *krow = kbase + keys[j] * key_stride;
        double qk = 0.0;
        for (int d = 0; d < D; d++) qk += (double)qrow[d] * (double)krow[d];
        s[j] = scale * qk;
        if (s[j] > smax) smax = s[j];
    }
    double denom = 0.0;
    for (int j = 0; j < nkeys; j++) denom += exp(s[j] - smax);
    *lse = smax + log(denom);
    double acc = 0.0;
    for (int j = 0; j < nkeys; j++) {
        const float *vrow = vbase + keys[j] * key_stride;
        double dp = 0.0;
        for (int d = 0; d < D; d++) dp += (double)dorow[d] * (double)vrow[d];
        acc += exp(s[j] - *lse) * dp;
    }
    *dsum = acc;
}

int oracle_attend_backward_kv_rows(const float *q, const float *k, const float *v,
                                   const float *dout, int B, int heads, int D,
                                   int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                                   double scale, const unsigned char *mask,
                                   const long *rows, long nrows, const int *hsel, int nh,
                                   double *dk, double *dv, int nthreads)
{
    if (!q || !k || !v || !dout || !mask || !rows || !hsel || !dk || !dv || nh <= 0) return -1;
    if (check_shape(B, heads, D, T, Hg, Wg, wt, wh, ww, border)) return -1;
    const long N = (long)T * Hg * Wg;
    for (int i = 0; i < nh; i++)
        if (hsel[i] < 0 || hsel[i] >= heads) return -1;
    for (long r = 0; r < nrows; r++) {
        if (rows[r] < 0 || rows[r] >= (long)B * N) return -1;
        for (long r2 = 0; r2 < r; r2++)
            if (rows[r2] == rows[r]) return -1; /* each key listed once */
    }
    const long tok_stride = (long)heads * D;
    for (long e = 0; e < nrows * nh * D; e++) {
        dk[e] = 0.0;
        dv[e] = 0.0;
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    /* needed[n] = 1 when row n of sample b holds a listed key in its key set;
     * lse and dsum are that row's statistics (per selected head). */
    unsigned char *needed = (unsigned char *)malloc((size_t)N);
    double *lse = (double *)malloc(sizeof(double) * (size_t)N * nh);
    double *dsum = (double *)malloc(sizeof(double) * (size_t)N * nh);
    int err = (!needed || !lse || !dsum);
    for (long b = 0; b < B && !err; b++) {
        int any = 0;
        for (long r = 0; r < nrows; r++) any |= rows[r] / N == b;
        if (!any) continue;
        /* Which rows of sample b see a listed key. */
#pragma omp parallel for schedule(dynamic, 64)
        for (long n = 0; n < N; n++) {
            needed[n] = 0;
            for (long r = 0; r < nrows && !needed[n]; r++)
                if (rows[r] / N == b &&
                    key_in_set((int)n, (int)(rows[r] % N), mask[b * N + n], T, Hg, Wg, wt, wh, ww, border))
                    needed[n] = 1;
        }
        /* Their statistics, each over the row's whole key set. */
#pragma omp parallel reduction(| : err)
        {
            int *keys = (int *)malloc(sizeof(int) * (size_t)N);
            double *s = (double *)malloc(sizeof(double) * (size_t)N);
            if (!keys || !s) {
                err = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (long n = 0; n < N; n++) {
                    if (!needed[n]) continue;
                    int nk = key_set((int)n, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border, keys);
                    for (int i = 0; i < nh; i++) {
                        const long base = b * N * tok_stride + (long)hsel[i] * D;
                        row_grad_stats(q + base + n * tok_stride, dout + base + n * tok_stride, k + base,
                                       v + base, tok_stride, D, keys, nk, scale, s, lse + n * nh + i,
                                       dsum + n * nh + i);
                    }
                }
            }
            free(keys);
            free(s);
        }
        /* Each listed key sums over the rows that see it, in row order:
         * dS_nj = p_nj (dP_nj - dsum_n), dK_j += scale dS_nj q_n,
         * dV_j += p_nj dout_n. */
#pragma omp parallel for schedule(dynamic, 1)
        for (long r = 0; r < nrows; r++) {
            if (rows[r] / N != b) continue;
            const long j = rows[r] % N;
            for (long n = 0; n < N; n++) {
                if (!needed[n] ||
                    !key_in_set((int)n, (int)j, mask[b * N + n], T, Hg, Wg, wt, wh, ww, border))
                    continue;
                for (int i = 0; i < nh; i++) {
                    const long base = b * N * tok_stride + (long)hsel[i] * D;
                    const float *qn = q + base + n * tok_stride, *don = dout + base + n * tok_stride;
                    const float *krow = k + base + j * tok_stride, *vrow = v + base + j * tok_stride;
                    double qk = 0.0, dp = 0.0;
                    for (int d = 0; d < D; d++) {
                        qk += (double)qn[d] * (double)krow[d];
                        dp += (double)don[d] * (double)vrow[d];
                    }
                    const double p = exp(scale * qk - lse[n * nh + i]);
                    const double ds = p * (dp - dsum[n * nh + i]);
                    double *dkr = dk + (r * nh + i) * (long)D, *dvr = dv + (r * nh + i) * (long)D;
                    for (int d = 0; d < D; d++) {
                        dkr[d] += scale * ds * (double)qn[d];
                        dvr[d] += p * (double)don[d];
                    }
                }
            }
        }
    }
    free(needed);
    free(lse);
    free(dsum);
    return err ? -2 : 0;
}
