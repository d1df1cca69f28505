/*
 * hetattn_oracle.h -- plain fp64 CPU oracle for uncertainty-routed
 * heterogeneous attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP path, and the HIP path never calls it.
 *
 * [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
 * Video Diffusion" (HetA-DiT, arXiv 2609.31050), full text.
 *
 * Conventions shared with the product boundary only through their written
 * definition (not through code):
 *   - tokens of sample b are flattened t-major: n = (t*Hg + y)*Wg + x;
 *   - Q, K, V, O are [B, N, heads, D] row-major;
 *   - mask[b*N + n] = 1 for a local ("certain") token, 0 for a dense one,
 *     as in [HetA §3.2.2 Eq. 12];
 *   - inputs arrive as float32 (bf16 values widen to float32 exactly) and every
 *     arithmetic step is done in double.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#ifndef HETATTN_ORACLE_H
#define HETATTN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Top-rho routing (the quantile reading of the threshold in [HetA §3.2.2
 * Eqs. 11-12]; rho is the dense fraction of [HetA §3.2.2, text of Eq. 14]).
 * K = floor(rho*N + 1/2) tokens per sample are dense: the K largest u, with
 * equal u ordered by ascending token index.  NaN counts as +inf and -0 as +0.
 * thresh[b] = the (mapped) u of the K-th ranked token, +inf when K = 0.
 * counts[2b] = K, counts[2b+1] = N - K.  dense_idx/local_idx rows are
 * ascending token indices; entries past the count are set to -1. */
int oracle_route_top_rho(const float *u, int B, int N, double rho,
                         unsigned char *mask, int *dense_idx, int *local_idx,
                         int *counts, double *thresh);

/* Mean-std routing, [HetA §3.2.2 Eqs. 11-12] as printed:
 * mu = mean(u), sigma = population standard deviation (1/N, two passes),
 * T = mu + c*sigma, and token i is local iff u_i < T (so dense iff not).
 * u values are mapped as in top-rho before use. */
int oracle_route_mean_std(const float *u, int B, int N, double c,
                          unsigned char *mask, int *dense_idx, int *local_idx,
                          int *counts, double *thresh);

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds of
 * the 4x32 Philox S-box on the counter ctr[4], with the key key[2] bumped by
 * the Weyl constants between rounds; the result goes to out[4]. */
void oracle_philox4x32_10(const unsigned int ctr[4], const unsigned int key[2], unsigned int out[4]);

/* Per-block random swap ([HetA §3.2.2, the text after Eq. 12: at each block
 * a subset of uncertain tokens is swapped with randomly selected certain
 * ones; App. B, Random Token Percentage and Table 8: the swap ratio r).
 * Reading: per sample b with K_b dense tokens in mask_in, S_b =
 * min(floor(r*N + 1/2), K_b, N - K_b) dense tokens become local and S_b local
 * tokens become dense, so K_b is unchanged.  Token i of sample b draws the
 * key philox4x32_10(ctr = {i, b, block, step}, key = {seed low 32 bits,
 * seed high 32 bits})[0]; in each of the two sets the S_b tokens with the
 * smallest key (equal keys: smaller token index first) are the ones swapped.
 * Writes the swapped route like oracle_route_top_rho (no thresh). */
int oracle_route_swap(const unsigned char *mask_in, int B, int N, double r,
                      unsigned long long seed, unsigned int step, unsigned int block,
                      unsigned char *mask, int *dense_idx, int *local_idx, int *counts);

/* The draws of oracle_route_swap for one sample: out[i] =
 * philox4x32_10({i, b, block, step}, {seed low, seed high})[0], i < N. */
void oracle_swap_draws(int N, unsigned int b, unsigned long long seed, unsigned int step,
                       unsigned int block, unsigned int *out);

/* Fixed uniform routing, the ablation router of [HetA §5.1, Routing
 * Strategy, Table 6], which picks tokens evenly over the token volume with a
 * fixed pattern.  The pattern is not given; reading: K = floor(rho*N + 1/2)
 * lattice points over the flattened (t-major) volume, the j-th dense token
 * being floor(j*N/K), j = 0 .. K-1; the same for every sample, step and
 * block.  Writes the route like oracle_route_top_rho (no thresh). */
int oracle_route_uniform(int B, int N, double rho, unsigned char *mask, int *dense_idx,
                         int *local_idx, int *counts);

/* Random routing, the ablation router of [HetA §5.1, Routing Strategy,
 * Table 6]: at every block an independent random subset of K =
 * floor(rho*N + 1/2) tokens is dense.  Reading: the K tokens with the smallest
 * draw of oracle_swap_draws(N, b, seed, step, block) (equal draws: smaller
 * index first).  Writes the route like oracle_route_top_rho (no thresh). */
int oracle_route_random(int B, int N, double rho, unsigned long long seed, unsigned int step,
                        unsigned int block, unsigned char *mask, int *dense_idx, int *local_idx,
                        int *counts);

/* The local neighbourhood of [HetA §3.1.1 Eq. 3] along one axis of extent S
 * for an odd window k at coordinate pos: length min(k, S), start shifted so
 * the box stays inside [0, S). */
int oracle_window_axis(int S, int k, int pos, int *start, int *len);

/* The other reading of the window border: the window of odd size k centred
 * on pos, cut at the border of [0, S): start = max(pos - (k-1)/2, 0),
 * end = min(pos + (k-1)/2 + 1, S), len = end - start (fewer keys near the
 * border). */
int oracle_window_axis_cut(int S, int k, int pos, int *start, int *len);

/* Heterogeneous attention [HetA §3.2.2 Eq. 13] for a list of rows.
 * rows[r] = b*N + n selects the token; out[r*heads*D + h*D + d] receives the
 * output of every head.  A token with mask 0 attends to all N tokens of its
 * sample ([HetA §3.1.1 Eq. 2]); a token with mask 1 attends to its 3D window
 * ([HetA §3.1.1 Eq. 3]), shifted inside the grid (border 0, oracle_window_axis)
 * or cut at its border (border 1, oracle_window_axis_cut).  Softmax is taken
 * over the key set with the given scale.  nthreads <= 0 uses the OpenMP
 * default. */
int oracle_attend_rows(const float *q, const float *k, const float *v,
                       int B, int heads, int D,
                       int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                       double scale, const unsigned char *mask,
                       const long *rows, long nrows, double *out, int nthreads);

/* Log-sum-exp of each listed row's scores over its key set (the same key
 * sets as oracle_attend_rows): out[r * heads + h] = log sum_j exp(scale *
 * q.k_j), natural log, double -- the log of the softmax's normaliser
 * ([HetA §3.1.1 Eqs. 2-3]), which the gradient of the layer reuses. */
int oracle_row_lse(const float *q, const float *k,
                   int B, int heads, int D,
                   int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                   double scale, const unsigned char *mask,
                   const long *rows, long nrows, double *out, int nthreads);

/* Same as oracle_attend_rows, but also returns the attention weights of one
 * (row, head) pair over all N tokens of the row's sample (zero outside the
 * key set).  Used to check support and normalisation. */
int oracle_attention_weights(const float *q, const float *k,
                             int B, int heads, int D,
                             int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                             double scale, const unsigned char *mask,
                             long row, int head, double *weights);

/* Backward of heterogeneous attention: given dout = dL/dO ([B, N, heads, D]),
 * the gradients dL/dQ, dL/dK, dL/dV (double, same layout) of the outputs of
 * oracle_attend_rows over all rows, with each row's key set and softmax as
 * there ([HetA §3.1.1 Eqs. 2-3, §3.2.2 Eq. 13] differentiated; the route is
 * a constant).  Per row: p = softmax(scale*q.k_j), dP_j = dout.v_j,
 * D = sum_j p_j dP_j, dS_j = p_j (dP_j - D); dQ = scale * sum_j dS_j k_j,
 * dK_j += scale * dS_j q, dV_j += p_j dout. */
int oracle_attend_backward(const float *q, const float *k, const float *v, const float *dout,
                           int B, int heads, int D,
                           int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                           double scale, const unsigned char *mask,
                           double *dq, double *dk, double *dv, int nthreads);

/* dL/dQ of the listed rows only (rows[r] = b*N + n), into dq[r*heads*D + h*D + d]. */
int oracle_attend_backward_dq_rows(const float *q, const float *k, const float *v,
                                   const float *dout, int B, int heads, int D,
                                   int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                                   double scale, const unsigned char *mask,
                                   const long *rows, long nrows, double *dq, int nthreads);

/* dL/dK and dL/dV of the listed key rows only (rows[r] = b*N + j, each listed
 * once) for the listed heads hsel[0 .. nh-1], into dk[(r*nh + i)*D + d] and
 * dv[(r*nh + i)*D + d]: the sums of oracle_attend_backward over every row n
 * of sample b whose key set holds token j (all dense rows; the local rows
 * whose 3D window contains j), each row's softmax taken over its whole key
 * set: p_nj = exp(s_nj - lse_n), dS_nj = p_nj (dP_nj - sum_j' p_nj' dP_nj'),
 * dK_j = scale * sum_n dS_nj q_n, dV_j = sum_n p_nj dout_n. */
int oracle_attend_backward_kv_rows(const float *q, const float *k, const float *v,
                                   const float *dout, int B, int heads, int D,
                                   int T, int Hg, int Wg, int wt, int wh, int ww, int border,
                                   double scale, const unsigned char *mask,
                                   const long *rows, long nrows, const int *hsel, int nh,
                                   double *dk, double *dv, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
