/*
 * hetattn.h -- C ABI of the uncertainty-routed heterogeneous attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
 * Video Diffusion" (HetA-DiT, arXiv 2609.31050), full text.
 *
 * The library computes one heterogeneous self-attention layer, [HetA §3.2.2
 * Eq. 13]: given Q, K, V of N spatio-temporal tokens ([HetA §3.1.1 Eq. 1])
 * and a per-token uncertainty u_i >= 0 ([HetA §3.2.1 Eq. 7]) predicted at
 * the previous denoising step ([HetA §3.2.2], mask reused at step tau-Delta;
 * [HetA §4] no extra pass at inference), it
 *   1. picks one threshold per sample ([HetA §3.2.2 Eq. 11]) and the binary
 *      mask m_i = 1[u_i < T] ([HetA §3.2.2 Eq. 12]): m = 1 is a "certain"
 *      token (local attention), m = 0 an "uncertain" one (dense attention);
 *   2. compacts the dense and the local token indices into ascending lists;
 *   3. computes dense softmax attention over all N keys for the dense tokens
 *      ([HetA §3.1.1 Eq. 2]) and softmax attention over a 3D window of the
 *      (T, H, W) latent grid for the local tokens ([HetA §3.1.1 Eq. 3]);
 *   4. writes both into one output: row i of O is the dense result when
 *      m_i = 0 and the local result when m_i = 1.
 *
 * Layout.  Tokens of a sample are flattened t-major: n = (t*grid_h + y)*grid_w
 * + x, N = grid_t*grid_h*grid_w.  Q, K, V and O are contiguous
 * [batch, N, heads, head_dim] arrays of one element type (bf16 or f32).
 *
 * Threshold forms.  HET_TOP_RHO makes exactly K = floor(rho*N + 1/2) tokens of
 * every sample dense (rho is the dense fraction of [HetA §3.2.2], text of
 * Eq. 14): the K largest u, equal u ranked by ascending token index.
 * HET_MEAN_STD is [HetA §3.2.2 Eq. 11] as printed: T = mu + c*sigma with the
 * mean and population standard deviation of the sample's u (fp64), dense iff
 * u_i >= T.  In both forms a NaN u counts as +inf and -0 as +0.
 * HET_UNIFORM is the fixed uniform router of the routing ablation ([HetA §5.1,
 * Routing Strategy, Table 6]), whose pattern the paper does not give: the K
 * dense tokens are the lattice floor(j*N/K), j = 0 .. K-1, over the flattened
 * volume, the same for every sample (u is not used; thresh is NaN).
 *
 * Window.  Along each axis of extent S, an odd window k covers min(k, S)
 * positions starting at clamp(pos - (k-1)/2, 0, S - min(k, S)): it is shifted,
 * not cut, at the grid border, so every local token sees the same number of
 * keys M (the constant M of [HetA §3.2.2 Eq. 14]).  A window at least as large
 * as the grid covers the whole axis.  shape->border = HET_BORDER_CUT selects
 * the other reading of the border: positions within (k-1)/2 of pos, cut to
 * [0, S), so tokens near the border see fewer keys.
 *
 * Memory.  All tensor arguments are device pointers owned by the caller; the
 * library allocates and frees nothing and keeps no state between calls,
 * except the static scratch array of het_attn_forward_noalloc (see there)
 * and a count of het_attn_route calls (which tags the words each call
 * exchanges through its workspace).
 * Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream) and
 * return without waiting for it.  `shape` and `route` themselves are host
 * structs read during the call only.
 *
 * Errors.  Argument errors are detected on the host before anything is
 * enqueued and returned as a status; nothing is written then.  A failed launch
 * returns HET_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation.  No call throws across the ABI.
 */
#ifndef HETATTN_H
#define HETATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HETATTN_ABI_VERSION 5

typedef enum {
    HET_OK = 0,
    HET_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, even window, bad param */
    HET_ERR_UNSUPPORTED = 2, /* head_dim not 64/128, window too wide, index overflow */
    HET_ERR_WORKSPACE = 3,   /* workspace smaller than het_attn_workspace_bytes() */
    HET_ERR_HIP = 4          /* a HIP launch failed */
} het_status;

typedef enum { HET_BF16 = 0, HET_F32 = 1 } het_dtype;

typedef enum {
    HET_TOP_RHO = 0,  /* param = rho in [0, 1] */
    HET_MEAN_STD = 1, /* param = c, finite */
    HET_UNIFORM = 2   /* param = rho in [0, 1]; u is not read (may be NULL) */
} het_thresh_mode;

typedef enum {
    HET_BORDER_SHIFT = 0, /* window shifted to stay inside the grid: M keys for every token */
    HET_BORDER_CUT = 1    /* window centred on the token and cut at the grid border */
} het_border;

typedef struct {
    int32_t batch;     /* B >= 1 */
    int32_t heads;     /* >= 1 */
    int32_t head_dim;  /* 64 or 128 */
    int32_t grid_t, grid_h, grid_w;  /* latent grid; N = product */
    int32_t win_t, win_h, win_w;     /* odd, >= 1 */
    int32_t dtype;     /* het_dtype of Q, K, V and O */
    float scale;       /* softmax scale; <= 0 selects 1/sqrt(head_dim) ([HetA §3.1.1 Eq. 2]) */
    int32_t border;    /* het_border of the local window (0 = HET_BORDER_SHIFT) */
} het_attn_shape;

typedef struct {
    uint8_t *mask;       /* [B, N]: 1 = local (m_i = 1), 0 = dense (m_i = 0) */
    int32_t *dense_idx;  /* [B, N]: dense tokens ascending, then -1 */
    int32_t *local_idx;  /* [B, N]: local tokens ascending, then -1 */
    int32_t *counts;     /* [B, 2]: (dense count, local count) per sample */
    double *thresh;      /* [B]: T_b (TOP_RHO: u of the K-th ranked token, +inf if K = 0) */
    int32_t dense_count_host; /* set by het_attn_route: K in TOP_RHO and UNIFORM modes, -1 in
                               * MEAN_STD mode;
                               * when >= 0 the attention calls size their launches by it, so
                               * it must equal every sample's dense count */
} het_route;

/* HETATTN_ABI_VERSION of the loaded library. */
int het_attn_abi_version(void);

/* Static description of a status code; never NULL. */
const char *het_status_string(int status);

/* Device workspace het_attn_forward needs for this shape, in bytes (may be 0).
 * Returns 0 for an invalid shape as well; het_attn_forward reports that. */
size_t het_attn_workspace_bytes(const het_attn_shape *shape);

/* Device workspace het_attn_route needs in HET_TOP_RHO mode for this shape,
 * in bytes (0: none; HET_MEAN_STD and HET_UNIFORM need none).  Samples of
 * 8192 to 262144 tokens (at most 1024 workgroups of 2048 tokens in all) are
 * routed by several workgroups per sample, which exchange histograms, counts
 * and candidate keys through it.  0 for an invalid shape too. */
size_t het_attn_route_workspace_bytes(const het_attn_shape *shape);

/* Threshold selection, mask and stable compaction ([HetA §3.2.2 Eqs. 11-12]).
 *   u      device, float32 [B, N], read only (not read, and may be NULL, for
 *          HET_UNIFORM).
 *   mode   het_thresh_mode; param = rho (TOP_RHO) or c (MEAN_STD).
 *   out    host struct of caller-owned device buffers, all written;
 *          out->dense_count_host is written on the host.
 *   workspace, workspace_bytes: device scratch of at least
 *          het_attn_route_workspace_bytes(shape) bytes (NULL allowed when
 *          that is 0), any contents: the call needs no clearing and leaves
 *          only scratch there.  Calls that may run at the same time need
 *          workspaces of their own.  Too small: HET_ERR_WORKSPACE.
 * Deterministic: the same u gives bit-identical outputs, whichever of the
 * two kernels routes the shape.  The workgroups of one sample wait for each
 * other's data; each wait is bounded, and counts[2b] = counts[2b+1] = -1
 * marks a sample whose workgroups were not all running at once within it or
 * whose exchanged data failed their consistency check (neither seen on an
 * otherwise idle device); its index lists are then not written. */
int het_attn_route(const het_attn_shape *shape, const float *u, int mode, double param,
                   het_route *out, void *workspace, size_t workspace_bytes, void *stream);

/* Random routing per block, the other router of the routing ablation
 * ([HetA §5.1, Routing Strategy, Table 6]): for each block l in
 * block .. block + n_blocks - 1 and sample b, the K = floor(rho*N + 1/2)
 * tokens with the smallest draw x_i are dense (equal draws: lower index
 * first), with x_i drawn as in het_attn_swap (Philox4x32-10 word 0 at counter
 * (i, b, l, step) under the 64-bit seed).
 *   rho       in [0, 1].
 *   n_blocks  1 .. 65535 routes, made by one launch.
 *   out       as in het_attn_swap: n_blocks routes back to back; thresh
 *             [n_blocks, B] is NaN (or NULL); out->dense_count_host = K.
 * Deterministic in (rho, seed, step, block). */
int het_attn_route_random(const het_attn_shape *shape, double rho, uint64_t seed, uint32_t step,
                          uint32_t block, int32_t n_blocks, het_route *out, void *stream);

/* Per-block random swap of a route ([HetA §3.2.2], the remark after Eq. 12:
 * at every block some uncertain tokens trade places with randomly chosen
 * certain ones; [HetA App. B], "Random Token Percentage", and Table 8 give
 * the swap ratio r).  For each block l in block .. block + n_blocks - 1 and
 * each sample b, with K_b the dense count of `in` and
 * S_b = min(floor(r*N + 1/2), K_b, N - K_b), the S_b dense tokens and the
 * S_b local tokens with the smallest draw x_i change sides (equal draws:
 * lower token index first), so the counts stay those of `in`.
 * x_i = output word 0 of Philox4x32-10 (Salmon et al., "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC 2011) at counter words (i, b, l, step)
 * under key words (seed & 0xffffffff, seed >> 32).
 *   in     host struct; in->mask [B, N] is read (0 = dense, else local);
 *          in->thresh, when it and out->thresh are set, is copied into every
 *          route; the other buffers of `in` are not read.
 *   r      in [0, 1]; r = 0 copies the route.
 *   n_blocks  1 .. 65535 routes, made by one launch.
 *   out    host struct of device buffers with n_blocks routes back to back:
 *          mask, dense_idx, local_idx [n_blocks, B, N], counts [n_blocks, B, 2],
 *          thresh [n_blocks, B] or NULL (NaN when in->thresh is NULL).  Route l
 *          starts at each pointer plus l times its per-route size.
 *          out->dense_count_host is set to in->dense_count_host.
 *          out must not overlap in->mask or in->thresh, except that with
 *          n_blocks = 1 out may be `in` itself (out->mask == in->mask, and
 *          out->thresh == in->thresh or either NULL): the swap in place.
 * Deterministic: the same in->mask, r, seed, step and block give bit-identical
 * routes. */
int het_attn_swap(const het_attn_shape *shape, const het_route *in, double r, uint64_t seed,
                  uint32_t step, uint32_t block, int32_t n_blocks, het_route *out, void *stream);

/* Heterogeneous attention ([HetA §3.2.2 Eq. 13]) with the route of
 * het_attn_route for the same shape.
 *   q, k, v  device, [B, N, heads, head_dim] of shape->dtype, read only.
 *   o        device, same layout and type; every row is written exactly once.
 *            Must not overlap q, k, v or the route buffers.
 *   workspace, workspace_bytes: device scratch of at least
 *            het_attn_workspace_bytes(shape) bytes (NULL allowed when 0).
 * Dense rows use fp32 accumulation and an fp32 online softmax; with bf16
 * inputs the probabilities are rounded to bf16 before the P*V product. */
int het_attn_forward(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                     const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                     void *stream);

/* het_attn_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same kernels and same results as het_attn_forward; the dense
 * kernel's scratch (the partial outputs of query tiles split between
 * workgroups) is taken from a static device array of the library instead of
 * a caller's workspace.  That array holds 67.6 MB on each device the library
 * runs on (kept until the process ends) and serves up to 256 persistent
 * workgroups at head_dim 128; on a device with more compute units the dense
 * kernel takes 256 workgroups.  The call allocates nothing; a shape whose
 * scratch would exceed the array returns HET_ERR_WORKSPACE (none does with
 * head_dim 64 or 128).  Every call on one device shares that device's
 * array and leaves its contents behind: calls that overlap in time on one
 * device (on different streams, or from different threads) race, and the
 * caller must order them.  Nothing in the array needs clearing between
 * calls.  q, k, v, route, o, stream: as het_attn_forward. */
int het_attn_forward_noalloc(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                             const het_route *route, void *o, void *stream);

/* The two halves of het_attn_forward, same arguments and rules.
 * het_attn_dense writes only the rows with m_i = 0 (dense attention over all
 * N keys, [HetA §3.1.1 Eq. 2]); het_attn_local writes only the rows with
 * m_i = 1 (the 3D window, [HetA §3.1.1 Eq. 3]).  Together they write every
 * row once, as het_attn_forward does ([HetA §3.2.2 Eq. 13]); since their
 * rows are disjoint, a caller may issue them on two streams that both wait
 * for the route. */
int het_attn_dense(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                   const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                   void *stream);
int het_attn_local(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                   const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                   void *stream);

/* het_attn_forward that also writes, for the gradient, the log-sum-exp of
 * every row's softmax ([HetA §3.1.1 Eqs. 2-3] over the row's key set, the
 * route held fixed as in het_attn_backward):
 *   lse[(b * heads + h) * N + i] = log2( sum_j 2^(scale * log2(e) * q_i.k_j) ),
 * j over the row's keys: all N for m_i = 0, the 3D window for m_i = 1.
 *   lse      device, B * heads * N fp32, written once per row; must not
 *            overlap q, k, v or o.  NULL is HET_ERR_INVALID_ARG.
 * The other arguments and rules are het_attn_forward's; o is identical to
 * het_attn_forward's.  bf16 only (fp32 inputs: HET_ERR_UNSUPPORTED). */
int het_attn_forward_lse(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                         const het_route *route, void *o, float *lse, void *workspace, size_t workspace_bytes,
                         void *stream);

/* Device workspace het_attn_backward needs for this shape, in bytes:
 * 2 * B * heads * N fp32 values (row statistics) plus 4 * 1024 * 256 fp32
 * values (partial statistics of the dense rows), and for bf16 inputs
 * 2 * B * N * heads * head_dim fp32 values more (the local queries' part of
 * dK and dV); 0 for an invalid shape. */
size_t het_attn_backward_workspace_bytes(const het_attn_shape *shape);

/* Backward pass of het_attn_forward with the route held fixed: the layer is
 * softmax attention over each row's key set ([HetA §3.1.1 Eqs. 2-3, §3.2.2
 * Eq. 13]), so for dout = dL/dO and P the softmax weights of a row,
 *   dP_j = dout.v_j, D = dout.o = sum_j P_j dP_j, dS_j = P_j (dP_j - D),
 *   dQ = scale * sum_j dS_j k_j, dK_j += scale * dS_j q, dV_j += P_j dout,
 * summed over every row whose key set holds key j.  The paper's second
 * training stage fine-tunes through this layer ([HetA §4, Training Setting]).
 *   q, k, v, route  as given to het_attn_forward (same shape).
 *   o        the output het_attn_forward wrote for them.
 *   dout     dL/dO, same layout and type.
 *   dq, dk, dv  device, same layout and type; every row is written once.
 *            Must not overlap the inputs or each other.
 *   workspace, workspace_bytes: at least het_attn_backward_workspace_bytes(shape).
 * Accumulation in fp32; with bf16 inputs P and dS are rounded to bf16 as
 * operands of the products.  Grid axes longer than 32767 are
 * HET_ERR_UNSUPPORTED. */
int het_attn_backward(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                      const het_route *route, const void *o, const void *dout, void *dq, void *dk,
                      void *dv, void *workspace, size_t workspace_bytes, void *stream);

/* het_attn_backward given the row LSE that het_attn_forward_lse wrote for the
 * same q, k, v and route (device, read only, must not overlap dq, dk, dv or
 * the workspace; NULL is HET_ERR_INVALID_ARG): the rows' statistics are not
 * computed again.  Same results as het_attn_backward, same workspace.
 * bf16 only (fp32 inputs: HET_ERR_UNSUPPORTED). */
int het_attn_backward_lse(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                          const het_route *route, const void *o, const void *dout, const float *lse, void *dq,
                          void *dk, void *dv, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* HETATTN_H */
