// kernels.hpp -- host-side launchers of the gfx950 kernels (internal; the
// public boundary is include/hetattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hetattn {

struct RouteArgs {
    const float *u;
    int batch, n;
    int mode;       // 0 = top-rho, 1 = mean-std, 2 = fixed uniform lattice (u not read)
    int k;          // dense count (top-rho, uniform)
    double c;       // mean-std coefficient
    uint8_t *mask;
    int32_t *dense_idx, *local_idx, *counts;
    double *thresh;
};

// Per-block random swap (random = 0), or per-block random routing (random =
// 1: the s0 tokens with the smallest draws are dense, mask_in not read):
// routes of blocks block0 .. block0 + n_blocks - 1, each [batch, n] (counts
// [batch, 2], thresh [batch]), back to back.
struct SwapArgs {
    int random;
    const uint8_t *mask_in;
    const double *thresh_in;  // copied into thresh when both are set
    int batch, n;
    int s0;                   // floor(r * n + 1/2), before the clamp to the set sizes
    uint32_t key0, key1;      // Philox key: seed low and high words
    uint32_t step, block0;
    uint8_t *mask;
    int32_t *dense_idx, *local_idx, *counts;
    double *thresh;           // may be null
};

struct AttnArgs {
    const void *q, *k, *v;
    void *o;
    const uint8_t *mask;
    const int32_t *dense_idx, *counts;
    int batch, n, heads, head_dim;
    int grid_t, grid_h, grid_w;
    int win_t, win_h, win_w;   // odd, requested
    int cut;                   // window border: 0 = shifted inside the grid, 1 = cut at it
    bool bf16;
    float scale;               // softmax scale (> 0)
    int max_dense;             // upper bound on any sample's dense count
    bool dense_exact;          // every sample has exactly max_dense dense tokens
    void *workspace;           // dense_workspace_bytes() bytes of device memory
    int cu_count;              // compute units of the device the launch runs on
    float *lse_out = nullptr;  // bf16, optional: each written row's LSE, [batch][heads][n], log2 units
};

// Grid and window of the local kernels and the backward pass (query tiles of
// tiles_y x tiles_x per frame).
struct LocalGeom {
    int T, Hg, Wg;     // grid
    int wt, wh, ww;    // requested (odd) window
    int lt, lh, lw;    // effective window lengths, min(w, extent)
    int tiles_y, tiles_x;
    int slot_row;      // SR: 16 or 32 column slots per box row
    int cut;           // window border: 0 = shifted inside the grid, 1 = cut at it
};

// Backward pass: gradients of the layer for dout = dL/dO, with the route held
// fixed.  lse and dsum are [batch, heads, n] fp32 workspace arrays.
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    void *dq, *dk, *dv;
    const uint8_t *mask;
    const int32_t *dense_idx, *counts;
    float *lse, *dsum;
    int batch, n, heads, head_dim;
    int grid_t, grid_h, grid_w;
    int win_t, win_h, win_w;
    int cut;
    bool bf16;
    float scale;
    int max_dense;     // upper bound on any sample's dense count
    bool dense_exact;  // every sample has exactly max_dense dense tokens
    void *lse_part;    // dense_lse_workspace_bytes(kBwdMaxLseGroups) bytes of device memory
    float *dk_part, *dv_part;  // [batch, n, heads, head_dim] fp32 local parts (bf16 path)
    int cu_count;      // persistent workgroups of the statistics kernel (<= kBwdMaxLseGroups)
    bool lse_given = false;  // bf16: lse holds the forward's row LSE; skip the statistics passes
};

// Largest effective window along w that the local kernel's key tiling holds.
constexpr int kLocalMaxWinW = 25;

// Device workspace of the dense kernel's stream-K pieces (fp32 partials).
size_t dense_workspace_bytes(int batch, int heads, int n, int head_dim, bool bf16, int cu_count);

// The allocation-free forward keeps the dense kernel's stream-K partials in a
// static device array sized for kNoAllocGroups persistent workgroups at
// head_dim 128 (the largest head size): 2 slots per workgroup of 256 queries
// x (128 partial outputs + running max + row sum) fp32 values, 67.6 MB.
constexpr int kNoAllocGroups = 256;
constexpr size_t kNoAllocScratchBytes = 2ull * kNoAllocGroups * (128 * 256 + 2 * 256) * sizeof(float);
// Device address of the current device's copy of that array (looked up once
// per device with hipGetSymbolAddress).
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_route(const RouteArgs &a, hipStream_t stream);

// Top-rho route over several workgroups per sample (route.hip): workgroup g
// holds tokens [kRouteMbChunk*g, kRouteMbChunk*(g+1)), and the groups of a
// sample exchange histograms, counts and candidate keys through a workspace
// of route_mb_stride(G) bytes per sample: two [G][kRouteMbBins / 2] arrays,
// [G] counts and [G][kRouteMbCandWords] candidate lists of 64-bit tagged
// words.  Samples of fewer than kRouteMbMinN
// tokens or of more than kRouteMbMaxGroups groups, and launches of more than
// kRouteMbMaxLaunch workgroups, keep the one-workgroup route.  The G
// workgroups of a sample wait for one another, so they must run at once: at
// most 128 of them (a CU holds two), and the samples' workgroups are
// dispatched in order, so a sample's are all placed once the samples before
// it are.
constexpr int kRouteMbChunk = 2048;
constexpr int kRouteMbMaxGroups = 128;
constexpr int kRouteMbMinN = 4 * kRouteMbChunk;
constexpr int kRouteMbBins = 2048;
constexpr int kRouteMbMaxLaunch = 1024;
constexpr int kRouteMbCandWords = kRouteMbChunk + 8;  // a count word, then up to a chunk of keys
inline int route_mb_groups(int n) { return (n + kRouteMbChunk - 1) / kRouteMbChunk; }
inline bool route_mb_applies(int mode, int n, int batch) {
    return mode == 0 && n >= kRouteMbMinN && route_mb_groups(n) <= kRouteMbMaxGroups &&
           (int64_t)batch * route_mb_groups(n) <= kRouteMbMaxLaunch;
}
inline size_t route_mb_stride(int groups) {
    const size_t bytes = (2ull * groups * (kRouteMbBins / 2) + groups + (size_t)groups * kRouteMbCandWords) * sizeof(uint64_t);
    return (bytes + 255) / 256 * 256;
}
// ws: batch * route_mb_stride(G) bytes, any contents; nonce: a value no
// earlier call on this workspace used.
hipError_t launch_route_mb(const RouteArgs &a, void *ws, uint32_t nonce, hipStream_t stream);
hipError_t launch_swap(const SwapArgs &a, int n_blocks, hipStream_t stream);
hipError_t launch_dense(const AttnArgs &a, hipStream_t stream);
// LSE of the dense rows (bf16 only) into lse[(b*heads + h)*n + token]; the
// workspace holds dense_lse_workspace_bytes(cu_count).
size_t dense_lse_workspace_bytes(int cu_count);
hipError_t launch_dense_lse(const AttnArgs &a, float *lse, hipStream_t stream);
hipError_t launch_local(const AttnArgs &a, hipStream_t stream);
// bf16 only: LSE of the local rows into lse[(b*heads + h)*n + token], and dQ
// of the local rows given that LSE and D = dO.O (dsum, same layout).
hipError_t launch_local_lse(const AttnArgs &a, float *lse, hipStream_t stream);
hipError_t launch_local_dq(const AttnArgs &a, const void *dout, const float *lse, const float *dsum, void *dq,
                           hipStream_t stream);
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
// The backward workspace holds the dense rows' partial statistics for at
// most this many persistent workgroups, so that its size does not depend on
// the device.
constexpr int kBwdMaxLseGroups = 1024;
size_t backward_workspace_bytes(int batch, int heads, int n, int head_dim, bool bf16);

}  // namespace hetattn
