// api.cpp -- the C ABI of include/hetattn.h: argument validation on the host,
// then launches on the caller's stream.  No allocation and no device-to-host
// traffic; the only state is the per-device address of the static scratch
// that het_attn_forward_noalloc uses (kept in dense.hip) and a counter of
// het_attn_route calls, whose value tags the words a call exchanges through
// the route workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "hetattn.h"
#include "kernels.hpp"

namespace {

using hetattn::AttnArgs;
using hetattn::RouteArgs;
using hetattn::SwapArgs;

struct Dims {
    int64_t B, N, H, D;
};

// Validates the shape; on success fills dims and the effective scale.
het_status check_shape(const het_attn_shape *s, Dims &d, float &scale) {
    if (!s) return HET_ERR_INVALID_ARG;
    if (s->batch <= 0 || s->heads <= 0 || s->head_dim <= 0) return HET_ERR_INVALID_ARG;
    if (s->grid_t <= 0 || s->grid_h <= 0 || s->grid_w <= 0) return HET_ERR_INVALID_ARG;
    if (s->win_t <= 0 || s->win_h <= 0 || s->win_w <= 0) return HET_ERR_INVALID_ARG;
    if (s->win_t % 2 == 0 || s->win_h % 2 == 0 || s->win_w % 2 == 0) return HET_ERR_INVALID_ARG;
    if (s->dtype != HET_BF16 && s->dtype != HET_F32) return HET_ERR_INVALID_ARG;
    if (std::isnan(s->scale) || std::isinf(s->scale)) return HET_ERR_INVALID_ARG;
    if (s->border != HET_BORDER_SHIFT && s->border != HET_BORDER_CUT) return HET_ERR_INVALID_ARG;
    if (s->head_dim != 64 && s->head_dim != 128) return HET_ERR_UNSUPPORTED;
    d.B = s->batch;
    d.H = s->heads;
    d.D = s->head_dim;
    d.N = (int64_t)s->grid_t * s->grid_h * s->grid_w;
    // Element offsets inside the kernels stay below 2^31 per tensor.
    if (d.N > INT32_MAX / 2 || d.B * d.N * d.H * d.D >= ((int64_t)1 << 31)) return HET_ERR_UNSUPPORTED;
    const int lw = s->win_w < s->grid_w ? s->win_w : s->grid_w;
    if (lw > hetattn::kLocalMaxWinW) return HET_ERR_UNSUPPORTED;
    scale = s->scale > 0.0f ? s->scale : 1.0f / std::sqrt((float)s->head_dim);
    return HET_OK;
}

// True when the byte ranges [p, p + n) and [q, q + m) share a byte.
bool overlaps(const void *p, size_t n, const void *q, size_t m) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + m && b < a + n;
}

// Dense count floor(rho*N + 1/2), clamped to [0, N] (rho in [0, 1]).
int rho_count(double rho, int64_t N) {
    double k = std::floor(rho * (double)N + 0.5);
    if (k < 0.0) k = 0.0;
    if (k > (double)N) k = (double)N;
    return (int)k;
}

// Checks the output routes of het_attn_swap / het_attn_route_random: n_blocks
// routes back to back, none overlapping the buffers the launch reads (the
// input mask and thresholds, NULL when absent); with n_blocks = 1 the output
// may be the input route itself.
het_status check_routes_out(const Dims &d, int32_t n_blocks, const het_route *out,
                            const uint8_t *in_mask, const double *in_thresh) {
    if (!out || !out->mask || !out->dense_idx || !out->local_idx || !out->counts) return HET_ERR_INVALID_ARG;
    if (n_blocks <= 0 || n_blocks > 65535) return HET_ERR_INVALID_ARG;
    const size_t routes = (size_t)n_blocks * (size_t)d.B;
    const size_t in_mask_bytes = (size_t)(d.B * d.N), in_th = (size_t)d.B * sizeof(double);
    auto hits_input = [&](const void *p, size_t bytes, bool may_be_mask, bool may_be_thresh) {
        if (in_mask && !(may_be_mask && p == in_mask) && overlaps(p, bytes, in_mask, in_mask_bytes))
            return true;
        return in_thresh && !(may_be_thresh && p == in_thresh) && overlaps(p, bytes, in_thresh, in_th);
    };
    const bool single = n_blocks == 1;
    if (hits_input(out->mask, routes * d.N, single, false) ||
        hits_input(out->dense_idx, routes * d.N * 4, false, false) ||
        hits_input(out->local_idx, routes * d.N * 4, false, false) ||
        hits_input(out->counts, routes * 8, false, false) ||
        (out->thresh && hits_input(out->thresh, routes * sizeof(double), false, single)))
        return HET_ERR_INVALID_ARG;
    return HET_OK;
}

// Compute units of the current device (0 if it cannot be queried).
int current_cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

}  // namespace

extern "C" {

int het_attn_abi_version(void) { return HETATTN_ABI_VERSION; }

const char *het_status_string(int status) {
    switch (status) {
        case HET_OK: return "ok";
        case HET_ERR_INVALID_ARG: return "invalid argument";
        case HET_ERR_UNSUPPORTED: return "unsupported shape";
        case HET_ERR_WORKSPACE: return "workspace too small";
        case HET_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t het_attn_workspace_bytes(const het_attn_shape *shape) {
    Dims d;
    float scale;
    if (check_shape(shape, d, scale) != HET_OK) return 0;
    const int cus = current_cu_count();
    if (cus <= 0) return 0;
    return hetattn::dense_workspace_bytes((int)d.B, (int)d.H, (int)d.N, (int)d.D, shape->dtype == HET_BF16, cus);
}

size_t het_attn_route_workspace_bytes(const het_attn_shape *shape) {
    Dims d;
    float scale;
    if (check_shape(shape, d, scale) != HET_OK) return 0;
    if (!hetattn::route_mb_applies(0, (int)d.N, (int)d.B)) return 0;
    return (size_t)d.B * hetattn::route_mb_stride(hetattn::route_mb_groups((int)d.N));
}

int het_attn_route(const het_attn_shape *shape, const float *u, int mode, double param,
                   het_route *out, void *workspace, size_t workspace_bytes, void *stream) {
    Dims d;
    float scale;
    const het_status st = check_shape(shape, d, scale);
    if (st != HET_OK) return st;
    if ((!u && mode != HET_UNIFORM) || !out || !out->mask || !out->dense_idx || !out->local_idx ||
        !out->counts || !out->thresh)
        return HET_ERR_INVALID_ARG;
    RouteArgs a;
    a.u = u;
    a.batch = (int)d.B;
    a.n = (int)d.N;
    a.mask = out->mask;
    a.dense_idx = out->dense_idx;
    a.local_idx = out->local_idx;
    a.counts = out->counts;
    a.thresh = out->thresh;
    a.c = 0.0;
    a.k = 0;
    if (mode == HET_TOP_RHO || mode == HET_UNIFORM) {
        if (!(param >= 0.0 && param <= 1.0)) return HET_ERR_INVALID_ARG;
        a.mode = mode == HET_TOP_RHO ? 0 : 2;
        a.k = rho_count(param, d.N);
    } else if (mode == HET_MEAN_STD) {
        if (!std::isfinite(param)) return HET_ERR_INVALID_ARG;
        a.mode = 1;
        a.c = param;
    } else {
        return HET_ERR_INVALID_ARG;
    }
    if (hetattn::route_mb_applies(a.mode, a.n, a.batch)) {
        const size_t need = (size_t)d.B * hetattn::route_mb_stride(hetattn::route_mb_groups(a.n));
        if (!workspace || workspace_bytes < need) return HET_ERR_WORKSPACE;
        // The call's number: the kernel tags the words it exchanges with a
        // hash of it, so words of the previous 2^29 calls never match.
        static std::atomic<uint32_t> calls{0};
        const uint32_t nonce = calls.fetch_add(1, std::memory_order_relaxed) + 1u;
        if (hetattn::launch_route_mb(a, workspace, nonce, (hipStream_t)stream) != hipSuccess) return HET_ERR_HIP;
    } else if (hetattn::launch_route(a, (hipStream_t)stream) != hipSuccess) {
        return HET_ERR_HIP;
    }
    out->dense_count_host = (a.mode == 1) ? -1 : a.k;
    return HET_OK;
}

int het_attn_swap(const het_attn_shape *shape, const het_route *in, double r, uint64_t seed,
                  uint32_t step, uint32_t block, int32_t n_blocks, het_route *out, void *stream) {
    Dims d;
    float scale;
    const het_status st = check_shape(shape, d, scale);
    if (st != HET_OK) return st;
    if (!in || !in->mask) return HET_ERR_INVALID_ARG;
    if (!(r >= 0.0 && r <= 1.0)) return HET_ERR_INVALID_ARG;
    if (in->dense_count_host < -1 || in->dense_count_host > d.N) return HET_ERR_INVALID_ARG;
    const het_status so = check_routes_out(d, n_blocks, out, in->mask, in->thresh);
    if (so != HET_OK) return so;
    SwapArgs a;
    a.random = 0;
    a.mask_in = in->mask;
    a.thresh_in = in->thresh;
    a.batch = (int)d.B;
    a.n = (int)d.N;
    a.s0 = (int)std::floor(r * (double)d.N + 0.5);
    a.key0 = (uint32_t)(seed & 0xffffffffu);
    a.key1 = (uint32_t)(seed >> 32);
    a.step = step;
    a.block0 = block;
    a.mask = out->mask;
    a.dense_idx = out->dense_idx;
    a.local_idx = out->local_idx;
    a.counts = out->counts;
    a.thresh = out->thresh;
    if (hetattn::launch_swap(a, n_blocks, (hipStream_t)stream) != hipSuccess) return HET_ERR_HIP;
    out->dense_count_host = in->dense_count_host;
    return HET_OK;
}

int het_attn_route_random(const het_attn_shape *shape, double rho, uint64_t seed, uint32_t step,
                          uint32_t block, int32_t n_blocks, het_route *out, void *stream) {
    Dims d;
    float scale;
    const het_status st = check_shape(shape, d, scale);
    if (st != HET_OK) return st;
    if (!(rho >= 0.0 && rho <= 1.0)) return HET_ERR_INVALID_ARG;
    const het_status so = check_routes_out(d, n_blocks, out, nullptr, nullptr);
    if (so != HET_OK) return so;
    SwapArgs a;
    a.random = 1;
    a.mask_in = nullptr;
    a.thresh_in = nullptr;
    a.batch = (int)d.B;
    a.n = (int)d.N;
    a.s0 = rho_count(rho, d.N);
    a.key0 = (uint32_t)(seed & 0xffffffffu);
    a.key1 = (uint32_t)(seed >> 32);
    a.step = step;
    a.block0 = block;
    a.mask = out->mask;
    a.dense_idx = out->dense_idx;
    a.local_idx = out->local_idx;
    a.counts = out->counts;
    a.thresh = out->thresh;
    if (hetattn::launch_swap(a, n_blocks, (hipStream_t)stream) != hipSuccess) return HET_ERR_HIP;
    out->dense_count_host = a.s0;
    return HET_OK;
}

}  // extern "C"

namespace {

enum Part { kBoth = 3, kDenseOnly = 1, kLocalOnly = 2 };

// no_alloc: run with the library's static scratch instead of the caller's
// workspace (het_attn_forward_noalloc); the dense kernel then takes at most
// kNoAllocGroups persistent workgroups, which that scratch holds.
int run_attention(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                  const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                  void *stream, int parts, float *lse = nullptr, bool no_alloc = false) {
    Dims d;
    float scale;
    const het_status st = check_shape(shape, d, scale);
    if (st != HET_OK) return st;
    if (!q || !k || !v || !o || !route || !route->mask || !route->dense_idx || !route->counts)
        return HET_ERR_INVALID_ARG;
    if (route->dense_count_host < -1 || route->dense_count_host > d.N) return HET_ERR_INVALID_ARG;
    if (lse && shape->dtype != HET_BF16) return HET_ERR_UNSUPPORTED;
    int cus = current_cu_count();
    if (cus <= 0) return HET_ERR_HIP;
    if (no_alloc) {
        if (cus > hetattn::kNoAllocGroups) cus = hetattn::kNoAllocGroups;
        if (hetattn::noalloc_scratch(&workspace) != hipSuccess) return HET_ERR_HIP;
        workspace_bytes = hetattn::kNoAllocScratchBytes;
    }
    const size_t need = hetattn::dense_workspace_bytes((int)d.B, (int)d.H, (int)d.N, (int)d.D,
                                                       shape->dtype == HET_BF16, cus);
    if (need > 0 && !workspace) return HET_ERR_INVALID_ARG;
    if (workspace_bytes < need) return HET_ERR_WORKSPACE;

    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.mask = route->mask;
    a.dense_idx = route->dense_idx;
    a.counts = route->counts;
    a.batch = (int)d.B;
    a.n = (int)d.N;
    a.heads = (int)d.H;
    a.head_dim = (int)d.D;
    a.grid_t = shape->grid_t;
    a.grid_h = shape->grid_h;
    a.grid_w = shape->grid_w;
    a.win_t = shape->win_t;
    a.win_h = shape->win_h;
    a.win_w = shape->win_w;
    a.cut = shape->border == HET_BORDER_CUT ? 1 : 0;
    a.bf16 = shape->dtype == HET_BF16;
    a.scale = scale;
    a.max_dense = route->dense_count_host >= 0 ? route->dense_count_host : (int)d.N;
    a.dense_exact = route->dense_count_host >= 0;
    a.workspace = workspace;
    a.cu_count = cus;
    if (lse) {
        const size_t lse_bytes = (size_t)(d.B * d.H * d.N) * sizeof(float);
        const size_t io_bytes = (size_t)(d.B * d.N * d.H * d.D) * 2;
        const void *ins[4] = {q, k, v, o};
        for (int j = 0; j < 4; ++j)
            if (overlaps(lse, lse_bytes, ins[j], io_bytes)) return HET_ERR_INVALID_ARG;
        a.lse_out = lse;
    }

    hipStream_t s = (hipStream_t)stream;
    // The two kernels write disjoint rows of o (Eq. 13 with m in {0, 1}).
    if ((parts & kLocalOnly) && hetattn::launch_local(a, s) != hipSuccess) return HET_ERR_HIP;
    if ((parts & kDenseOnly) && hetattn::launch_dense(a, s) != hipSuccess) return HET_ERR_HIP;
    return HET_OK;
}

}  // namespace

extern "C" {

int het_attn_forward(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                     const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                     void *stream) {
    return run_attention(shape, q, k, v, route, o, workspace, workspace_bytes, stream, kBoth);
}

int het_attn_dense(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                   const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                   void *stream) {
    return run_attention(shape, q, k, v, route, o, workspace, workspace_bytes, stream, kDenseOnly);
}

int het_attn_local(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                   const het_route *route, void *o, void *workspace, size_t workspace_bytes,
                   void *stream) {
    return run_attention(shape, q, k, v, route, o, workspace, workspace_bytes, stream, kLocalOnly);
}

int het_attn_forward_noalloc(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                             const het_route *route, void *o, void *stream) {
    return run_attention(shape, q, k, v, route, o, nullptr, 0, stream, kBoth, nullptr, true);
}

int het_attn_forward_lse(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                         const het_route *route, void *o, float *lse, void *workspace, size_t workspace_bytes,
                         void *stream) {
    if (!lse) return HET_ERR_INVALID_ARG;
    return run_attention(shape, q, k, v, route, o, workspace, workspace_bytes, stream, kBoth, lse);
}

}  // extern "C"

extern "C" {

size_t het_attn_backward_workspace_bytes(const het_attn_shape *shape) {
    Dims d;
    float scale;
    if (check_shape(shape, d, scale) != HET_OK) return 0;
    return hetattn::backward_workspace_bytes((int)d.B, (int)d.H, (int)d.N, (int)d.D, shape->dtype == HET_BF16);
}

// lse: the forward's row LSE (bf16 only), or null to compute it here.
static int run_backward(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                        const het_route *route, const void *o, const void *dout, const float *lse, void *dq,
                        void *dk, void *dv, void *workspace, size_t workspace_bytes, void *stream) {
    Dims d;
    float scale;
    const het_status st = check_shape(shape, d, scale);
    if (st != HET_OK) return st;
    if (!q || !k || !v || !o || !dout || !dq || !dk || !dv || !route || !route->mask ||
        !route->dense_idx || !route->counts)
        return HET_ERR_INVALID_ARG;
    if (route->dense_count_host < -1 || route->dense_count_host > d.N) return HET_ERR_INVALID_ARG;
    // The dK/dV kernel packs window ends of an axis into 16 bits.
    if (shape->grid_t > 32767 || shape->grid_h > 32767 || shape->grid_w > 32767) return HET_ERR_UNSUPPORTED;
    const size_t elem = shape->dtype == HET_BF16 ? 2 : 4;
    const size_t bytes = (size_t)(d.B * d.N * d.H * d.D) * elem;
    const void *ins[5] = {q, k, v, o, dout};
    void *outs[3] = {dq, dk, dv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], bytes, ins[j], bytes)) return HET_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], bytes, outs[j], bytes)) return HET_ERR_INVALID_ARG;
    }
    const size_t lse_bytes = (size_t)(d.B * d.H * d.N) * sizeof(float);
    if (lse) {
        if (shape->dtype != HET_BF16) return HET_ERR_UNSUPPORTED;
        for (int i = 0; i < 3; ++i)
            if (overlaps(outs[i], bytes, lse, lse_bytes)) return HET_ERR_INVALID_ARG;
    }
    const size_t need =
        hetattn::backward_workspace_bytes((int)d.B, (int)d.H, (int)d.N, (int)d.D, shape->dtype == HET_BF16);
    if (!workspace || workspace_bytes < need) return HET_ERR_WORKSPACE;
    const int cus = current_cu_count();
    if (cus <= 0) return HET_ERR_HIP;
    hetattn::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.mask = route->mask;
    a.dense_idx = route->dense_idx;
    a.counts = route->counts;
    a.lse = (float *)workspace;
    a.dsum = (float *)workspace + (size_t)(d.B * d.H * d.N);
    a.batch = (int)d.B;
    a.n = (int)d.N;
    a.heads = (int)d.H;
    a.head_dim = (int)d.D;
    a.grid_t = shape->grid_t;
    a.grid_h = shape->grid_h;
    a.grid_w = shape->grid_w;
    a.win_t = shape->win_t;
    a.win_h = shape->win_h;
    a.win_w = shape->win_w;
    a.cut = shape->border == HET_BORDER_CUT ? 1 : 0;
    a.bf16 = shape->dtype == HET_BF16;
    a.scale = scale;
    a.max_dense = route->dense_count_host >= 0 ? route->dense_count_host : (int)d.N;
    a.dense_exact = route->dense_count_host >= 0;
    a.lse_part = (float *)workspace + 2 * (size_t)(d.B * d.H * d.N);
    // bf16: the local dK and dV parts follow the statistics of the dense rows
    a.dk_part = a.dv_part = nullptr;
    if (shape->dtype == HET_BF16) {
        float *parts = (float *)((char *)a.lse_part + hetattn::dense_lse_workspace_bytes(hetattn::kBwdMaxLseGroups));
        a.dk_part = parts;
        a.dv_part = parts + (size_t)(d.B * d.N * d.H * d.D);
    }
    a.cu_count = cus < hetattn::kBwdMaxLseGroups ? cus : hetattn::kBwdMaxLseGroups;
    if (lse) {
        if (overlaps(workspace, need, lse, lse_bytes)) return HET_ERR_INVALID_ARG;
        a.lse = const_cast<float *>(lse);  // read only when given
        a.lse_given = true;
    }
    if (hetattn::launch_backward(a, (hipStream_t)stream) != hipSuccess) return HET_ERR_HIP;
    return HET_OK;
}

int het_attn_backward(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                      const het_route *route, const void *o, const void *dout, void *dq, void *dk,
                      void *dv, void *workspace, size_t workspace_bytes, void *stream) {
    return run_backward(shape, q, k, v, route, o, dout, nullptr, dq, dk, dv, workspace, workspace_bytes, stream);
}

int het_attn_backward_lse(const het_attn_shape *shape, const void *q, const void *k, const void *v,
                          const het_route *route, const void *o, const void *dout, const float *lse, void *dq,
                          void *dk, void *dv, void *workspace, size_t workspace_bytes, void *stream) {
    if (!lse) return HET_ERR_INVALID_ARG;
    return run_backward(shape, q, k, v, route, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, stream);
}

}  // extern "C"
