// Exercises every entry point of include/hetattn.h on the host (launchers
// stubbed, see api_stubs.cpp) with valid and invalid arguments, under the
// host sanitizers.  Device pointers are fake addresses that only the stubs
// receive; nothing dereferences them.  Exits non-zero on the first check
// that fails.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "hetattn.h"
#include "kernels.hpp"

namespace stub {
extern int launches;
extern hetattn::RouteArgs route;
extern hetattn::AttnArgs attn;
extern hetattn::BwdArgs bwd;
extern int swap_blocks;
extern int route_mb_launches;
extern void *route_ws;
extern uint32_t route_nonce;
}  // namespace stub

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static het_attn_shape shape(int B, int H, int D, int T, int Hg, int Wg, int dtype = HET_BF16) {
    het_attn_shape s = {};
    s.batch = B; s.heads = H; s.head_dim = D;
    s.grid_t = T; s.grid_h = Hg; s.grid_w = Wg;
    s.win_t = 3; s.win_h = 7; s.win_w = 7;
    s.dtype = dtype; s.scale = 0.0f; s.border = HET_BORDER_SHIFT;
    return s;
}

static void *fake(uintptr_t gib) { return (void *)(gib << 30); }

int main() {
    CHECK(het_attn_abi_version() == HETATTN_ABI_VERSION);
    for (int st = -1; st < 7; ++st) CHECK(het_status_string(st) != nullptr);

    het_attn_shape s = shape(1, 12, 128, 21, 30, 52);
    const int N = 21 * 30 * 52;
    het_route r = {(uint8_t *)fake(1), (int32_t *)fake(2), (int32_t *)fake(3), (int32_t *)fake(4),
                   (double *)fake(5), -1};
    // route: top-rho count, rejects
    // top-rho at this size runs over several workgroups and needs the workspace
    const size_t rws = het_attn_route_workspace_bytes(&s);
    CHECK(rws > 0);
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_WORKSPACE);
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, fake(7), rws - 1, nullptr) ==
          HET_ERR_WORKSPACE);
    int mb = stub::route_mb_launches;
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, fake(7), rws, nullptr) == HET_OK);
    CHECK(stub::route_mb_launches == mb + 1 && stub::route_ws == fake(7));
    CHECK(stub::route.k == (int)std::floor(0.2 * N + 0.5) && r.dense_count_host == stub::route.k);
    const uint32_t nonce0 = stub::route_nonce;
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, fake(7), rws, nullptr) == HET_OK);
    CHECK(stub::route_nonce == nonce0 + 1);
    // small samples keep the one-workgroup route and need no workspace
    het_attn_shape small = shape(2, 4, 64, 4, 8, 8);
    CHECK(het_attn_route_workspace_bytes(&small) == 0);
    mb = stub::route_mb_launches;
    CHECK(het_attn_route(&small, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_OK);
    CHECK(stub::route_mb_launches == mb);
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_MEAN_STD, 0.9, &r, nullptr, 0, nullptr) == HET_OK);
    CHECK(r.dense_count_host == -1);
    CHECK(het_attn_route(&s, nullptr, HET_UNIFORM, 0.3, &r, nullptr, 0, nullptr) == HET_OK);
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_TOP_RHO, 1.5, &r, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_route(&s, (const float *)fake(6), HET_MEAN_STD, NAN, &r, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_route(&s, nullptr, HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_route(&s, (const float *)fake(6), 7, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_route(nullptr, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    het_attn_shape bad = s;
    bad.win_w = 4;
    CHECK(het_attn_route(&bad, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    bad = s;
    bad.head_dim = 96;
    CHECK(het_attn_route(&bad, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_UNSUPPORTED);
    bad = s;
    bad.grid_t = 1 << 20;
    bad.grid_h = 1 << 20;
    CHECK(het_attn_route(&bad, (const float *)fake(6), HET_TOP_RHO, 0.2, &r, nullptr, 0, nullptr) == HET_ERR_UNSUPPORTED);

    // forward, halves, LSE and allocation-free forms
    r.dense_count_host = 6552;
    const size_t ws = het_attn_workspace_bytes(&s);
    CHECK(ws > 0);
    void *q = fake(10), *k = fake(11), *v = fake(12), *o = fake(13);
    CHECK(het_attn_forward(&s, q, k, v, &r, o, fake(20), ws, nullptr) == HET_OK);
    CHECK(stub::attn.max_dense == 6552 && stub::attn.dense_exact && stub::attn.cu_count == 256);
    CHECK(het_attn_forward(&s, q, k, v, &r, o, fake(20), ws - 1, nullptr) == HET_ERR_WORKSPACE);
    CHECK(het_attn_forward(&s, q, k, v, &r, o, nullptr, ws, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_dense(&s, q, k, v, &r, o, fake(20), ws, nullptr) == HET_OK);
    CHECK(het_attn_local(&s, q, k, v, &r, o, fake(20), ws, nullptr) == HET_OK);
    CHECK(het_attn_forward_noalloc(&s, q, k, v, &r, o, nullptr) == HET_OK);
    CHECK(stub::attn.workspace != nullptr && stub::attn.cu_count <= hetattn::kNoAllocGroups);
    CHECK(het_attn_forward_lse(&s, q, k, v, &r, o, (float *)fake(14), fake(20), ws, nullptr) == HET_OK);
    CHECK(het_attn_forward_lse(&s, q, k, v, &r, o, nullptr, fake(20), ws, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_forward_lse(&s, q, k, v, &r, o, (float *)q, fake(20), ws, nullptr) == HET_ERR_INVALID_ARG);
    het_attn_shape f32 = shape(1, 2, 64, 4, 8, 8, HET_F32);
    het_route rs = r;
    rs.dense_count_host = 64;
    CHECK(het_attn_forward_lse(&f32, q, k, v, &rs, o, (float *)fake(14), nullptr, 0, nullptr) == HET_ERR_UNSUPPORTED);
    rs.dense_count_host = 257;
    CHECK(het_attn_forward(&f32, q, k, v, &rs, o, nullptr, 0, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_forward(&s, nullptr, k, v, &r, o, fake(20), ws, nullptr) == HET_ERR_INVALID_ARG);

    // swap and random routing
    het_route out = {(uint8_t *)fake(30), (int32_t *)fake(31), (int32_t *)fake(32), (int32_t *)fake(33),
                     (double *)fake(34), -1};
    CHECK(het_attn_swap(&s, &r, 0.07, 7, 1, 0, 30, &out, nullptr) == HET_OK && stub::swap_blocks == 30);
    CHECK(het_attn_swap(&s, &r, 0.07, 7, 1, 0, 1, &r, nullptr) == HET_OK);  // in place
    CHECK(het_attn_swap(&s, &r, 0.07, 7, 1, 0, 2, &r, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_swap(&s, &r, -0.1, 7, 1, 0, 1, &out, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_swap(&s, &r, 0.07, 7, 1, 0, 0, &out, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_route_random(&s, 0.2, 9, 0, 0, 4, &out, nullptr) == HET_OK);
    CHECK(het_attn_route_random(&s, 2.0, 9, 0, 0, 4, &out, nullptr) == HET_ERR_INVALID_ARG);

    // backward
    const size_t bws = het_attn_backward_workspace_bytes(&s);
    CHECK(bws > 0);
    void *dout = fake(40), *dq = fake(41), *dk = fake(42), *dv = fake(43);
    CHECK(het_attn_backward(&s, q, k, v, &r, o, dout, dq, dk, dv, fake(50), bws, nullptr) == HET_OK);
    CHECK(!stub::bwd.lse_given && stub::bwd.dk_part != nullptr);
    CHECK(het_attn_backward_lse(&s, q, k, v, &r, o, dout, (const float *)fake(44), dq, dk, dv, fake(50), bws,
                                nullptr) == HET_OK);
    CHECK(stub::bwd.lse_given);
    CHECK(het_attn_backward(&s, q, k, v, &r, o, dout, dq, dk, dv, fake(50), bws - 1, nullptr) == HET_ERR_WORKSPACE);
    CHECK(het_attn_backward(&s, q, k, v, &r, o, dout, dq, dq, dv, fake(50), bws, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_backward(&s, q, k, v, &r, o, dout, q, dk, dv, fake(50), bws, nullptr) == HET_ERR_INVALID_ARG);
    CHECK(het_attn_backward_lse(&s, q, k, v, &r, o, dout, nullptr, dq, dk, dv, fake(50), bws, nullptr) ==
          HET_ERR_INVALID_ARG);

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("api driver ok (%d launches recorded)\n", stub::launches);
    return 0;
}
