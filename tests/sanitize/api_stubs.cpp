// Host-only stand-ins for the device side of libhetattn, so that api.cpp
// (the C ABI's argument checks and argument marshalling) can be built with
// the host AddressSanitizer and UndefinedBehaviorSanitizer and run without a
// GPU.  Every launcher records its arguments and returns hipSuccess; the
// device queries report one device with 256 compute units.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace stub {
int launches = 0;
hetattn::RouteArgs route;
hetattn::AttnArgs attn;
hetattn::BwdArgs bwd;
int swap_blocks = 0;
int route_mb_launches = 0;
void *route_ws = nullptr;
uint32_t route_nonce = 0;
}  // namespace stub

extern "C" hipError_t hipGetDevice(int *dev) {
    *dev = 0;
    return hipSuccess;
}

extern "C" hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int dev) {
    (void)dev;
    *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}

namespace hetattn {

size_t dense_workspace_bytes(int, int, int, int head_dim, bool bf16, int cu_count) {
    return bf16 ? 2ull * cu_count * ((size_t)head_dim * 256 + 512) * sizeof(float) : 0;
}
size_t dense_lse_workspace_bytes(int cu_count) { return 2ull * cu_count * 2 * 256 * sizeof(float); }
size_t backward_workspace_bytes(int batch, int heads, int n, int head_dim, bool bf16) {
    const size_t rows = (size_t)batch * heads * n;
    return 2 * rows * sizeof(float) + dense_lse_workspace_bytes(kBwdMaxLseGroups) +
           (bf16 ? 2 * rows * head_dim * sizeof(float) : 0);
}
hipError_t noalloc_scratch(void **ptr) {
    static unsigned char host_scratch[64];
    *ptr = host_scratch;
    return hipSuccess;
}
hipError_t launch_route(const RouteArgs &a, hipStream_t) {
    stub::route = a;
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_route_mb(const RouteArgs &a, void *ws, uint32_t nonce, hipStream_t) {
    stub::route = a;
    stub::route_ws = ws;
    stub::route_nonce = nonce;
    ++stub::route_mb_launches;
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_swap(const SwapArgs &, int n_blocks, hipStream_t) {
    stub::swap_blocks = n_blocks;
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_dense(const AttnArgs &a, hipStream_t) {
    stub::attn = a;
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_local(const AttnArgs &a, hipStream_t) {
    stub::attn = a;
    ++stub::launches;
    return hipSuccess;
}
hipError_t launch_backward(const BwdArgs &a, hipStream_t) {
    stub::bwd = a;
    ++stub::launches;
    return hipSuccess;
}

}  // namespace hetattn
