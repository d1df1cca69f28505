// route.hip -- threshold selection, routing mask and stable compaction.
//
// [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
// Video Diffusion" (HetA-DiT), §3.2.2 Eqs. 11-12.
//
// One 1024-thread workgroup per sample.  The route is computed once per
// denoising step and shared by every head and every transformer block, so it
// is latency- rather than bandwidth-bound (u of one sample is at most a few
// hundred KB and stays in L2 across the passes below).
//
// Top-rho: the K-th largest u is found by a 4-pass MSB-first radix select
// over order-preserving 32-bit keys (integers only, no rounding).  Tokens
// with a larger key are dense; of the tokens equal to the K-th key, the first
// E by index are dense, where E is what the select leaves over.
// Mean-std: mu and sigma in fp64 with a fixed reduction order, then
// dense iff u >= mu + c*sigma.
// Compaction: tiles of 1024 tokens in index order; a ballot-based block scan
// gives each token its slot, so both index lists come out ascending.
#include "common.hpp"
#include "kernels.hpp"

namespace hetattn {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Order-preserving key: larger u <-> larger key.  NaN reads as +inf and -0
// as +0, so equal values get equal keys.
__device__ __forceinline__ uint32_t rank_key(float x) {
    uint32_t f = __float_as_uint(x);
    if (x != x) f = 0x7f800000u;
    if (f == 0x80000000u) f = 0u;
    return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
    uint32_t f = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
    return __uint_as_float(f);
}

__device__ __forceinline__ double mapped_u(float x) {
    if (x != x) return __builtin_inf();
    return (x == 0.0f) ? 0.0 : (double)x;
}

// Exclusive prefix count of `flag` over the workgroup in thread order; the
// workgroup total goes to `total`.  Uses s_wave[kRouteWaves].
__device__ __forceinline__ int block_scan_flag(bool flag, int *s_wave, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) {
        const int c = s_wave[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + in_wave;
}

// Sum of one double per thread in a fixed order (butterfly in the wave, then
// the wave partials in wave order).
__device__ __forceinline__ double block_sum_f64(double x, double *s_part) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) s_part[wave] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) t += s_part[w];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
    const int b = blockIdx.x, tid = threadIdx.x, N = a.n;
    const float *ub = a.u + (size_t)b * N;
    __shared__ uint32_t hist[256];
    __shared__ int s_wave[kRouteWaves];
    __shared__ double s_part[kRouteWaves];
    __shared__ int s_sel[2];

    const bool top = (a.mode == 0);
    uint32_t tkey = 0xffffffffu;  // K = 0: no key is strictly larger, none equal is taken
    int take_equal = 0;
    double T = __builtin_inf();

    if (top && a.k > 0) {
        uint32_t prefix = 0, pmask = 0;
        int remaining = a.k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int i = tid; i < N; i += kRouteThreads) {
                const uint32_t key = rank_key(ub[i]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < 64) {
                // Wave 0 finds the digit d with count(> d) < remaining <= count(>= d).
                // Lane l owns digits 255-4l .. 252-4l (descending).
                int c0 = hist[255 - 4 * tid], c1 = hist[254 - 4 * tid];
                int c2 = hist[253 - 4 * tid], c3 = hist[252 - 4 * tid];
                int mine = c0 + c1 + c2 + c3;
                int incl = mine;  // inclusive scan over lanes (descending digits)
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    int y = __shfl_up(incl, off);
                    if (tid >= off) incl += y;
                }
                const int excl = incl - mine;
                if (excl < remaining && remaining <= incl) {
                    int d = 255 - 4 * tid, before = excl;
                    if (before + c0 < remaining) { before += c0; d--;
                        if (before + c1 < remaining) { before += c1; d--;
                            if (before + c2 < remaining) { before += c2; d--; } } }
                    s_sel[0] = d;
                    s_sel[1] = remaining - before;
                }
            }
            __syncthreads();
            prefix |= (uint32_t)s_sel[0] << shift;
            pmask |= 255u << shift;
            remaining = s_sel[1];
            __syncthreads();
        }
        tkey = prefix;
        take_equal = remaining;
        T = (double)key_to_float(tkey);
    } else if (!top) {
        double s = 0.0;
        for (int i = tid; i < N; i += kRouteThreads) s += mapped_u(ub[i]);
        const double mu = block_sum_f64(s, s_part) / (double)N;
        double ss = 0.0;
        for (int i = tid; i < N; i += kRouteThreads) {
            const double d = mapped_u(ub[i]) - mu;
            ss += d * d;
        }
        const double sigma = sqrt(block_sum_f64(ss, s_part) / (double)N);
        T = mu + a.c * sigma;
    }

    uint8_t *mask = a.mask + (size_t)b * N;
    int32_t *dense_idx = a.dense_idx + (size_t)b * N;
    int32_t *local_idx = a.local_idx + (size_t)b * N;
    int seen_equal = 0, n_dense = 0;
    for (int base = 0; base < N; base += kRouteThreads) {
        const int i = base + tid;
        const bool in = i < N;
        const float x = in ? ub[i] : 0.0f;
        bool dense;
        if (top) {
            const uint32_t key = rank_key(x);
            const bool eq = in && key == tkey;
            int eq_total;
            const int eq_rank = seen_equal + block_scan_flag(eq, s_wave, eq_total);
            seen_equal += eq_total;
            dense = in && (key > tkey || (eq && eq_rank < take_equal));
        } else {
            dense = in && !(mapped_u(x) < T);
        }
        int d_total;
        const int d_before = n_dense + block_scan_flag(dense, s_wave, d_total);
        if (in) {
            mask[i] = dense ? 0 : 1;
            if (dense) dense_idx[d_before] = i;
            else local_idx[i - d_before] = i;
        }
        n_dense += d_total;
    }
    for (int i = n_dense + tid; i < N; i += kRouteThreads) dense_idx[i] = -1;
    for (int i = (N - n_dense) + tid; i < N; i += kRouteThreads) local_idx[i] = -1;
    if (tid == 0) {
        a.counts[2 * b] = n_dense;
        a.counts[2 * b + 1] = N - n_dense;
        a.thresh[b] = T;
    }
}

hipError_t launch_route(const RouteArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(route_kernel, dim3(a.batch), dim3(kRouteThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hetattn
