// route.hip -- threshold selection, routing mask and stable compaction.
//
// [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
// Video Diffusion" (HetA-DiT), §3.2.2 Eqs. 11-12.
//
// One 1024-thread workgroup per sample.  The route is computed once per
// denoising step and shared by every head and every transformer block; u of
// one sample is at most a few hundred KB, so the kernel is latency-bound and
// is built to make one coalesced pass over memory in each direction: wave w
// owns the contiguous range of tokens [w*C, w*C + C), which it reads 64
// consecutive tokens at a time and keeps in registers (C = 64 * P with
// P = 8 .. 64, i.e. up to 65536 tokens; larger samples re-read u from memory,
// where it stays in L2).
//
// Top-rho: the K-th largest u is found by an MSB-first radix select over
// order-preserving 32-bit keys (integers only, no rounding).  The bits that
// every key of the sample shares (the common prefix of the smallest and the
// largest key) are skipped, so the first histogram already spreads over the
// sample's range.  Tokens with a larger key are dense; of the tokens equal to
// the K-th key, the first E by index are dense, where E is what the select
// leaves over.
// Mean-std: mu and sigma in fp64 with a fixed reduction order, then
// dense iff u >= mu + c*sigma.
// Compaction: ranks inside a wave come from ballots; one exclusive scan of
// the 16 per-wave counts places the waves, so both index lists come out
// ascending and every store of a wave goes to consecutive addresses.
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

// Inverse of rank_key on its image: the float a key stands for (NaN was
// already read as +inf and -0 as +0).
__device__ __forceinline__ float key_to_float(uint32_t key) {
    uint32_t f = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
    return __uint_as_float(f);
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

// Workgroup min and max of one key per thread.
__device__ __forceinline__ void block_min_max(uint32_t lo, uint32_t hi, uint32_t *s_w,
                                              uint32_t &out_lo, uint32_t &out_hi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
    }
    if (lane == 0) { s_w[wave] = lo; s_w[kRouteWaves + wave] = hi; }
    __syncthreads();
    lo = s_w[0];
    hi = s_w[kRouteWaves];
#pragma unroll
    for (int w = 1; w < kRouteWaves; ++w) {
        lo = min(lo, s_w[w]);
        hi = max(hi, s_w[kRouteWaves + w]);
    }
    __syncthreads();
    out_lo = lo;
    out_hi = hi;
}

// Calls f(j) for the first `rows` rows of this wave's range, fully unrolled
// when the range is a compile-time constant (so that keys[j] stays in
// registers).  `rows` is uniform over the wave.
template <int kPer, typename F>
__device__ __forceinline__ void for_rows(int rows, F &&f) {
    if constexpr (kPer > 0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (j < rows) f(j);
    } else {
        for (int j = 0; j < rows; ++j) f(j);
    }
}

// Exclusive prefix sums over the waves of two values per wave (taken from
// lane 0), in wave order; the workgroup totals go to tx, ty.
__device__ __forceinline__ void wave_excl_scan2(int x, int y, int *s_wave, int &bx, int &by,
                                                int &tx, int &ty) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { s_wave[wave] = x; s_wave[kRouteWaves + wave] = y; }
    __syncthreads();
    bx = by = tx = ty = 0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) {
        const int cx = s_wave[w], cy = s_wave[kRouteWaves + w];
        bx += (w < wave) ? cx : 0;
        by += (w < wave) ? cy : 0;
        tx += cx;
        ty += cy;
    }
    __syncthreads();
}

// p[0 .. n) = -1, by the whole workgroup: 16-byte stores from the first
// 16-byte boundary of p on (p is 4-byte aligned), single ones around them.
__device__ __forceinline__ void fill_minus_one(int32_t *p, int n) {
    const int tid = threadIdx.x;
    const int head = imin(n, (int)(((16u - ((uint32_t)(uintptr_t)p & 15u)) & 15u) >> 2));
    const int nv = (n - head) >> 2;
    for (int i = tid; i < head; i += kRouteThreads) p[i] = -1;
    i32x4 *pv = reinterpret_cast<i32x4 *>(p + head);
    for (int i = tid; i < nv; i += kRouteThreads) pv[i] = i32x4{-1, -1, -1, -1};
    for (int i = head + 4 * nv + tid; i < n; i += kRouteThreads) p[i] = -1;
}

// Number of lanes below this one whose bit is set in `bal`.
__device__ __forceinline__ int lanes_below(uint64_t bal) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// Histogram of the radix select: one copy of the 256 bins per lane index, so
// that the 64 lanes of one atomic never update the same word.  Copy c starts
// at word 257*c, which puts bin b of copy c in bank (b + c) mod 64: lanes
// whose keys fall in one bin (neighbouring tokens of a smooth u) also hit 64
// different banks.
constexpr int kHistStride = 257;
constexpr int kHistWords = 64 * kHistStride;
static_assert(kHistWords % 4 == 0, "the histogram is cleared in 16-byte words");

// Candidate list of the radix select: after the first digit pass, the member
// keys that carry the selected prefix are copied to LDS when at most
// kCandCap of them do, and the later passes read that list instead of every
// member's key (for a smooth u the selected digit holds a few hundred to a
// few thousand tokens; the register pass over all of them cost about 3 us).
constexpr int kCandCap = 8192;

// MSB-first radix select over the keys of the members of one sample.
// Precondition: 1 <= k <= the number of members, and [lo, hi] is the range of
// the members' keys (workgroup-uniform).  Returns in tkey the k-th largest
// member key and in take_equal the number of members equal to tkey that the
// k largest hold, i.e. k minus the number of members above tkey.  The bits
// above the highest bit in which lo and hi differ are shared by every member
// and are skipped.  hcopy must be all zero on entry and is all zero on exit;
// member(j) and key_at(j) describe row j of this wave's range as in
// route_kernel.  cand holds kCandCap keys and s_sel three ints (LDS).
template <int kPer, typename KeyAt, typename Member>
__device__ __forceinline__ void radix_select_largest(int k, uint32_t lo, uint32_t hi, int rows,
                                                     KeyAt &&key_at, Member &&member,
                                                     uint32_t *hcopy, uint32_t *hpart, int *s_sel,
                                                     uint32_t *cand, uint32_t &tkey, int &take_equal) {
    const int tid = threadIdx.x, lane = tid & 63;
    int top_bit = (lo == hi) ? 0 : 32 - __builtin_clz(lo ^ hi);
    uint32_t pmask = (top_bit >= 32) ? 0u : ~((1u << top_bit) - 1u);
    uint32_t prefix = hi & pmask;
    int remaining = k;
    uint32_t *my_hist = hcopy + kHistStride * lane;
    int n_cand = -1;  // < 0: the passes read every member's key
    while (top_bit > 0) {
        const int width = imin(8, top_bit);
        const int shift = top_bit - width;
        const uint32_t dmask = (1u << width) - 1u;
        auto count = [&](uint32_t x) HET_INLINE {
            if ((x & pmask) == prefix) atomicAdd(&my_hist[(x >> shift) & dmask], 1u);
        };
        if (n_cand < 0) {
            for_rows<kPer>(rows, [&](int j) HET_INLINE {
                if (member(j)) count(key_at(j));
            });
        } else {
            for (int c = tid; c < n_cand; c += kRouteThreads) count(cand[c]);
        }
        __syncthreads();
        {
            // Thread t sums bin t%256 over copies 16*(t/256) .. +15 and
            // clears them for the next pass.
            const int bin = tid & 255, c0 = 16 * (tid >> 8);
            uint32_t sum = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                sum += hcopy[(c0 + c) * kHistStride + bin];
                hcopy[(c0 + c) * kHistStride + bin] = 0u;
            }
            hpart[tid] = sum;
        }
        __syncthreads();
        if (tid < 64) {
            // Wave 0 finds the digit d with count(> d) < remaining <= count(>= d).
            // Lane l owns digits 255-4l .. 252-4l (descending).
            auto bin_count = [&](int d) HET_INLINE -> int {
                return (int)(hpart[d] + hpart[256 + d] + hpart[512 + d] + hpart[768 + d]);
            };
            const int c0 = bin_count(255 - 4 * tid), c1 = bin_count(254 - 4 * tid);
            const int c2 = bin_count(253 - 4 * tid), c3 = bin_count(252 - 4 * tid);
            const int mine = c0 + c1 + c2 + c3;
            int incl = mine;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off);
                if (tid >= off) incl += y;
            }
            const int excl = incl - mine;
            if (excl < remaining && remaining <= incl) {
                int d = 255 - 4 * tid, before = excl, in_bin = c0;
                if (before + c0 < remaining) { before += c0; d--; in_bin = c1;
                    if (before + c1 < remaining) { before += c1; d--; in_bin = c2;
                        if (before + c2 < remaining) { before += c2; d--; in_bin = c3; } } }
                s_sel[0] = d;
                s_sel[1] = remaining - before;
                s_sel[2] = in_bin;  // members with the new prefix
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_sel[0] << shift;
        pmask |= dmask << shift;
        remaining = s_sel[1];
        top_bit = shift;
        const int in_bin = s_sel[2];
        if (n_cand < 0 && top_bit > 0 && in_bin <= kCandCap) {
            // Copy the members with the new prefix to the candidate list:
            // per row, the lowest matching lane reserves the row's run.
            __syncthreads();  // every thread has read s_sel
            if (tid == 0) s_sel[2] = 0;
            __syncthreads();
            for_rows<kPer>(rows, [&](int j) HET_INLINE {
                const uint32_t x = key_at(j);
                const bool m = member(j) && (x & pmask) == prefix;
                const uint64_t bal = __ballot(m);
                if (bal != 0ull) {
                    const int leader = __builtin_ctzll(bal);
                    int base = 0;
                    if (lane == leader) base = atomicAdd(&s_sel[2], __popcll(bal));
                    base = __shfl(base, leader);
                    if (m) cand[base + lanes_below(bal)] = x;
                }
            });
            __syncthreads();
            n_cand = in_bin;
        }
    }
    tkey = prefix;
    take_equal = remaining;
}

// kPer > 0: every lane holds kPer keys in registers (N <= 1024 * kPer).
// kPer == 0: per-wave ranges of ceil(N / 1024) rows of 64, re-read from u.
// kUniform: the fixed uniform lattice (mode 2), a separate instantiation so
// that its index arithmetic stays out of the threshold modes' code.
template <int kPer, bool kUniform>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
    const int b = blockIdx.x, tid = threadIdx.x, N = a.n;
    const int lane = tid & 63, wave = tid >> 6;
    const float *ub = a.u ? a.u + (size_t)b * N : nullptr;  // not read in the uniform mode
    __shared__ __attribute__((aligned(16))) uint32_t hcopy[kHistWords];
    __shared__ uint32_t hpart[4 * 256];
    __shared__ int s_wave[2 * kRouteWaves];
    __shared__ uint32_t s_mm[2 * kRouteWaves];
    __shared__ double s_part[kRouteWaves];
    __shared__ int s_sel[3];
    __shared__ uint32_t cand[kCandCap];

    // Row j of this wave is tokens w*C + 64*j + (0..63); `rows` rows hold
    // tokens below N.  Keys of tokens at or beyond N read as 0, which no
    // token's key equals (rank_key never returns 0).
    const int per = kPer > 0 ? kPer : (N + kRouteThreads - 1) / kRouteThreads;
    const int w0 = wave * per * 64;
    const int rows = imax(0, imin(per, (N - w0 + 63) >> 6));
    auto token = [&](int j) HET_INLINE { return w0 + 64 * j + lane; };
    constexpr bool uniform = kUniform;
    const bool top = !kUniform && a.mode == 0;
    auto load_key = [&](int j) HET_INLINE -> uint32_t {
        return (!uniform && token(j) < N) ? rank_key(ub[token(j)]) : 0u;
    };
    uint32_t lo = 0xffffffffu, hi = 0u;
    uint32_t keys[kPer > 0 ? kPer : 1];
    if constexpr (kPer > 0) {
        // Every lane loads (a clamped index past N), so the loads are in
        // flight together instead of one branch and wait each.
        float uv[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) uv[j] = uniform ? 0.0f : ub[imin(token(j), N - 1)];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            keys[j] = (!uniform && token(j) < N) ? rank_key(uv[j]) : 0u;
            lo = min(lo, keys[j] ? keys[j] : 0xffffffffu);
            hi = max(hi, keys[j]);
        }
    } else if (top) {
        for (int j = 0; j < rows; ++j) {
            const uint32_t k = load_key(j);
            lo = min(lo, k ? k : 0xffffffffu);
            hi = max(hi, k);
        }
    }
    auto key_at = [&](int j) HET_INLINE -> uint32_t {
        if constexpr (kPer > 0) return keys[j];
        else return load_key(j);
    };

    uint32_t tkey = 0xffffffffu;  // K = 0: no key is larger, none equal is taken
    int take_equal = 0;
    double T = __builtin_inf();

    if (top && a.k > 0) {
        block_min_max(lo, hi, s_mm, lo, hi);
        for (int i = tid; i < kHistWords / 4; i += kRouteThreads)
            reinterpret_cast<u32x4 *>(hcopy)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        radix_select_largest<kPer>(
            a.k, lo, hi, rows, key_at, [&](int j) HET_INLINE { return key_at(j) != 0u; }, hcopy,
            hpart, s_sel, cand, tkey, take_equal);
        T = (double)key_to_float(tkey);
    } else if (!kUniform && a.mode == 1) {
        double s = 0.0;
        for_rows<kPer>(rows, [&](int j) HET_INLINE {
            if (token(j) < N) s += (double)key_to_float(key_at(j));
        });
        const double mu = block_sum_f64(s, s_part) / (double)N;
        double ss = 0.0;
        for_rows<kPer>(rows, [&](int j) HET_INLINE {
            if (token(j) < N) {
                const double d = (double)key_to_float(key_at(j)) - mu;
                ss += d * d;
            }
        });
        const double sigma = sqrt(block_sum_f64(ss, s_part) / (double)N);
        T = mu + a.c * sigma;
    }

    // Top-rho: token i is dense iff key > tkey, or key == tkey and fewer
    // than take_equal keys equal to tkey precede it.  Mean-std: iff
    // !(u < T).  Uniform lattice (dense tokens floor(j*N/K), j < K): token i
    // is dense iff the first lattice index at or after it, ceil(i*K/N), lands
    // on i, i.e. ceil(i*K/N)*N < (i+1)*K.  Ballot of the first kind of row j:
    auto above_row = [&](int j) HET_INLINE -> uint64_t {
        if constexpr (kUniform) {
            const uint64_t i = (uint64_t)token(j), K = (uint64_t)a.k, n = (uint64_t)N;
            return __ballot(token(j) < N && (i * K + n - 1) / n * n < (i + 1) * K);
        }
        const uint32_t key = key_at(j);
        if (top) return __ballot(key > tkey);
        return __ballot(token(j) < N && !((double)key_to_float(key) < T));
    };
    int n_gt = 0, n_eq = 0;
    for_rows<kPer>(rows, [&](int j) HET_INLINE {
        n_gt += __popcll(above_row(j));
        if (top) n_eq += __popcll(__ballot(key_at(j) == tkey));
    });
    int gt_before, eq_before, gt_total, eq_total;
    wave_excl_scan2(n_gt, n_eq, s_wave, gt_before, eq_before, gt_total, eq_total);
    const int n_dense = gt_total + imin(eq_total, take_equal);
    int d_seen = gt_before + imin(eq_before, take_equal);

    uint8_t *mask = a.mask + (size_t)b * N;
    int32_t *dense_idx = a.dense_idx + (size_t)b * N;
    int32_t *local_idx = a.local_idx + (size_t)b * N;
    int eq_run = eq_before;
    for_rows<kPer>(rows, [&](int j) HET_INLINE {
        uint64_t bal = above_row(j);
        if (top) {
            const uint64_t eq_bal = __ballot(key_at(j) == tkey);
            if (eq_bal != 0ull) {
                const bool eq = (eq_bal >> lane) & 1u;
                bal |= __ballot(eq && eq_run + lanes_below(eq_bal) < take_equal);
                eq_run += __popcll(eq_bal);
            }
        }
        const int i = token(j);
        const bool dn = (bal >> lane) & 1u;
        const int d = d_seen + lanes_below(bal);
        if (i < N) {
            mask[i] = dn ? 0 : 1;
            // One store per row: the dense lanes fill a run of dense_idx, the
            // others a run of local_idx.
            *(dn ? dense_idx + d : local_idx + (i - d)) = i;
        }
        d_seen += __popcll(bal);
    });
    fill_minus_one(dense_idx + n_dense, N - n_dense);
    fill_minus_one(local_idx + (N - n_dense), n_dense);
    if (tid == 0) {
        a.counts[2 * b] = n_dense;
        a.counts[2 * b + 1] = N - n_dense;
        a.thresh[b] = uniform ? __builtin_nan("") : T;
    }
}

// ---------------------------------------------------------------------------
// Per-block random swap ([HetA §3.2.2], the remark after Eq. 12; App. B,
// "Random Token Percentage", Table 8).  Starting from a route, S of the dense
// tokens become local and S of the local tokens become dense, with
// S = min(s0, K_b, N - K_b), so the counts do not change.  Token i of sample b
// draws x_i = word 0 of Philox4x32-10 at counter (i, b, block, step) under the
// 64-bit seed; in each set the S tokens with the smallest x (equal x: lower
// index first) are the ones that move.  Selecting the S smallest x is the
// radix select of the S largest ~x, whose tie rule (lower index first) is the
// route's, so the swap reuses the route's select and compaction unchanged.
// Grid (batch, n_blocks): workgroup (b, l) writes the route of block
// block0 + l for sample b; one launch makes the routes of every block of a
// step, which depend only on the step's route and the block index.

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011): ten rounds; in each, the words 0 and 2 are
// multiplied by two fixed odd constants into 64-bit products, the high halves
// are mixed with words 1 and 3 and the round key, and the key advances by two
// Weyl constants (the fractional parts of the golden ratio and of sqrt(3)).
// Only output word 0 is used, so the compiler drops the rest of the last round.
__device__ __forceinline__ uint32_t philox4x32_10_word0(uint32_t x0, uint32_t x1, uint32_t x2,
                                                        uint32_t x3, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;
    constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t hi0 = __umulhi(kMul0, x0), lo0 = kMul0 * x0;
        const uint32_t hi1 = __umulhi(kMul1, x2), lo1 = kMul1 * x2;
        x0 = hi1 ^ x1 ^ k0;
        x1 = lo1;
        x2 = hi0 ^ x3 ^ k1;
        x3 = lo0;
        k0 += kWeyl0;
        k1 += kWeyl1;
    }
    return x0;
}

// Exclusive prefix sums over the waves of kNV wave-uniform values, in wave
// order; the workgroup totals go to total[].
template <int kNV>
__device__ __forceinline__ void wave_excl_scan(const int (&x)[kNV], int *s_wave, int (&before)[kNV],
                                               int (&total)[kNV]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
#pragma unroll
        for (int v = 0; v < kNV; ++v) s_wave[v * kRouteWaves + wave] = x[v];
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < kNV; ++v) {
        int bv = 0, tv = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            const int c = s_wave[v * kRouteWaves + w];
            bv += (w < wave) ? c : 0;
            tv += c;
        }
        before[v] = bv;
        total[v] = tv;
    }
    __syncthreads();
}

// kPer as in route_kernel: > 0 keeps kPer draws and the set bits in
// registers, 0 draws again and re-reads mask_in in every pass.
template <int kPer>
__global__ __launch_bounds__(kRouteThreads) void swap_kernel(SwapArgs a) {
    const int b = blockIdx.x, l = blockIdx.y, tid = threadIdx.x, N = a.n;
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t blk = a.block0 + (uint32_t)l;
    const uint8_t *min_b = a.random ? nullptr : a.mask_in + (size_t)b * N;
    const size_t r = (size_t)l * a.batch + b;  // index of the route written
    __shared__ __attribute__((aligned(16))) uint32_t hcopy[kHistWords];
    __shared__ uint32_t hpart[4 * 256];
    __shared__ int s_wave[5 * kRouteWaves];
    __shared__ uint32_t s_mm[2 * kRouteWaves];
    __shared__ int s_sel[3];
    __shared__ uint32_t cand[kCandCap];

    const int per = kPer > 0 ? kPer : (N + kRouteThreads - 1) / kRouteThreads;
    const int w0 = wave * per * 64;
    const int rows = imax(0, imin(per, (N - w0 + 63) >> 6));
    auto token = [&](int j) HET_INLINE { return w0 + 64 * j + lane; };
    // Selection key of token i: ~x_i, so that the largest keys are the
    // smallest draws.
    auto draw_key = [&](int j) HET_INLINE -> uint32_t {
        return ~philox4x32_10_word0((uint32_t)token(j), (uint32_t)b, blk, a.step, a.key0, a.key1);
    };
    // Random routing starts from an all-local route.
    auto read_dense = [&](int j) HET_INLINE -> bool {
        return !a.random && token(j) < N && min_b[token(j)] == 0;
    };

    uint32_t keys[kPer > 0 ? kPer : 1];
    uint64_t dbits = 0;  // bit j: token(j) is in the dense set of the input route
    if constexpr (kPer > 0) {
        // The mask bytes are loaded by every lane (a clamped index past N),
        // all in flight together.
        uint8_t mbyte[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) mbyte[j] = 1;
        if (!a.random) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) mbyte[j] = min_b[imin(token(j), N - 1)];
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j < rows) {
                keys[j] = draw_key(j);
                if (token(j) < N && mbyte[j] == 0) dbits |= 1ull << j;
            } else {
                keys[j] = 0u;
            }
        }
    }
    auto key_at = [&](int j) HET_INLINE -> uint32_t {
        if constexpr (kPer > 0) return keys[j];
        else return draw_key(j);
    };
    auto in_dense = [&](int j) HET_INLINE -> bool {
        if constexpr (kPer > 0) return (dbits >> j) & 1u;
        else return read_dense(j);
    };
    auto in_local = [&](int j) HET_INLINE -> bool { return token(j) < N && !in_dense(j); };

    // Set sizes and the key range of each set.
    int nd_w = 0;
    uint32_t dlo = 0xffffffffu, dhi = 0u, llo = 0xffffffffu, lhi = 0u;
    for_rows<kPer>(rows, [&](int j) HET_INLINE {
        const uint32_t x = key_at(j);
        const bool dn = in_dense(j), lc = in_local(j);
        nd_w += __popcll(__ballot(dn));
        if (dn) { dlo = min(dlo, x); dhi = max(dhi, x); }
        if (lc) { llo = min(llo, x); lhi = max(lhi, x); }
    });
    block_min_max(dlo, dhi, s_mm, dlo, dhi);
    block_min_max(llo, lhi, s_mm, llo, lhi);
    int nd_total;
    {
        int x[1] = {nd_w}, bf[1], tt[1];
        wave_excl_scan<1>(x, s_wave, bf, tt);
        nd_total = tt[0];
    }
    // Tokens that leave the dense set (s_out) and the local set (s_in): S
    // each way for the swap; for random routing none leave the (empty) dense
    // set and the s0 smallest draws of all tokens come in.
    const int S = imin(a.s0, imin(nd_total, N - nd_total));
    const int s_out = a.random ? 0 : S, s_in = a.random ? imin(a.s0, N) : S;

    // A count of 0 leaves tkey = ~0 with nothing equal taken: no token moves.
    uint32_t tkd = 0xffffffffu, tkl = 0xffffffffu;
    int ted = 0, tel = 0;
    if (s_out > 0 || s_in > 0) {
        for (int i = tid; i < kHistWords / 4; i += kRouteThreads)
            reinterpret_cast<u32x4 *>(hcopy)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
    }
    if (s_out > 0)
        radix_select_largest<kPer>(s_out, dlo, dhi, rows, key_at, in_dense, hcopy, hpart, s_sel, cand, tkd,
                                   ted);
    if (s_in > 0)
        radix_select_largest<kPer>(s_in, llo, lhi, rows, key_at, in_local, hcopy, hpart, s_sel, cand, tkl,
                                   tel);

    // Per wave: dense-set size, and in each set the tokens above the select
    // key and those equal to it.
    int cnt[5] = {nd_w, 0, 0, 0, 0};
    for_rows<kPer>(rows, [&](int j) HET_INLINE {
        const uint32_t x = key_at(j);
        const bool dn = in_dense(j), lc = in_local(j);
        cnt[1] += __popcll(__ballot(dn && x > tkd));
        cnt[2] += __popcll(__ballot(dn && x == tkd));
        cnt[3] += __popcll(__ballot(lc && x > tkl));
        cnt[4] += __popcll(__ballot(lc && x == tkl));
    });
    int bef[5], tot[5];
    wave_excl_scan<5>(cnt, s_wave, bef, tot);
    // Dense tokens of the output before this wave: the input's, less those
    // that left, plus those that came.
    int d_seen = bef[0] - (bef[1] + imin(bef[2], ted)) + (bef[3] + imin(bef[4], tel));
    const int n_dense = nd_total - s_out + s_in;

    uint8_t *mask = a.mask + r * N;
    int32_t *dense_idx = a.dense_idx + r * N;
    int32_t *local_idx = a.local_idx + r * N;
    int eqd_run = bef[2], eql_run = bef[4];
    for_rows<kPer>(rows, [&](int j) HET_INLINE {
        const uint32_t x = key_at(j);
        const bool dn = in_dense(j), lc = in_local(j);
        uint64_t out_d = __ballot(dn && x > tkd);  // dense tokens that move
        uint64_t in_l = __ballot(lc && x > tkl);   // local tokens that move
        const uint64_t eqd = __ballot(dn && x == tkd), eql = __ballot(lc && x == tkl);
        if (eqd != 0ull) {
            out_d |= __ballot(((eqd >> lane) & 1u) && eqd_run + lanes_below(eqd) < ted);
            eqd_run += __popcll(eqd);
        }
        if (eql != 0ull) {
            in_l |= __ballot(((eql >> lane) & 1u) && eql_run + lanes_below(eql) < tel);
            eql_run += __popcll(eql);
        }
        const uint64_t bal = (__ballot(dn) & ~out_d) | in_l;
        const int i = token(j);
        const bool now_dense = (bal >> lane) & 1u;
        const int d = d_seen + lanes_below(bal);
        if (i < N) {
            mask[i] = now_dense ? 0 : 1;
            *(now_dense ? dense_idx + d : local_idx + (i - d)) = i;
        }
        d_seen += __popcll(bal);
    });
    fill_minus_one(dense_idx + n_dense, N - n_dense);
    fill_minus_one(local_idx + (N - n_dense), n_dense);
    if (tid == 0) {
        a.counts[2 * r] = n_dense;
        a.counts[2 * r + 1] = N - n_dense;
        if (a.thresh) a.thresh[r] = (!a.random && a.thresh_in) ? a.thresh_in[b] : __builtin_nan("");
    }
}

// ---------------------------------------------------------------------------
// Top-rho route over several workgroups per sample.  The one-workgroup route
// runs its steps (load, radix passes, counts, compaction) on one CU; for a
// sample of tens of thousands of tokens the same steps are spread over
// G = ceil(N / kRouteMbChunk) workgroups of one sample, which exchange data
// twice (four times when many keys tie with the K-th):
//   - workgroup g holds tokens [2048 g, 2048 g + 2048), 8 per lane
//     (wave w: rows 512 w + 64 j + lane, j < 8), as order-preserving keys;
//   - the K-th largest key is found by radix passes with fixed digits (key
//     bits 31..21, 20..10, 9..0).  In the first, each workgroup publishes the
//     histogram of the top digit over its keys, and every workgroup sums the
//     G histograms and picks the same digit, the bin that holds the K-th key;
//   - when that bin holds at most kMbCandCap keys, each workgroup publishes
//     its keys in the bin (in token order) and its count of keys above the
//     bin.  Every workgroup gathers the lists into LDS, runs the two other
//     passes there, and counts from them each workgroup's keys above and
//     equal to the K-th key;
//   - otherwise the two other passes exchange histograms as the first does
//     (over the keys that carry the prefix chosen so far), and each
//     workgroup then publishes its counts of keys above and equal to the
//     K-th key;
//   - from the counts of the workgroups before it, each workgroup places its
//     dense and local tokens exactly as the one-workgroup route does (keys
//     above are dense; of the keys equal to the K-th, the lowest indices
//     are, up to K in all).
// Exchange: every published 32-bit value travels with a 32-bit tag in one
// 64-bit atomic store at device scope, and a reader loads words (64-bit
// loads at device scope) until each carries the tag it expects.  The tag is
// a bijective 32-bit hash of (call number, exchange number), so a word left
// by an earlier exchange or by one of the previous 2^29 calls never passes,
// and no word needs to be ordered after another: no flag, no cache
// write-back or invalidation, and no clearing of the workspace between calls.
// What a reader assembles is also checked: the histogram of a pass holds as
// many keys as the digit chosen before it (N for the first), the candidate
// lists as many as the chosen bin, the counts add up to K, and the counts a
// workgroup derives for itself from the lists are its own.  Every wait is
// bounded (kMbSpinLimit rounds of loads).  A workgroup whose wait ran out or
// whose check failed writes no index (it cannot know where its tokens go),
// and if it is workgroup 0 the sample's counts read -1; the compaction's
// indices are clamped to the sample in any case.
constexpr int kMbThreads = 256;
constexpr int kMbWaves = kMbThreads / 64;
constexpr int kMbPer = kRouteMbChunk / kMbThreads;  // keys per lane
constexpr int kMbSpinLimit = 1 << 20;
constexpr int kMbSlotWords = kRouteMbBins / 2;  // one published histogram: two 16-bit counts a word
constexpr int kMbBatch = 16;                     // histograms whose words are loaded together
static_assert(kRouteMbBins == 8 * kMbThreads, "each thread sums eight bins");
static_assert(kRouteMbChunk < 65536, "a workgroup's counts fit 16 bits");
// The candidate path holds up to kMbCandCap keys in LDS (16 KiB), kMbCandPer
// loads in flight a lane.  A larger list costs more than the histogram
// exchange it saves: 5.7K candidates took 3 us longer than gathering a
// second histogram and then a list of a few keys.
constexpr int kMbCandPer = 16;
constexpr int kMbCandCap = kMbCandPer * kMbThreads;
static_assert(kRouteMbMaxGroups <= 256, "a workgroup number fits a byte");
static_assert(kMbCandCap <= 4 * kRouteMbBins, "the owner table fits the histogram's memory");

__device__ __forceinline__ uint64_t mb_tagged(uint32_t value, uint32_t tag) {
    return (uint64_t)value | ((uint64_t)tag << 32);
}
__device__ __forceinline__ void mb_put(uint64_t *p, uint32_t value, uint32_t tag) {
    __hip_atomic_store(p, mb_tagged(value, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t mb_get(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Tag of exchange e (0..7) of call number `call`: the finalizer of
// MurmurHash3 (Appleby), a bijection of 32-bit words, on 8*call + e.
__device__ __forceinline__ uint32_t mb_tag(uint32_t call, int e) {
    uint32_t x = (call << 3) | (uint32_t)e;
    x ^= x >> 16;
    x *= 0x85ebca6bu;
    x ^= x >> 13;
    x *= 0xc2b2ae35u;
    x ^= x >> 16;
    return x;
}

// Cache policy of the 16-byte exchange loads: device-scope coherent (sc1),
// as the compiler emits for the 64-bit atomic loads at that scope.
constexpr int kMbCoherent = 16;

// Wave 0 reads word 0 of each of the G slots (stride `stride` words) until
// all carry `tag`; returns false for every thread when the wait ran out (and
// does not wait once ok is false).  All threads of the workgroup call it.
__device__ __forceinline__ bool mb_wait_words(const uint64_t *slots, int stride, int G, uint32_t tag, bool ok,
                                              int *s_ok) {
    const int tid = threadIdx.x;
    ok = __syncthreads_and(ok);
    if (tid < 64) {
        bool seen = !ok;
        for (int it = 0; !seen && it < kMbSpinLimit; ++it) {
            const uint64_t w0 = tid < G ? mb_get(slots + (size_t)tid * stride) : mb_tagged(0u, tag);
            const uint64_t w1 = tid + 64 < G ? mb_get(slots + (size_t)(tid + 64) * stride) : mb_tagged(0u, tag);
            seen = __all((uint32_t)(w0 >> 32) == tag && (uint32_t)(w1 >> 32) == tag);
            if (!seen) __builtin_amdgcn_s_sleep(1);
        }
        if (tid == 0) *s_ok = seen;
    }
    __syncthreads();
    return ok && *s_ok != 0;
}

__global__ __launch_bounds__(kMbThreads) void route_mb_kernel(RouteArgs a, unsigned char *ws, size_t ws_stride,
                                                            int G, uint32_t nonce) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = a.n, K = a.k;
    unsigned char *wsb = ws + (size_t)b * ws_stride;
    uint64_t *hist = reinterpret_cast<uint64_t *>(wsb);  // [2][G][kMbSlotWords]
    uint64_t *cnt = hist + 2 * (size_t)G * kMbSlotWords;  // [G]
    uint64_t *cands = cnt + G;                            // [G][kRouteMbCandWords]
    __shared__ __attribute__((aligned(16))) uint32_t h[kRouteMbBins];
    __shared__ uint32_t cand[kMbCandCap];  // keys of the K-th key's 11-bit bin, workgroup by workgroup
    __shared__ int s_red[2 * kMbWaves];
    __shared__ int s_sel[4];
    __shared__ int s_blk[4];
    __shared__ int s_ok;
    __shared__ int s_off[kRouteMbMaxGroups + 1];  // candidates of the workgroups before each
    __shared__ int s_gt[kRouteMbMaxGroups], s_eq[kRouteMbMaxGroups];

    // Keys of tokens at or beyond N read as 0, which no token's key equals.
    // Every lane loads (a clamped index past N), so the eight loads are in
    // flight together instead of one branch and wait each.
    const float *ub = a.u + (size_t)b * N;
    const int w0 = g * kRouteMbChunk + wave * (kMbPer * 64);
    auto token = [&](int j) HET_INLINE { return w0 + 64 * j + lane; };
    float uv[kMbPer];
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) uv[j] = ub[imin(token(j), N - 1)];
    uint32_t keys[kMbPer];
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) keys[j] = token(j) < N ? rank_key(uv[j]) : 0u;

    bool ok = true;  // every wait ended with the expected words and every check held
    uint32_t prefix = 0u, pmask = 0u;
    int remaining = K;
    int members = N;  // keys that carry the prefix chosen so far

    // The next digit (bits shift .. shift + width of the key) from a
    // histogram of the members' digits, thread t holding bins 8t .. 8t+7 in
    // cs: the digit d with count(> d) < remaining <= count(>= d).  The
    // histogram must hold every member.
    auto choose_digit = [&](const int (&cs)[8], int shift, uint32_t dmask) HET_INLINE {
        int tot = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) tot += cs[i];
        // Members in bins >= 8t: suffix sum over the threads t .. 255.
        int suf = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_down(suf, off);
            if (lane + off < 64) suf += y;
        }
        if (lane == 0) s_red[wave] = suf;
        __syncthreads();
        int incl = suf;
        for (int w = wave + 1; w < kMbWaves; ++w) incl += s_red[w];
        const int excl = incl - tot;  // members in bins above 8t + 7
        if (tid == 0) s_sel[3] = incl;  // all the histogram's keys
        if (excl < remaining && remaining <= incl) {
            int i = 7, before = excl;
            while (i > 0 && before + cs[i] < remaining) before += cs[i--];
            s_sel[0] = 8 * tid + i;
            s_sel[1] = remaining - before;
            s_sel[2] = cs[i];
        }
        __syncthreads();
        ok = ok && s_sel[3] == members;
        prefix |= (uint32_t)s_sel[0] << shift;
        pmask |= dmask << shift;
        remaining = s_sel[1];
        members = s_sel[2];
        __syncthreads();  // s_red and s_sel are rewritten by the next choice
    };

    // Radix pass p over the histograms all G workgroups publish (exchange p).
    auto exchange_pass = [&](int p) HET_INLINE {
        const int shift = p == 0 ? 21 : (p == 1 ? 10 : 0);
        const uint32_t dmask = p == 2 ? 0x3ffu : 0x7ffu;
        const uint32_t tag = mb_tag(nonce, p);
        for (int i = tid; i < kRouteMbBins / 4; i += kMbThreads)
            reinterpret_cast<u32x4 *>(h)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMbPer; ++j) {
            const uint32_t x = keys[j];
            if (x != 0u && (x & pmask) == prefix) atomicAdd(&h[(x >> shift) & dmask], 1u);
        }
        __syncthreads();
        // Thread t publishes bins 8t .. 8t+7 as four words of two 16-bit
        // counts (a workgroup holds 2048 tokens).
        uint64_t *slots = hist + (size_t)(p & 1) * G * kMbSlotWords;
        {
            const u32x4 lo = reinterpret_cast<const u32x4 *>(h)[2 * tid];
            const u32x4 hi = reinterpret_cast<const u32x4 *>(h)[2 * tid + 1];
            uint64_t *mine = slots + (size_t)g * kMbSlotWords + 4 * tid;
            mb_put(mine + 0, lo[0] | (lo[1] << 16), tag);
            mb_put(mine + 1, lo[2] | (lo[3] << 16), tag);
            mb_put(mine + 2, hi[0] | (hi[1] << 16), tag);
            mb_put(mine + 3, hi[2] | (hi[3] << 16), tag);
        }
        // Wave 0 first waits until word 0 of every histogram carries the
        // tag (one word per workgroup, so the waiting costs little traffic).
        ok = mb_wait_words(slots, kMbSlotWords, G, tag, ok, &s_ok);
        // Thread t sums the same bins over the G histograms: 16-byte
        // device-scope loads of kMbBatch histograms at a time, loaded again
        // (rarely) while any of their words is stale.
        int cs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            slots, (short)0, (int)((size_t)G * kMbSlotWords * sizeof(uint64_t)), kBufferRsrcWord3);
        for (int g0 = 0; g0 < G; g0 += kMbBatch) {
            u32x4 v[kMbBatch][2];  // words 4t .. 4t+3 of histogram g0 + k: (value, tag) pairs
            bool fresh = !ok;     // after a wait ran out, do not wait again
            for (int it = 0; it < kMbSpinLimit; ++it) {
#pragma unroll
                for (int k = 0; k < kMbBatch; ++k)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int off = (int)(((size_t)(g0 + k) * kMbSlotWords + 4 * tid + 2 * hh) * sizeof(uint64_t));
                        v[k][hh] = g0 + k < G ? __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kMbCoherent)
                                              : u32x4{0u, tag, 0u, tag};
                    }
                bool all = true;
#pragma unroll
                for (int k = 0; k < kMbBatch; ++k)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) all = all && v[k][hh][1] == tag && v[k][hh][3] == tag;
                if (all || fresh) {
                    fresh = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            ok = ok && fresh;
#pragma unroll
            for (int k = 0; k < kMbBatch; ++k)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        cs[4 * hh + 2 * e] += (int)(v[k][hh][2 * e] & 0xffffu);
                        cs[4 * hh + 2 * e + 1] += (int)(v[k][hh][2 * e] >> 16);
                    }
        }
        choose_digit(cs, shift, dmask);
    };

    // Radix pass over the n candidates in LDS (no exchange).
    auto local_pass = [&](int n, int shift, uint32_t dmask) HET_INLINE {
        for (int i = tid; i < kRouteMbBins / 4; i += kMbThreads)
            reinterpret_cast<u32x4 *>(h)[i] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        for (int c = tid; c < n; c += kMbThreads) {
            const uint32_t x = cand[c];
            if ((x & pmask) == prefix) atomicAdd(&h[(x >> shift) & dmask], 1u);
        }
        __syncthreads();
        int cs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cs[i] = (int)h[8 * tid + i];
        choose_digit(cs, shift, dmask);
    };

    // After the histogram exchange of pass first_local - 1 chose a bin of at
    // most kMbCandCap keys: each workgroup publishes its keys in the bin (and
    // its count of keys above it), and every workgroup gathers the lists in
    // LDS, finishes the select there (passes first_local .. 2) and counts,
    // per workgroup, the keys above and equal to the K-th key.
    auto cand_select = [&](int first_local) HET_INLINE {
        const uint32_t ctag = mb_tag(nonce, 4);
        int nm = 0, na = 0;
#pragma unroll
        for (int j = 0; j < kMbPer; ++j) {
            nm += __popcll(__ballot(keys[j] != 0u && (keys[j] & pmask) == prefix));
            na += __popcll(__ballot((keys[j] & pmask) > prefix));
        }
        if (lane == 0) {
            s_red[wave] = nm;
            s_red[kMbWaves + wave] = na;
        }
        __syncthreads();
        int run = 0, nm_b = 0, na_b = 0;
#pragma unroll
        for (int w = 0; w < kMbWaves; ++w) {
            run += w < wave ? s_red[w] : 0;
            nm_b += s_red[w];
            na_b += s_red[kMbWaves + w];
        }
        __syncthreads();  // s_red is rewritten below
        // Word 0: (keys in the bin, keys above it); words 1.. the keys in
        // the bin in token order.
        uint64_t *slot = cands + (size_t)g * kRouteMbCandWords;
#pragma unroll
        for (int j = 0; j < kMbPer; ++j) {
            const bool m = keys[j] != 0u && (keys[j] & pmask) == prefix;
            const uint64_t bal = __ballot(m);
            if (m) mb_put(slot + 1 + run + lanes_below(bal), keys[j], ctag);
            run += __popcll(bal);
        }
        if (tid == 0) mb_put(slot, (uint32_t)nm_b | ((uint32_t)na_b << 16), ctag);
        ok = __syncthreads_and(ok);
        if (tid < 64) {
            // Wave 0: every count word, then where each list starts in
            // the concatenation of the lists.
            uint64_t c0 = 0ull, c1 = 0ull;
            bool seen = !ok;
            for (int it = 0; it < kMbSpinLimit; ++it) {
                c0 = tid < G ? mb_get(cands + (size_t)tid * kRouteMbCandWords) : mb_tagged(0u, ctag);
                c1 = tid + 64 < G ? mb_get(cands + (size_t)(tid + 64) * kRouteMbCandWords) : mb_tagged(0u, ctag);
                seen = seen || __all((uint32_t)(c0 >> 32) == ctag && (uint32_t)(c1 >> 32) == ctag);
                if (seen) break;
                __builtin_amdgcn_s_sleep(1);
            }
            const int n0 = tid < G ? (int)(c0 & 0xffffu) : 0;
            const int n1 = tid + 64 < G ? (int)(c1 & 0xffffu) : 0;
            int i0 = n0, i1 = n1;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y0 = __shfl_up(i0, off), y1 = __shfl_up(i1, off);
                if (tid >= off) {
                    i0 += y0;
                    i1 += y1;
                }
            }
            const int t0 = __shfl(i0, 63), t1 = __shfl(i1, 63);
            if (tid < G) {
                s_off[tid] = i0 - n0;
                s_gt[tid] = (int)((c0 >> 16) & 0xffffu);
            }
            if (tid + 64 < G) {
                s_off[tid + 64] = t0 + i1 - n1;
                s_gt[tid + 64] = (int)((c1 >> 16) & 0xffffu);
            }
            if (tid == 0) {
                s_off[G] = t0 + t1;
                s_ok = seen;
            }
        }
        __syncthreads();
        ok = ok && s_ok != 0 && s_off[G] == members;
        // Candidate c of the concatenation belongs to workgroup owner[c]
        // (the histogram's memory, free until the next pass).
        const int n_cand = ok ? members : 0;
        uint8_t *owner = reinterpret_cast<uint8_t *>(h);
        if (n_cand > 0)
            for (int w = wave; w < G; w += kMbWaves)
                for (int c = s_off[w] + lane; c < s_off[w + 1]; c += 64) owner[c] = (uint8_t)w;
        __syncthreads();
        // The lists -> LDS: every lane loads kMbCandPer words at once
        // (indices past the end load the last candidate again), and all
        // of them again while any is still stale.
        if (n_cand > 0) {
            u32x2 v[kMbCandPer];
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                cands, (short)0, (int)((size_t)G * kRouteMbCandWords * sizeof(uint64_t)), kBufferRsrcWord3);
            int off[kMbCandPer];
#pragma unroll
            for (int k = 0; k < kMbCandPer; ++k) {
                const int c = imin(k * kMbThreads + tid, n_cand - 1);
                const int w = owner[c];
                off[k] = (int)(((size_t)w * kRouteMbCandWords + 1 + (c - s_off[w])) * sizeof(uint64_t));
            }
            bool fresh = false;
            for (int it = 0; it < kMbSpinLimit; ++it) {
#pragma unroll
                for (int k = 0; k < kMbCandPer; ++k)
                    v[k] = __builtin_amdgcn_raw_buffer_load_b64(rs, off[k], 0, kMbCoherent);
                bool all = true;
#pragma unroll
                for (int k = 0; k < kMbCandPer; ++k) all = all && v[k][1] == ctag;
                if (all) {
                    fresh = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            ok = ok && fresh;
#pragma unroll
            for (int k = 0; k < kMbCandPer; ++k) {
                const int c = k * kMbThreads + tid;
                if (c < n_cand) cand[c] = v[k][0];
            }
        }
        ok = __syncthreads_and(ok);
        // The select's remaining digits on the candidates.
        const int n_sel = ok ? n_cand : 0;
#pragma unroll 1
        for (int q = first_local; q < 3; ++q) local_pass(n_sel, q == 1 ? 10 : 0, q == 1 ? 0x7ffu : 0x3ffu);
        // Each workgroup's keys above the K-th (above its bin, from its
        // count word, and in its list) and equal to it.
        if (n_sel > 0)
            for (int w = wave; w < G; w += kMbWaves) {
                int gt = 0, eq = 0;
                for (int c0 = s_off[w]; c0 < s_off[w + 1]; c0 += 64) {
                    const int c = c0 + lane;
                    const uint32_t x = c < s_off[w + 1] ? cand[c] : 0u;
                    gt += __popcll(__ballot(x > prefix));
                    eq += __popcll(__ballot(x == prefix));
                }
                if (lane == 0) {
                    s_gt[w] += gt;
                    s_eq[w] = eq;
                }
            }
        __syncthreads();
    };

    // Exchange 1 chooses the top 11 bits of the K-th key, and when more than
    // kMbCandCap keys carry them, exchange 2 the next 11; the keys that carry
    // the prefix chosen then are exchanged as candidates.  Only when more
    // than kMbCandCap keys share the K-th key's top 22 bits do a third
    // histogram exchange and one of the counts follow.
    bool by_cand = false;
    if (K > 0) {
        // One copy of the pass in the code (a loop kept rolled), so that the
        // kernel's instructions stay few.
        int p = 0;
#pragma unroll 1
        for (;;) {
            exchange_pass(p++);
            if (p == 3) break;
            if (members <= kMbCandCap) {  // workgroup-uniform (from LDS)
                by_cand = true;
                break;
            }
        }
        if (by_cand) cand_select(p);
    }
    // The K-th largest key and how many keys equal to it the K largest hold
    // (K = 0: no key is larger, none equal is taken).
    const uint32_t tkey = K > 0 ? prefix : 0xffffffffu;
    const int take_equal = K > 0 ? remaining : 0;

    // Counts of this wave and workgroup.
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        n_gt += __popcll(__ballot(keys[j] > tkey));
        n_eq += __popcll(__ballot(keys[j] == tkey));
    }
    if (lane == 0) {
        s_red[wave] = n_gt;
        s_red[kMbWaves + wave] = n_eq;
    }
    __syncthreads();
    int gt_w = 0, eq_w = 0, gt_b = 0, eq_b = 0;  // waves before this one; the workgroup
#pragma unroll
    for (int w = 0; w < kMbWaves; ++w) {
        gt_w += w < wave ? s_red[w] : 0;
        eq_w += w < wave ? s_red[kMbWaves + w] : 0;
        gt_b += s_red[w];
        eq_b += s_red[kMbWaves + w];
    }
    // Every workgroup's counts: from the candidate lists (exchange 2), else
    // from one more exchange.
    const uint32_t ctag = mb_tag(nonce, 3);
    if (!by_cand && tid == 0) mb_put(cnt + g, (uint32_t)gt_b | ((uint32_t)eq_b << 16), ctag);
    if (tid < 64) {
        // Wave 0: the counts of the workgroups before this one, and the totals.
        int x[2], y[2];
        if (by_cand) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int gg = tid + 64 * r;
                x[r] = gg < G ? s_gt[gg] : 0;
                y[r] = gg < G ? s_eq[gg] : 0;
            }
        } else {
            uint64_t c[2];
            bool fresh = !ok;
            for (int it = 0; it < kMbSpinLimit; ++it) {
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    c[r] = tid + 64 * r < G ? mb_get(cnt + tid + 64 * r) : mb_tagged(0u, ctag);
                if (fresh || ((uint32_t)(c[0] >> 32) == ctag && (uint32_t)(c[1] >> 32) == ctag)) {
                    fresh = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            ok = ok && fresh;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                x[r] = (int)(c[r] & 0xffffu);
                y[r] = (int)((c[r] >> 16) & 0xffffu);
            }
        }
        int gb = 0, eb = 0, gt = 0, et = 0;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int gg = tid + 64 * r;
            gb += gg < g ? x[r] : 0;
            eb += gg < g ? y[r] : 0;
            gt += x[r];
            et += y[r];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            gb += __shfl_xor(gb, off);
            eb += __shfl_xor(eb, off);
            gt += __shfl_xor(gt, off);
            et += __shfl_xor(et, off);
        }
        if (tid == 0) {
            s_blk[0] = gb;
            s_blk[1] = eb;
            s_blk[2] = gt;
            s_blk[3] = et;
        }
    }
    // Every wait of every thread ended with the expected words, and the
    // counts are those of K tokens (this workgroup's own among them).
    ok = __syncthreads_and(ok);
    ok = ok && s_blk[2] == K - take_equal && s_blk[3] >= take_equal && s_blk[2] + s_blk[3] <= N;
    if (by_cand) ok = ok && s_gt[g] == gt_b && s_eq[g] == eq_b;
    const int n_dense = s_blk[2] + imin(s_blk[3], take_equal);
    int eq_run = s_blk[1] + eq_w;
    int d_seen = s_blk[0] + gt_w + imin(eq_run, take_equal);

    uint8_t *mask = a.mask + (size_t)b * N;
    int32_t *dense_idx = a.dense_idx + (size_t)b * N;
    int32_t *local_idx = a.local_idx + (size_t)b * N;
    if (g == 0 && tid == 0) {
        a.counts[2 * b] = ok ? n_dense : -1;
        a.counts[2 * b + 1] = ok ? N - n_dense : -1;
        a.thresh[b] = K > 0 ? (double)key_to_float(tkey) : __builtin_inf();
    }
    // After a wait that ran out the other workgroups' counts are not known,
    // so no index may be trusted: nothing more is written.
    if (!ok) return;
#pragma unroll
    for (int j = 0; j < kMbPer; ++j) {
        uint64_t bal = __ballot(keys[j] > tkey);
        const uint64_t eq_bal = __ballot(keys[j] == tkey);
        if (eq_bal != 0ull) {
            const bool eq = (eq_bal >> lane) & 1u;
            bal |= __ballot(eq && eq_run + lanes_below(eq_bal) < take_equal);
            eq_run += __popcll(eq_bal);
        }
        const int i = token(j);
        const bool dn = (bal >> lane) & 1u;
        // d <= i by construction; the clamps keep every store inside the
        // sample whatever the exchanged data held.
        const int d = imin(imax(d_seen + lanes_below(bal), 0), imin(i, N - 1));
        if (i < N) {
            mask[i] = dn ? 0 : 1;
            *(dn ? dense_idx + d : local_idx + (i - d)) = i;
        }
        d_seen += __popcll(bal);
    }
    // -1 after the valid entries of both lists, over this workgroup's range.
    const int lo = g * kRouteMbChunk, hi = imin(N, lo + kRouteMbChunk);
    for (int i = lo + tid; i < hi; i += kMbThreads) {
        if (i >= n_dense) dense_idx[i] = -1;
        if (i >= N - n_dense) local_idx[i] = -1;
    }
}

hipError_t launch_route_mb(const RouteArgs &a, void *ws, uint32_t nonce, hipStream_t stream) {
    const int G = route_mb_groups(a.n);
    hipLaunchKernelGGL(route_mb_kernel, dim3(G, a.batch), dim3(kMbThreads), 0, stream, a,
                       static_cast<unsigned char *>(ws), route_mb_stride(G), G, nonce);
    return hipGetLastError();
}

template <bool kUniform>
static void launch_route_kind(const RouteArgs &a, hipStream_t stream) {
    const dim3 grid(a.batch), block(kRouteThreads);
    if (a.n <= 8 * kRouteThreads)
        hipLaunchKernelGGL((route_kernel<8, kUniform>), grid, block, 0, stream, a);
    else if (a.n <= 16 * kRouteThreads)
        hipLaunchKernelGGL((route_kernel<16, kUniform>), grid, block, 0, stream, a);
    else if (a.n <= 32 * kRouteThreads)
        hipLaunchKernelGGL((route_kernel<32, kUniform>), grid, block, 0, stream, a);
    else if (a.n <= 64 * kRouteThreads)
        hipLaunchKernelGGL((route_kernel<64, kUniform>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((route_kernel<0, kUniform>), grid, block, 0, stream, a);
}

hipError_t launch_route(const RouteArgs &a, hipStream_t stream) {
    if (a.mode == 2) launch_route_kind<true>(a, stream);
    else launch_route_kind<false>(a, stream);
    return hipGetLastError();
}

hipError_t launch_swap(const SwapArgs &a, int n_blocks, hipStream_t stream) {
    const dim3 grid(a.batch, n_blocks), block(kRouteThreads);
    if (a.n <= 8 * kRouteThreads)
        hipLaunchKernelGGL(swap_kernel<8>, grid, block, 0, stream, a);
    else if (a.n <= 16 * kRouteThreads)
        hipLaunchKernelGGL(swap_kernel<16>, grid, block, 0, stream, a);
    else if (a.n <= 32 * kRouteThreads)
        hipLaunchKernelGGL(swap_kernel<32>, grid, block, 0, stream, a);
    else if (a.n <= 64 * kRouteThreads)
        hipLaunchKernelGGL(swap_kernel<64>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(swap_kernel<0>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace hetattn
