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

// MSB-first radix select over the keys of the members of one sample.
// Precondition: 1 <= k <= the number of members, and [lo, hi] is the range of
// the members' keys (workgroup-uniform).  Returns in tkey the k-th largest
// member key and in take_equal the number of members equal to tkey that the
// k largest hold, i.e. k minus the number of members above tkey.  The bits
// above the highest bit in which lo and hi differ are shared by every member
// and are skipped.  hcopy must be all zero on entry and is all zero on exit;
// member(j) and key_at(j) describe row j of this wave's range as in
// route_kernel.
template <int kPer, typename KeyAt, typename Member>
__device__ __forceinline__ void radix_select_largest(int k, uint32_t lo, uint32_t hi, int rows,
                                                     KeyAt &&key_at, Member &&member,
                                                     uint32_t *hcopy, uint32_t *hpart, int *s_sel,
                                                     uint32_t &tkey, int &take_equal) {
    const int tid = threadIdx.x, lane = tid & 63;
    int top_bit = (lo == hi) ? 0 : 32 - __builtin_clz(lo ^ hi);
    uint32_t pmask = (top_bit >= 32) ? 0u : ~((1u << top_bit) - 1u);
    uint32_t prefix = hi & pmask;
    int remaining = k;
    uint32_t *my_hist = hcopy + kHistStride * lane;
    while (top_bit > 0) {
        const int width = imin(8, top_bit);
        const int shift = top_bit - width;
        const uint32_t dmask = (1u << width) - 1u;
        for_rows<kPer>(rows, [&](int j) HET_INLINE {
            const uint32_t x = key_at(j);
            if (member(j) && (x & pmask) == prefix) atomicAdd(&my_hist[(x >> shift) & dmask], 1u);
        });
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
        pmask |= dmask << shift;
        remaining = s_sel[1];
        top_bit = shift;
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
    __shared__ int s_sel[2];

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
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            keys[j] = load_key(j);
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
            hpart, s_sel, tkey, take_equal);
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
    for (int i = n_dense + tid; i < N; i += kRouteThreads) dense_idx[i] = -1;
    for (int i = (N - n_dense) + tid; i < N; i += kRouteThreads) local_idx[i] = -1;
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
    __shared__ int s_sel[2];

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
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (j < rows) {
                keys[j] = draw_key(j);
                if (read_dense(j)) dbits |= 1ull << j;
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
        radix_select_largest<kPer>(s_out, dlo, dhi, rows, key_at, in_dense, hcopy, hpart, s_sel, tkd,
                                   ted);
    if (s_in > 0)
        radix_select_largest<kPer>(s_in, llo, lhi, rows, key_at, in_local, hcopy, hpart, s_sel, tkl,
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
    for (int i = n_dense + tid; i < N; i += kRouteThreads) dense_idx[i] = -1;
    for (int i = (N - n_dense) + tid; i < N; i += kRouteThreads) local_idx[i] = -1;
    if (tid == 0) {
        a.counts[2 * r] = n_dense;
        a.counts[2 * r + 1] = N - n_dense;
        if (a.thresh) a.thresh[r] = (!a.random && a.thresh_in) ? a.thresh_in[b] : __builtin_nan("");
    }
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
