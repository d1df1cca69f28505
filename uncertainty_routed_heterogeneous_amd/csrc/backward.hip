// backward.hip -- backward pass of heterogeneous attention: dQ, dK, dV.
//
// [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
// Video Diffusion" (HetA-DiT).  With the route held fixed, the layer of
// §3.2.2 Eq. 13 is softmax attention over a per-row key set: all N tokens for
// a dense row (§3.1.1 Eq. 2), the 3D window for a local row (§3.1.1 Eq. 3).
// Its gradients, for L with dL/dO = dO, row i and key j of its set:
//   P_ij = exp(s_ij - LSE_i),  s_ij = scale * q_i.k_j,
//   D_i = dO_i . O_i = sum_j P_ij dP_ij,  dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),
//   dQ_i = scale * sum_j dS_ij k_j,  dK_j = scale * sum_i dS_ij q_i,
//   dV_j = sum_i P_ij dO_i.
//
// Four kernels; every workgroup owns its output rows (no atomics; every row
// of dQ, dK, dV is written once):
//   bwd_prep_kernel      D_i for every (token, head);
//   bwd_dq_dense_kernel  128 dense rows, 32 per wave: a first pass over the
//                        key blocks for LSE_i (written to the workspace for
//                        the dK/dV kernel), then S, P, dP, dS per block and
//                        dQ += dS K; the four waves share each 32-key block
//                        of K and V staged in LDS;
//   bwd_dq_kernel        the same for a 4x8 tile of local rows of one frame
//                        over its window box (one wave);
//   bwd_dkdv_kernel      128 keys (four 4x8 tiles of one frame, a wave each,
//                        K and V rows in registers): every dense query of the
//                        sample, then the local queries whose windows may
//                        hold these keys (per axis an interval of positions);
//                        the waves share each staged 32-query block;
//                        dV += P^T dO and dK += dS^T Q.
// Products run on the 32x32 MFMA of the element type (bf16 with fp32
// accumulation: P and dS are rounded to bf16 as operands; fp32: fp32 MFMA).
// Operands whose rows are read transposed (K for dQ, Q and dO for dK and dV)
// go through LDS.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace hetattn {

namespace {

constexpr int kBwdQY = 4, kBwdQX = 8;  // query / key tile of the local rows: 4 (h) x 8 (w)

template <typename T>
struct Frag {
    static constexpr bool kBf16 = std::is_same<T, __bf16>::value;
    using type = typename std::conditional<kBf16, bf16x8, float>::type;
    // MFMA k-steps over D: 16 bf16 or 2 fp32 per step.
    template <int D>
    static constexpr int steps() { return kBf16 ? D / 16 : D / 2; }
};

// Fragment c of a row for a 32x32 MFMA operand (A: the lane's row; B: the
// lane's column): bf16 elements 16c + 8*half .. +7, or fp32 element 2c + half.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag(const T *row, int c, bool ok) {
    const int half = (threadIdx.x & 63) >> 5;
    if constexpr (Frag<T>::kBf16) {
        return ok ? *(const bf16x8 *)(row + 16 * c + 8 * half) : bf16x8{};
    } else {
        return ok ? row[2 * c + half] : 0.0f;
    }
}

template <typename T>
__device__ __forceinline__ f32x16 mma(const typename Frag<T>::type &a, const typename Frag<T>::type &b,
                                      const f32x16 &c) {
    if constexpr (Frag<T>::kBf16) return mfma32_bf16(a, b, c);
    else return mfma32_f32(a, b, c);
}

// LDS slab of 32 rows of D elements (row pitch padded against bank
// conflicts, as in the local kernel's V slab).
template <typename T, int D>
struct Slab {
    static constexpr int kPitch = Frag<T>::kBf16 ? D + 16 : D + 4;
    static constexpr int kVec = 16 / sizeof(T);     // elements per 16-byte load
    static constexpr int kChunks = D / kVec;        // 16-byte chunks per row
    static constexpr int kStage = 32 * kChunks / 64; // chunks per lane
};

// Copies row `row_of(s)` (or zeros when !ok_of(s)) of each slot s < 32 into
// the slab; the first kThreads threads of the workgroup move the 16-byte
// chunks between them.
template <typename T, int D, int kThreads = 64, typename RowOf, typename OkOf>
__device__ __forceinline__ void stage_rows(T *slab, RowOf &&row_of, OkOf &&ok_of) {
    using S = Slab<T, D>;
    constexpr int kTotal = 32 * S::kChunks;
    static_assert(kTotal % kThreads == 0, "chunks per thread");
    const int tid = threadIdx.x % kThreads;
#pragma unroll
    for (int it = 0; it < kTotal / kThreads; ++it) {
        const int e = tid + kThreads * it, s = e / S::kChunks, ch = e % S::kChunks;
        const u32x4 val = ok_of(s) ? *(const u32x4 *)(row_of(s) + S::kVec * ch) : u32x4{0, 0, 0, 0};
        *(u32x4 *)(slab + s * S::kPitch + S::kVec * ch) = val;
    }
}

// Fragment c of slab row l%32 as a 32x32 MFMA operand (as load_frag).
template <typename T, int D>
__device__ __forceinline__ typename Frag<T>::type lds_frag(const T *slab, int c) {
    using S = Slab<T, D>;
    const int lane = threadIdx.x & 63, half = lane >> 5, row = lane & 31;
    if constexpr (Frag<T>::kBf16) return *(const bf16x8 *)(slab + row * S::kPitch + 16 * c + 8 * half);
    else return slab[row * S::kPitch + 2 * c + half];
}

// acc[db] += X^T B, X = the slab (32 slots x D, slot order of the B
// operand's k index), B = the 16 per-lane values w[i] of a C-layout block
// (lane: column l%32; w[i]: slot 8(i/4) + 4*half + i%4).  Result rows are
// dims db*32 + l%32.
template <typename T, int D>
__device__ __forceinline__ void mma_slab_t(const T *slab, const float (&w)[16], f32x16 (&acc)[D / 32]) {
    using S = Slab<T, D>;
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    if constexpr (Frag<T>::kBf16) {
        bf16x8 wf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 u;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) u[jj] = pack_bf16x2(w[8 * c + 2 * jj], w[8 * c + 2 * jj + 1]);
            wf[c] = __builtin_bit_cast(bf16x8, u);
        }
        const int gq = lane >> 4, j16 = lane & 15;
        const int key_off = 4 * half + (j16 >> 2), col_off = 16 * (gq & 1) + 4 * (j16 & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const __bf16 *base = (const __bf16 *)slab + (16 * c + key_off) * S::kPitch + db * 32 + col_off;
                const bf16x4 lo = lds_read_tr16((const HET_LDS void *)base);
                const bf16x4 hi = lds_read_tr16((const HET_LDS void *)(base + 8 * S::kPitch));
                acc[db] = mfma32_bf16(concat8(lo, hi), wf[c], acc[db]);
            }
    } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = ((const float *)slab)[(8 * (i / 4) + 4 * half + (i % 4)) * S::kPitch + db * 32 + col];
                acc[db] = mfma32_f32(a, w[i], acc[db]);
            }
    }
}

// Stores the C-layout accumulators (rows = dims) of this lane's column as one
// output row times `mul`.
template <typename T, int D>
__device__ __forceinline__ void store_row_t(T *row, const f32x16 (&acc)[D / 32], float mul) {
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = db * 32 + 8 * i4 + 4 * half;
            if constexpr (Frag<T>::kBf16) {
                u32x2 w;
                w[0] = pack_bf16x2(acc[db][4 * i4 + 0] * mul, acc[db][4 * i4 + 1] * mul);
                w[1] = pack_bf16x2(acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul);
                *(u32x2 *)((__bf16 *)row + d) = w;
            } else {
                f32x4 w = {acc[db][4 * i4 + 0] * mul, acc[db][4 * i4 + 1] * mul, acc[db][4 * i4 + 2] * mul,
                           acc[db][4 * i4 + 3] * mul};
                *(f32x4 *)((float *)row + d) = w;
            }
        }
}

// First and last position p of an axis whose window [lo(p), hi(p)) meets
// the positions [j0, j1] (both ends are non-decreasing in p, and a position
// lies in its own window, so p0 <= j0 and p1 >= j1).
__device__ __forceinline__ void inverse_window(int j0, int j1, int k, int len, int S, int cut, int &p0,
                                               int &p1) {
    p0 = imax(0, j0 - k);
    while (win_hi(p0, k, len, S, cut) <= j0) ++p0;
    p1 = imin(S - 1, j1 + k);
    while (win_lo(p1, k, len, S, cut) > j1) --p1;
}

}  // namespace

// D_i = dO_i . O_i for every (token, head), into dsum[(b*H + h)*N + n].
// A group of kChunks lanes takes one row, 16 bytes per lane.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const T *__restrict__ o, const T *__restrict__ dout,
                                                       float *__restrict__ dsum, long rows, int N, int H) {
    constexpr int kVec = 16 / sizeof(T), kChunks = D / kVec, kRowsPerWave = 64 / kChunks;
    const int lane = threadIdx.x & 63;
    const long r = ((long)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * kRowsPerWave + lane / kChunks;
    const int ch = lane % kChunks;
    float acc = 0.0f;
    if (r < rows) {
        const T *op = o + r * D + kVec * ch, *dp = dout + r * D + kVec * ch;
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc += (float)op[e] * (float)dp[e];
    }
#pragma unroll
    for (int off = kChunks / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (r < rows && ch == 0) {
        const long bn = r / H;  // rows are (b, n, h) in [B, N, heads, D] order
        const int h = (int)(r % H), n = (int)(bn % N), b = (int)(bn / N);
        dsum[((long)b * H + h) * N + n] = acc;
    }
}

constexpr int kBwdWaves = 4;  // waves of the dense-dQ and dK/dV workgroups

// dQ and LSE of 128 dense rows (consecutive entries of the dense index list):
// wave w takes 32 of them; the four waves share every 32-key block of K and
// V, staged once into LDS (row reads for S and dP, transposed reads of K for
// dQ += dS K).
template <typename T, int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_dq_dense_kernel(BwdArgs a, int n_units) {
    using F = Frag<T>;
    using S = Slab<T, D>;
    constexpr int kSteps = F::template steps<D>();
    __shared__ __attribute__((aligned(16))) T Ks[32 * S::kPitch];
    __shared__ __attribute__((aligned(16))) T Vs[32 * S::kPitch];

    const int unit = blockIdx.x;
    if (unit >= n_units) return;
    const int N = a.n, H = a.heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5, col = lane & 31;
    const T *q = (const T *)a.q, *k = (const T *)a.k, *v = (const T *)a.v, *dout = (const T *)a.dout;
    const size_t tok_stride = (size_t)H * D;
    const int groups = (a.max_dense + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
    const int grp = unit % groups, h = (unit / groups) % H, b = unit / groups / H;
    const int cnt = a.counts[2 * b];
    if (32 * kBwdWaves * grp >= cnt) return;  // the whole workgroup
    const int slot = 32 * kBwdWaves * grp + 32 * wave + col;
    const bool valid = slot < cnt;
    const int tok = valid ? a.dense_idx[(size_t)b * N + slot] : 0;
    const size_t sample = (size_t)b * N * tok_stride + (size_t)h * D;
    const size_t row_bh = ((size_t)b * H + h) * N;
    const float sl2 = a.scale * kLog2e;

    typename F::type qf[kSteps], df[kSteps];
#pragma unroll
    for (int c = 0; c < kSteps; ++c) {
        qf[c] = load_frag(q + sample + (size_t)tok * tok_stride, c, valid);
        df[c] = load_frag(dout + sample + (size_t)tok * tok_stride, c, valid);
    }
    const float dq_i = valid ? a.dsum[row_bh + tok] : 0.0f;
    const int n_blocks = (N + 31) / 32;
    auto in_block = [&](int kb, int i) HET_INLINE {
        return valid && 32 * kb + 8 * (i / 4) + 4 * half + (i % 4) < N;
    };
    // Staging of key block kb, software-pipelined: the rows of block kb+1
    // are loaded into registers while block kb is computed.
    constexpr int kThreads = 64 * kBwdWaves;
    constexpr int kPer = 32 * S::kChunks / kThreads;
    const int tid = threadIdx.x;
    u32x4 rk[kPer], rv[kPer];
    auto fetch = [&](int kb, bool with_v) HET_INLINE {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int e = tid + kThreads * it, key = 32 * kb + e / S::kChunks;
            const size_t off = sample + (size_t)imin(key, N - 1) * tok_stride + (e % S::kChunks) * S::kVec;
            rk[it] = key < N ? *(const u32x4 *)(k + off) : u32x4{0, 0, 0, 0};
            if (with_v) rv[it] = key < N ? *(const u32x4 *)(v + off) : u32x4{0, 0, 0, 0};
        }
    };
    auto store = [&](bool with_v) HET_INLINE {
#pragma unroll
        for (int it = 0; it < kPer; ++it) {
            const int e = tid + kThreads * it, o = (e / S::kChunks) * S::kPitch + (e % S::kChunks) * S::kVec;
            *(u32x4 *)(Ks + o) = rk[it];
            if (with_v) *(u32x4 *)(Vs + o) = rv[it];
        }
    };

    // Pass 1: LSE of every row (log2 units of scale * q.k).
    float m_run = -__builtin_inff(), l_run = 0.0f;
    fetch(0, false);
    for (int kb = 0; kb < n_blocks; ++kb) {
        __syncthreads();  // every wave is done with the previous block
        store(false);
        __syncthreads();
        if (kb + 1 < n_blocks) fetch(kb + 1, false);
        f32x16 sc = f32x16{};
#pragma unroll
        for (int c = 0; c < kSteps; ++c) sc = mma<T>(lds_frag<T, D>(Ks, c), qf[c], sc);
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (in_block(kb, i)) mx = fmaxf(mx, sc[i] * sl2);
        mx = half_pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        float part = 0.0f;
        if (m_new != -__builtin_inff()) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (in_block(kb, i)) part += __builtin_amdgcn_exp2f(sc[i] * sl2 - m_new);
            l_run = l_run * (m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new));
        }
        l_run += part;
        m_run = m_new;
    }
    const float lse2 = valid ? m_run + __builtin_log2f(half_pair_sum(l_run)) : 0.0f;
    if (valid && half == 0) a.lse[row_bh + tok] = lse2;

    // Pass 2: dQ^T += K^T dS^T.
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    fetch(0, true);
    for (int kb = 0; kb < n_blocks; ++kb) {
        __syncthreads();
        store(true);
        __syncthreads();
        if (kb + 1 < n_blocks) fetch(kb + 1, true);
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int c = 0; c < kSteps; ++c) {
            sc = mma<T>(lds_frag<T, D>(Ks, c), qf[c], sc);
            dp = mma<T>(lds_frag<T, D>(Vs, c), df[c], dp);
        }
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = in_block(kb, i) ? __builtin_amdgcn_exp2f(sc[i] * sl2 - lse2) : 0.0f;
            ds[i] = p * (dp[i] - dq_i);
        }
        mma_slab_t<T, D>(Ks, ds, acc);
    }
    if (valid) store_row_t<T, D>((T *)a.dq + sample + (size_t)tok * tok_stride, acc, a.scale);
}

// dQ of 32 query rows (kDense: 32 consecutive entries of the dense index
// list -- the one-wave form; the dense rows use bwd_dq_dense_kernel -- else
// a 4x8 tile of local rows of one frame), and LSE of those rows.
template <typename T, int D, bool kDense, int SR>
__global__ __launch_bounds__(64) void bwd_dq_kernel(BwdArgs a, LocalGeom g, int n_units) {
    using F = Frag<T>;
    using S = Slab<T, D>;
    constexpr int kSteps = F::template steps<D>();
    constexpr int rpb = 32 / SR;  // box rows per key block (local rows)
    __shared__ __attribute__((aligned(16))) T Ks[32 * S::kPitch];

    const int unit = blockIdx.x;
    if (unit >= n_units) return;
    const int N = a.n, H = a.heads;
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
    const T *q = (const T *)a.q, *k = (const T *)a.k, *v = (const T *)a.v, *dout = (const T *)a.dout;
    const size_t tok_stride = (size_t)H * D;

    // This lane's query and the key geometry of the unit.
    int b, h, tok = 0;
    bool valid;
    int t0 = 0, uy0 = 0, ux0 = 0, ny = 1, nx = 1, rows = 0, ylo = 0, yhi = 0, xlo = 0, xhi = 0;
    int n_blocks;
    if constexpr (kDense) {
        const int tiles = (a.max_dense + 31) / 32;
        const int qt = unit % tiles;
        h = (unit / tiles) % H;
        b = unit / tiles / H;
        const int cnt = a.counts[2 * b];
        if (32 * qt >= cnt) return;
        const int slot = 32 * qt + col;
        valid = slot < cnt;
        tok = valid ? a.dense_idx[(size_t)b * N + slot] : 0;
        n_blocks = (N + 31) / 32;
    } else {
        const int tx = unit % g.tiles_x;
        int rest = unit / g.tiles_x;
        const int ty = rest % g.tiles_y;
        rest /= g.tiles_y;
        const int t = rest % g.T;
        rest /= g.T;
        h = rest % H;
        b = rest / H;
        const int ybase = ty * kBwdQY, xbase = tx * kBwdQX;
        const int y = ybase + col / kBwdQX, x = xbase + col % kBwdQX;
        const bool in_grid = y < g.Hg && x < g.Wg;
        tok = in_grid ? (t * g.Hg + y) * g.Wg + x : 0;
        valid = in_grid && a.mask[(size_t)b * N + tok] != 0;
        if (!__any(valid)) return;
        t0 = win_lo(t, g.wt, g.lt, g.T, g.cut);
        const int nt = win_hi(t, g.wt, g.lt, g.T, g.cut) - t0;
        ylo = win_lo(imin(y, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut);
        yhi = win_hi(imin(y, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut);
        const int ylast = imin(ybase + kBwdQY - 1, g.Hg - 1), xlast = imin(xbase + kBwdQX - 1, g.Wg - 1);
        uy0 = win_lo(ybase, g.wh, g.lh, g.Hg, g.cut);
        ux0 = win_lo(xbase, g.ww, g.lw, g.Wg, g.cut);
        ny = win_hi(ylast, g.wh, g.lh, g.Hg, g.cut) - uy0;
        nx = win_hi(xlast, g.ww, g.lw, g.Wg, g.cut) - ux0;
        xlo = win_lo(imin(x, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut) - ux0;
        xhi = imin(win_hi(imin(x, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut) - ux0, nx);
        rows = nt * ny;
        n_blocks = (rows + rpb - 1) / rpb;
    }
    const size_t sample = (size_t)b * N * tok_stride + (size_t)h * D;

    // Key slot s (0..31) of block kb: its token (a clamped in-range address)
    // and whether it exists.
    auto slot_token = [&](int kb, int s) HET_INLINE -> int {
        if constexpr (kDense) {
            return imin(32 * kb + s, N - 1);
        } else {
            const int r = imin(kb * rpb + s / SR, rows - 1);
            return ((t0 + r / ny) * g.Hg + uy0 + r % ny) * g.Wg + ux0 + imin(s % SR, nx - 1);
        }
    };
    auto slot_ok = [&](int kb, int s) HET_INLINE -> bool {
        if constexpr (kDense) return 32 * kb + s < N;
        else return kb * rpb + s / SR < rows && s % SR < nx;
    };
    // Whether register i of a C-layout block (slot 8(i/4) + 4*half + i%4) is
    // a key of this lane's query.
    auto key_in = [&](int kb, int i) HET_INLINE -> bool {
        const int s = 8 * (i / 4) + 4 * half + (i % 4);
        if (!valid || !slot_ok(kb, s)) return false;
        if constexpr (kDense) {
            return true;
        } else {
            const int r = kb * rpb + s / SR, yy = uy0 + r % ny, xo = s % SR;
            return yy >= ylo && yy < yhi && xo >= xlo && xo < xhi;
        }
    };

    typename F::type qf[kSteps], df[kSteps];
#pragma unroll
    for (int c = 0; c < kSteps; ++c) {
        qf[c] = load_frag(q + sample + (size_t)tok * tok_stride, c, valid);
        df[c] = load_frag(dout + sample + (size_t)tok * tok_stride, c, valid);
    }
    const float sl2 = a.scale * kLog2e;
    const size_t row_bh = ((size_t)b * H + h) * N;
    const float dq_i = valid ? a.dsum[row_bh + tok] : 0.0f;

    // S^T of block kb (key slots x 32 queries), unscaled.
    auto scores = [&](int kb) HET_INLINE -> f32x16 {
        const int kt = slot_token(kb, col);
        const bool kok = slot_ok(kb, col);
        f32x16 s = f32x16{};
#pragma unroll
        for (int c = 0; c < kSteps; ++c) s = mma<T>(load_frag(k + sample + (size_t)kt * tok_stride, c, kok), qf[c], s);
        return s;
    };

    // Pass 1: LSE of every query (log2 units of scale * q.k).
    float m_run = -__builtin_inff(), l_run = 0.0f;
    for (int kb = 0; kb < n_blocks; ++kb) {
        const f32x16 s = scores(kb);
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (key_in(kb, i)) mx = fmaxf(mx, s[i] * sl2);
        mx = half_pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        float part = 0.0f;
        if (m_new != -__builtin_inff()) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key_in(kb, i)) part += __builtin_amdgcn_exp2f(s[i] * sl2 - m_new);
            l_run = l_run * (m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new));
        }
        l_run += part;
        m_run = m_new;
    }
    const float l_tot = half_pair_sum(l_run);
    const float lse2 = valid ? m_run + __builtin_log2f(l_tot) : 0.0f;
    if (valid && half == 0) a.lse[row_bh + tok] = lse2;

    // Pass 2: dQ^T += K^T dS^T.
    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    for (int kb = 0; kb < n_blocks; ++kb) {
        stage_rows<T, D>(
            Ks, [&](int s) HET_INLINE { return k + sample + (size_t)slot_token(kb, s) * tok_stride; },
            [&](int s) HET_INLINE { return slot_ok(kb, s); });
        const f32x16 s = scores(kb);
        const int kt = slot_token(kb, col);
        const bool kok = slot_ok(kb, col);
        f32x16 dp = f32x16{};
#pragma unroll
        for (int c = 0; c < kSteps; ++c) dp = mma<T>(load_frag(v + sample + (size_t)kt * tok_stride, c, kok), df[c], dp);
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = key_in(kb, i) ? __builtin_amdgcn_exp2f(s[i] * sl2 - lse2) : 0.0f;
            ds[i] = p * (dp[i] - dq_i);
        }
        __syncthreads();  // the K slab is visible to the whole wave
        mma_slab_t<T, D>(Ks, ds, acc);
        __syncthreads();  // slab free for the next block
    }
    if (valid) store_row_t<T, D>((T *)a.dq + sample + (size_t)tok * tok_stride, acc, a.scale);
}

// dK and dV of 128 keys: the 4x8 tiles (ty, 4*xg + w) of frame t, wave w
// taking one tile with its K and V rows in registers.  The four waves share
// every 32-query block: Q and dO rows, LSE, D and the window of each query,
// staged once into LDS (row reads for S and dP, transposed reads for dK and
// dV).
template <typename T, int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_dkdv_kernel(BwdArgs a, LocalGeom g, int x_groups,
                                                                  int n_units) {
    using F = Frag<T>;
    using S = Slab<T, D>;
    constexpr int kSteps = F::template steps<D>();
    constexpr int kThreads = 64 * kBwdWaves;
    __shared__ __attribute__((aligned(16))) T Qs[32 * S::kPitch];
    __shared__ __attribute__((aligned(16))) T Ds[32 * S::kPitch];
    // Per query slot: LSE (+inf for a slot without a query, so that P = 0)
    // and the window [lo, hi) per axis packed as lo | hi << 16 (t, y, x);
    // D apart.  One 16-byte record per slot is one LDS read per register.
    __shared__ __attribute__((aligned(16))) int4 s_rec[32];
    __shared__ float s_d[32];

    const int unit = blockIdx.x;
    if (unit >= n_units) return;
    const int N = a.n, H = a.heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
    const T *q = (const T *)a.q, *k = (const T *)a.k, *v = (const T *)a.v, *dout = (const T *)a.dout;
    const size_t tok_stride = (size_t)H * D;

    const int xg = unit % x_groups;
    int rest = unit / x_groups;
    const int ty = rest % g.tiles_y;
    rest /= g.tiles_y;
    const int t = rest % g.T;
    rest /= g.T;
    const int h = rest % H, b = rest / H;
    const int tx = kBwdWaves * xg + wave;
    const int ky = ty * kBwdQY + col / kBwdQX, kx = tx * kBwdQX + col % kBwdQX;
    const bool key_ok = tx < g.tiles_x && ky < g.Hg && kx < g.Wg;
    const int ktok = key_ok ? (t * g.Hg + ky) * g.Wg + kx : 0;
    const size_t sample = (size_t)b * N * tok_stride + (size_t)h * D;
    const size_t row_bh = ((size_t)b * H + h) * N;
    const float sl2 = a.scale * kLog2e;

    typename F::type kf[kSteps], vf[kSteps];
#pragma unroll
    for (int c = 0; c < kSteps; ++c) {
        kf[c] = load_frag(k + sample + (size_t)ktok * tok_stride, c, key_ok);
        vf[c] = load_frag(v + sample + (size_t)ktok * tok_stride, c, key_ok);
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = f32x16{};

    // Blocks of 32 query slots, software-pipelined: while block qb is
    // computed, the Q and dO rows (and LSE, D) of block qb+1 are in flight,
    // and the slot metadata of block qb+2 (its token, and whether it holds a
    // query) -- itself a global load for both query sources.  meta(qb, s,
    // tok, ok) gives slot s's token (any in-range token when it holds no
    // query); `windowed` queries see their window, the others every key.
    constexpr int kPer = 32 * S::kChunks / kThreads;  // staged chunks per thread and tensor
    auto chunk_slot = [&](int it) HET_INLINE { return (tid + kThreads * it) / S::kChunks; };
    auto chunk_off = [&](int it) HET_INLINE { return ((tid + kThreads * it) % S::kChunks) * S::kVec; };
    auto run = [&](int n_blocks, auto &&meta, auto windowed_tag) HET_INLINE {
        constexpr bool windowed = decltype(windowed_tag)::value;
        if (n_blocks <= 0) return;
        int mtok[kPer + 1];  // slots of this thread's chunks, then slot tid % 32
        bool mok[kPer + 1];
        u32x4 rq[kPer], rd[kPer];
        float r_lse = 0.0f, r_d = 0.0f;
        int own_tok = 0;
        bool own_ok = false;
        auto fetch_meta = [&](int qb) HET_INLINE {
#pragma unroll
            for (int it = 0; it < kPer; ++it) meta(qb, chunk_slot(it), mtok[it], mok[it]);
            meta(qb, tid & 31, mtok[kPer], mok[kPer]);
        };
        auto fetch_rows = [&]() HET_INLINE {
#pragma unroll
            for (int it = 0; it < kPer; ++it) {
                const size_t off = sample + (size_t)mtok[it] * tok_stride + chunk_off(it);
                rq[it] = mok[it] ? *(const u32x4 *)(q + off) : u32x4{0, 0, 0, 0};
                rd[it] = mok[it] ? *(const u32x4 *)(dout + off) : u32x4{0, 0, 0, 0};
            }
            own_tok = mtok[kPer];
            own_ok = mok[kPer];
            if (tid < 32) {
                r_lse = own_ok ? a.lse[row_bh + own_tok] : 0.0f;
                r_d = own_ok ? a.dsum[row_bh + own_tok] : 0.0f;
            }
        };
        fetch_meta(0);
        fetch_rows();
        if (n_blocks > 1) fetch_meta(1);
        for (int qb = 0; qb < n_blocks; ++qb) {
            __syncthreads();  // every wave is done with the previous block
#pragma unroll
            for (int it = 0; it < kPer; ++it) {
                const int sl = chunk_slot(it), o = chunk_off(it);
                *(u32x4 *)(Qs + sl * S::kPitch + o) = rq[it];
                *(u32x4 *)(Ds + sl * S::kPitch + o) = rd[it];
            }
            if (tid < 32) {
                int4 rec = {0, 0, 0, __float_as_int(own_ok ? r_lse : __builtin_inff())};
                if (windowed && own_ok) {
                    const int qtt = own_tok / (g.Hg * g.Wg), qy = (own_tok / g.Wg) % g.Hg, qx = own_tok % g.Wg;
                    rec.x = win_lo(qtt, g.wt, g.lt, g.T, g.cut) | (win_hi(qtt, g.wt, g.lt, g.T, g.cut) << 16);
                    rec.y = win_lo(qy, g.wh, g.lh, g.Hg, g.cut) | (win_hi(qy, g.wh, g.lh, g.Hg, g.cut) << 16);
                    rec.z = win_lo(qx, g.ww, g.lw, g.Wg, g.cut) | (win_hi(qx, g.ww, g.lw, g.Wg, g.cut) << 16);
                }
                s_rec[tid] = rec;
                s_d[tid] = r_d;
            }
            __syncthreads();  // slabs and per-query data visible
            if (qb + 1 < n_blocks) {
                fetch_rows();
                if (qb + 2 < n_blocks) fetch_meta(qb + 2);
            }
            // S and dP of the block: rows = query slots, columns = this wave's keys.
            f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int c = 0; c < kSteps; ++c) {
                sc = mma<T>(lds_frag<T, D>(Qs, c), kf[c], sc);
                dp = mma<T>(lds_frag<T, D>(Ds, c), vf[c], dp);
            }
            float p[16], ds[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qs = 8 * (i / 4) + 4 * half + (i % 4);
                const int4 rec = s_rec[qs];
                bool in = key_ok;
                if constexpr (windowed) {
                    auto inside = [](int c, int w) HET_INLINE { return c >= (w & 0xffff) && c < (w >> 16); };
                    in = in && inside(t, rec.x) && inside(ky, rec.y) && inside(kx, rec.z);
                }
                p[i] = in ? __builtin_amdgcn_exp2f(sc[i] * sl2 - __int_as_float(rec.w)) : 0.0f;
                ds[i] = p[i] * (dp[i] - s_d[qs]);
            }
            mma_slab_t<T, D>(Ds, p, dv);   // dV^T += dO^T P
            mma_slab_t<T, D>(Qs, ds, dk);  // dK^T += Q^T dS
        }
    };

    // Every dense query of the sample sees every key.
    const int cnt = a.counts[2 * b];
    const int32_t *didx = a.dense_idx + (size_t)b * N;
    run((cnt + 31) / 32,
        [&](int qb, int s, int &tk, bool &ok) HET_INLINE {
            ok = 32 * qb + s < cnt;
            tk = didx[imin(32 * qb + s, cnt - 1)];
        },
        std::false_type{});
    // Local queries whose window may hold a key of the workgroup's tiles.
    const int tx0 = kBwdWaves * xg, tx1 = imin(tx0 + kBwdWaves, g.tiles_x) - 1;
    int pt0, pt1, py0, py1, px0, px1;
    inverse_window(t, t, g.wt, g.lt, g.T, g.cut, pt0, pt1);
    inverse_window(ty * kBwdQY, imin(ty * kBwdQY + kBwdQY - 1, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut, py0, py1);
    inverse_window(tx0 * kBwdQX, imin(tx1 * kBwdQX + kBwdQX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut, px0, px1);
    const int nby = py1 - py0 + 1, nbx = px1 - px0 + 1;
    const int total = (pt1 - pt0 + 1) * nby * nbx;
    const uint8_t *mb = a.mask + (size_t)b * N;
    run((total + 31) / 32,
        [&](int qb, int s, int &tk, bool &ok) HET_INLINE {
            const int e = imin(32 * qb + s, total - 1);
            tk = ((pt0 + e / (nby * nbx)) * g.Hg + py0 + (e / nbx) % nby) * g.Wg + px0 + e % nbx;
            ok = 32 * qb + s < total && mb[tk] != 0;
        },
        std::true_type{});

    if (key_ok) {
        store_row_t<T, D>((T *)a.dk + sample + (size_t)ktok * tok_stride, dk, a.scale);
        store_row_t<T, D>((T *)a.dv + sample + (size_t)ktok * tok_stride, dv, 1.0f);
    }
}

size_t backward_workspace_bytes(int batch, int heads, int n) {
    return 2 * (size_t)batch * heads * n * sizeof(float);
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t stream) {
    LocalGeom g;
    g.T = a.grid_t; g.Hg = a.grid_h; g.Wg = a.grid_w;
    g.wt = a.win_t; g.wh = a.win_h; g.ww = a.win_w;
    g.lt = a.win_t < a.grid_t ? a.win_t : a.grid_t;
    g.lh = a.win_h < a.grid_h ? a.win_h : a.grid_h;
    g.lw = a.win_w < a.grid_w ? a.win_w : a.grid_w;
    g.tiles_y = (a.grid_h + kBwdQY - 1) / kBwdQY;
    g.tiles_x = (a.grid_w + kBwdQX - 1) / kBwdQX;
    g.slot_row = kBwdQX + g.lw - 1 <= 16 ? 16 : 32;
    g.cut = a.cut;
    if (kBwdQX + g.lw - 1 > 32) return hipErrorInvalidValue;  // rejected earlier by the ABI layer

    const long rows = (long)a.batch * a.n * a.heads;
    const int dense_units = a.batch * a.heads * ((a.max_dense + 32 * kBwdWaves - 1) / (32 * kBwdWaves));
    const int tile_units = a.batch * a.heads * g.T * g.tiles_y * g.tiles_x;
    const int x_groups = (g.tiles_x + kBwdWaves - 1) / kBwdWaves;
    const int key_units = a.batch * a.heads * g.T * g.tiles_y * x_groups;
    const bool sr16 = g.slot_row == 16;
#define HET_BWD(T_, D_)                                                                                        \
    do {                                                                                                       \
        constexpr int kRowsPerBlock = 4 * (64 / ((D_) * (int)sizeof(T_) / 16));                               \
        hipLaunchKernelGGL((bwd_prep_kernel<T_, D_>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), \
                           dim3(256), 0, stream, (const T_ *)a.o, (const T_ *)a.dout, a.dsum, rows, a.n, a.heads); \
        if (dense_units > 0)                                                                                   \
            hipLaunchKernelGGL((bwd_dq_dense_kernel<T_, D_>), dim3(dense_units), dim3(64 * kBwdWaves), 0, stream, \
                               a, dense_units);                                                                \
        if (sr16)                                                                                              \
            hipLaunchKernelGGL((bwd_dq_kernel<T_, D_, false, 16>), dim3(tile_units), dim3(64), 0, stream, a, g,  \
                               tile_units);                                                                    \
        else                                                                                                   \
            hipLaunchKernelGGL((bwd_dq_kernel<T_, D_, false, 32>), dim3(tile_units), dim3(64), 0, stream, a, g,  \
                               tile_units);                                                                    \
        hipLaunchKernelGGL((bwd_dkdv_kernel<T_, D_>), dim3(key_units), dim3(64 * kBwdWaves), 0, stream, a, g,   \
                           x_groups, key_units);                                                               \
    } while (0)
    if (a.bf16) {
        if (a.head_dim == 128) HET_BWD(__bf16, 128);
        else HET_BWD(__bf16, 64);
    } else {
        if (a.head_dim == 128) HET_BWD(float, 128);
        else HET_BWD(float, 64);
    }
#undef HET_BWD
    return hipGetLastError();
}

}  // namespace hetattn
