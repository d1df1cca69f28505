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
//   bwd_dkdv_bf16_kernel 128 consecutive keys, two waves per 32 keys (one
//                        with K: S, P, dV; one with V: dP, dS, dK): every
//                        dense query of the sample, then the local queries
//                        whose windows may hold these keys, in tiles of 64
//                        gathered into LDS by DMA;
//   bwd_dkdv_kernel      the fp32 form: 128 keys (four 4x8 tiles of one frame,
//                        a wave each, K and V rows in registers), the waves
//                        sharing each staged 32-query block.
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

// The fp32 kernels' MFMA (v_mfma_f32_32x32x2_f32) takes one element per
// lane and operand: k-step c of a D-element row is element 2c + half.

// Fragment c of a row for a 32x32 MFMA operand (A: the lane's row; B: the
// lane's column), zero when !ok.
__device__ __forceinline__ float load_frag(const float *row, int c, bool ok) {
    const int half = (threadIdx.x & 63) >> 5;
    return ok ? row[2 * c + half] : 0.0f;
}

// LDS slab of 32 fp32 rows of D elements (row pitch padded against bank
// conflicts, as in the local kernel's V slab).
template <int D>
struct Slab {
    static constexpr int kPitch = D + 4;
    static constexpr int kVec = 4;                   // elements per 16-byte load
    static constexpr int kChunks = D / kVec;         // 16-byte chunks per row
    static constexpr int kStage = 32 * kChunks / 64; // chunks per lane
};

// Copies row `row_of(s)` (or zeros when !ok_of(s)) of each slot s < 32 into
// the slab; the first kThreads threads of the workgroup move the 16-byte
// chunks between them.
template <int D, int kThreads = 64, typename RowOf, typename OkOf>
__device__ __forceinline__ void stage_rows(float *slab, RowOf &&row_of, OkOf &&ok_of) {
    using S = Slab<D>;
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
template <int D>
__device__ __forceinline__ float lds_frag(const float *slab, int c) {
    const int lane = threadIdx.x & 63, half = lane >> 5, row = lane & 31;
    return slab[row * Slab<D>::kPitch + 2 * c + half];
}

// acc[db] += X^T B, X = the slab (32 slots x D, slot order of the B
// operand's k index), B = the 16 per-lane values w[i] of a C-layout block
// (lane: column l%32; w[i]: slot 8(i/4) + 4*half + i%4).  Result rows are
// dims db*32 + l%32.
template <int D>
__device__ __forceinline__ void mma_slab_t(const float *slab, const float (&w)[16], f32x16 (&acc)[D / 32]) {
    const int lane = threadIdx.x & 63, half = lane >> 5, col = lane & 31;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float a = slab[(8 * (i / 4) + 4 * half + (i % 4)) * Slab<D>::kPitch + db * 32 + col];
            acc[db] = mfma32_f32(a, w[i], acc[db]);
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
            if constexpr (std::is_same<T, __bf16>::value) {
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
__host__ __device__ __forceinline__ void inverse_window(int j0, int j1, int k, int len, int S, int cut, int &p0,
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
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_dq_dense_kernel(BwdArgs a, int n_units) {
    using T = float;
    using S = Slab<D>;
    constexpr int kSteps = D / 2;
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

    float qf[kSteps], df[kSteps];
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
        for (int c = 0; c < kSteps; ++c) sc = mfma32_f32(lds_frag<D>(Ks, c), qf[c], sc);
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
            sc = mfma32_f32(lds_frag<D>(Ks, c), qf[c], sc);
            dp = mfma32_f32(lds_frag<D>(Vs, c), df[c], dp);
        }
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = in_block(kb, i) ? __builtin_amdgcn_exp2f(sc[i] * sl2 - lse2) : 0.0f;
            ds[i] = p * (dp[i] - dq_i);
        }
        mma_slab_t<D>(Ks, ds, acc);
    }
    if (valid) store_row_t<T, D>((T *)a.dq + sample + (size_t)tok * tok_stride, acc, a.scale);
}

// dQ of 128 dense rows (consecutive entries of the dense index list), bf16,
// given their LSE (the dense forward kernel's statistics, launched in its
// LSE form before this kernel).  Query group g (32 rows; this lane's row is
// its column in every product) has two waves on one SIMD, g and g + 4,
// which take the first and the second 32 keys of every 64-key tile, so that
// the exponentials of one overlap the products of the other:
//   S^T = K Q^T, dP^T = V dO^T, dS = P (dP - D), dQ^T += K^T dS^T (K read
//   transposed); the two halves' partial dQ are added through LDS.
// K and V tiles move global -> LDS by DMA (contiguous key rows, the
// descriptor's range ending at key N so that the ragged last tile reads
// zeros), chunk-swizzled as in the forward dense kernel, through rings of
// three buffers (two tiles in flight), with one barrier per tile.
template <int D>
constexpr uint32_t dq_dense_lds_bytes() { return 6 * 64 * D * 2; }

template <int D>
__device__ __forceinline__ void bwd_dq_dense_bf16(const BwdArgs &a, int unit, HET_LDS char *lds) {
    constexpr int kBN = 64;                          // keys per tile
    constexpr int kBM = 128;                         // dense rows per workgroup
    constexpr int kCpr = D / 8;                      // 16-byte chunks per row
    constexpr int kRowsPerLoad = 64 / kCpr;          // rows per wave DMA (1 KB)
    constexpr int kLoads = kBN / kRowsPerLoad / 8;   // DMAs per wave and tensor
    constexpr int NC = D / 16, NDB = D / 32;
    static_assert(kLoads >= 1, "tile shape");
    // LDS, in bytes: K and V through rings of three tile buffers of kBN key
    // rows each; after the key loop the same bytes carry the second half's
    // partial dQ.
    constexpr uint32_t kTileB = kBN * D * 2;
    constexpr uint32_t kK = 0, kV = 3 * kTileB;
    constexpr uint32_t kLdsBytes = 6 * kTileB;
    static_assert(4 * 64 * (D / 2) * 4 <= kLdsBytes, "dQ exchange fits the tile buffers");
    static_assert(kLdsBytes == dq_dense_lds_bytes<D>(), "LDS size");

    const int N = a.n, H = a.heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
    const int grp = wave & 3, kh = wave >> 2;  // query group, key half
    const int groups = (a.max_dense + kBM - 1) / kBM;
    const int qt = unit % groups, h = (unit / groups) % H, b = unit / groups / H;
    const int cnt = a.counts[2 * b];
    if (kBM * qt >= cnt) return;  // the whole workgroup
    const int slot = kBM * qt + 32 * grp + col;
    const bool valid = slot < cnt;
    const int tok = valid ? a.dense_idx[(size_t)b * N + slot] : 0;
    const int tok_stride = H * D;
    const size_t sample = (size_t)b * N * tok_stride + (size_t)h * D;
    const __bf16 *ksrc = (const __bf16 *)a.k + sample, *vsrc = (const __bf16 *)a.v + sample;
    const size_t row_bh = ((size_t)b * H + h) * N;
    const float sl2 = a.scale * kLog2e;
    const int n_kt = (N + kBN - 1) / kBN;

    bf16x8 qf[NC], df[NC];
    {
        const size_t off = sample + (size_t)tok * tok_stride + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qf[c] = valid ? *(const bf16x8 *)((const __bf16 *)a.q + off + 16 * c) : bf16x8{};
            df[c] = valid ? *(const bf16x8 *)((const __bf16 *)a.dout + off + 16 * c) : bf16x8{};
        }
    }
    const float d_i = valid ? a.dsum[row_bh + tok] : 0.0f;

    // DMA: load j of this wave fills key rows from (wave*kLoads + j)*kRowsPerLoad
    // on; the descriptor base is the tile's first key row, so the offsets
    // inside a tile are fixed.
    int dma_voff[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int r = (wave * kLoads + j) * kRowsPerLoad + lane / kCpr;
        dma_voff[j] = 2 * (r * tok_stride + 8 * ((lane % kCpr) ^ swz<D>(r)));
    }
    auto dma = [&](HET_LDS char *wr, const __bf16 *src, uint32_t dst_base, int kt) HET_INLINE {
        const int key0 = kt * kBN;
        const uint32_t bytes = (uint32_t)(N - key0) * (uint32_t)tok_stride * 2u;
        const __bf16 *base = src + (size_t)key0 * tok_stride;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const uint32_t dst = dst_base + (wave * kLoads + j) * kRowsPerLoad * D * 2;
            buffer_load_lds16(base, bytes, (HET_LDS void *)(wr + dst), dma_voff[j]);
        }
    };
    // A operands (byte offsets in a tile): key rows 32*kh + col at chunk
    // 2c + half, and the transposed K reads with the forward dense kernel's V
    // offsets, from key row 32*kh on.
    const int g16 = lane >> 4, j16 = lane & 15;
    uint32_t r_off[NC], t_off[NDB][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) r_off[c] = 2 * ((32 * kh + col) * D + 8 * ((2 * c + half) ^ swz<D>(col)));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int lohi = 0; lohi < 2; ++lohi) {
            const int row = 4 * half + (j16 >> 2) + 8 * lohi;
            t_off[db][lohi] = 2 * ((32 * kh + row) * D +
                                   8 * ((4 * db + 2 * (g16 & 1) + ((j16 & 3) >> 1)) ^ swz<D>(row)) + 4 * (j16 & 1));
        }
    auto ld128 = [&](const HET_LDS char *rd, uint32_t off) HET_INLINE -> bf16x8 {
        return *(const HET_LDS bf16x8 *)(rd + off);
    };
    constexpr int kA = 4;  // A operands read ahead of their MFMA
    // S^T (this wave's 32 keys x 32 rows) of the K tile at kbase, and, when
    // vbase is given, dP^T of the V tile, as independent chains.
    auto row_products = [&](const HET_LDS char *rd, uint32_t kbase, uint32_t vbase, bool with_dp, f32x16 &sc,
                            f32x16 &dp) HET_INLINE {
        sc = f32x16{};
        dp = f32x16{};
        uint32_t ka[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[c] = kbase + r_off[c];
        const uint32_t vdelta = vbase - kbase;
        bf16x8 ring[kA];
        if (with_dp) {
            constexpr int n = 2 * NC;  // step i: K (even) or V (odd), k-chunk i>>1
            auto op = [&](int i) HET_INLINE -> bf16x8 { return ld128(rd, ka[i >> 1] + ((i & 1) ? vdelta : 0u)); };
#pragma unroll
            for (int x = 0; x < kA; ++x) ring[x] = op(x);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < n; ++i) {
                if (i & 1) dp = mfma32_bf16(ring[i % kA], df[i >> 1], dp);
                else sc = mfma32_bf16(ring[i % kA], qf[i >> 1], sc);
                if (i + kA < n) ring[i % kA] = op(i + kA);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int x = 0; x < kA; ++x) ring[x] = ld128(rd, ka[x]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                sc = mfma32_bf16(ring[i % kA], qf[i], sc);
                if (i + kA < NC) ring[i % kA] = ld128(rd, ka[i + kA]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Whether register i of a C-layout block of tile kt is a key below N.
    auto key_in = [&](int kt, int i) HET_INLINE {
        return kt * kBN + 32 * kh + 8 * (i / 4) + 4 * half + (i % 4) < N;
    };

    // s_waitcnt immediate: at most n vector-memory operations of this wave
    // outstanding (no wait on the other counters).
    auto vm_wait = [](int n) constexpr { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); };
    const float lse2 = valid ? a.lse[row_bh + tok] : 0.0f;

    // ---- dQ^T += K^T dS^T over this wave's key half
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
#pragma unroll
    for (int x = 0; x < 2; ++x)
        if (x < n_kt) {
            dma(lds, ksrc, kK + x * kTileB, x);
            dma(lds, vsrc, kV + x * kTileB, x);
        }
    // Nothing outside the loop's non-aliasing DMAs may be in flight when it
    // starts, or the compiler waits for it inside every iteration.
    __builtin_amdgcn_s_waitcnt(0);
    int cur = 0;  // kt % 3
    for (int kt = 0; kt < n_kt; ++kt) {
        if (kt + 1 < n_kt) __builtin_amdgcn_s_waitcnt(vm_wait(2 * kLoads));
        else __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __syncthreads();  // tiles kt in LDS; tiles kt-1 done
        const int nx2 = cur == 0 ? 2 : cur - 1;  // (kt + 2) % 3
        // The DMA into buffer nx2 and the reads of buffer cur go through
        // pointers declared not to alias (their bytes are disjoint), so the
        // compiler does not wait for the DMA before the transposed reads.
        // (wr: K buffer nx2, rd: K buffer cur; the V buffers sit kV - kK
        // bytes above their K buffers.)
        auto tile = [&](HET_LDS char *__restrict__ wr, const HET_LDS char *__restrict__ rd) HET_INLINE {
        if (kt + 2 < n_kt) {
            dma(wr, ksrc, 0, kt + 2);
            dma(wr, vsrc, kV - kK, kt + 2);
        }
        f32x16 sc, dp;
        row_products(rd, 0, kV - kK, true, sc, dp);
        const uint32_t kb = 0;
        auto op3 = [&](int i) HET_INLINE -> bf16x8 {
            const int db = i % NDB, c2 = i / NDB;
            const uint32_t o = kb + c2 * 16 * D * 2;
            return concat8(lds_read_tr16((const HET_LDS void *)(rd + t_off[db][0] + o)),
                           lds_read_tr16((const HET_LDS void *)(rd + t_off[db][1] + o)));
        };
        bf16x8 ring[kA];
#pragma unroll
        for (int x = 0; x < kA; ++x) ring[x] = op3(x);
        // chunk c2 of the block = registers 8*c2 .. 8*c2+7
        const bool ragged = kt * kBN + kBN > N;
        bf16x8 sf[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            u32x4 ws;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float s2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = 8 * c2 + 2 * jj + e;
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], sl2, -lse2));
                    if (ragged && !key_in(kt, i)) p = 0.0f;
                    s2[e] = p * (dp[i] - d_i);
                }
                ws[jj] = pack_bf16x2(s2[0], s2[1]);
            }
            sf[c2] = __builtin_bit_cast(bf16x8, ws);
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int n3 = 2 * NDB;
#pragma unroll
        for (int i = 0; i < n3; ++i) {
            acc[i % NDB] = mfma32_bf16(ring[i % kA], sf[i / NDB], acc[i % NDB]);
            if (i + kA < n3) ring[i % kA] = op3(i + kA);
            __builtin_amdgcn_sched_barrier(0);
        }
        };
        tile(lds + kK + nx2 * kTileB, lds + kK + cur * kTileB);
        cur = cur == 2 ? 0 : cur + 1;
    }

    // the second key half's partial dQ through LDS, in [group][4 registers]
    // [lane] f32x4 order (consecutive lanes, consecutive 16 bytes)
    __syncthreads();  // every wave is done with the tile buffers
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *(HET_LDS f32x4 *)(lds + 16 * ((grp * (NDB * 4) + db * 4 + i4) * 64 + lane)) =
                    f32x4{acc[db][4 * i4], acc[db][4 * i4 + 1], acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]};
    }
    __syncthreads();
    if (kh == 0 && valid) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 o = *(const HET_LDS f32x4 *)(lds + 16 * ((grp * (NDB * 4) + db * 4 + i4) * 64 + lane));
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[db][4 * i4 + e] += o[e];
            }
        store_row_t<__bf16, D>((__bf16 *)a.dq + sample + (size_t)tok * tok_stride, acc, a.scale);
    }
}

// dQ of 32 query rows (kDense: 32 consecutive entries of the dense index
// list -- the one-wave form; the dense rows use bwd_dq_dense_kernel -- else
// a 4x8 tile of local rows of one frame), and LSE of those rows.
template <int D, bool kDense, int SR>
__global__ __launch_bounds__(64) void bwd_dq_kernel(BwdArgs a, LocalGeom g, int n_units) {
    using T = float;
    using S = Slab<D>;
    constexpr int kSteps = D / 2;
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

    float qf[kSteps], df[kSteps];
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
        for (int c = 0; c < kSteps; ++c) s = mfma32_f32(load_frag(k + sample + (size_t)kt * tok_stride, c, kok), qf[c], s);
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
        stage_rows<D>(
            Ks, [&](int s) HET_INLINE { return k + sample + (size_t)slot_token(kb, s) * tok_stride; },
            [&](int s) HET_INLINE { return slot_ok(kb, s); });
        const f32x16 s = scores(kb);
        const int kt = slot_token(kb, col);
        const bool kok = slot_ok(kb, col);
        f32x16 dp = f32x16{};
#pragma unroll
        for (int c = 0; c < kSteps; ++c) dp = mfma32_f32(load_frag(v + sample + (size_t)kt * tok_stride, c, kok), df[c], dp);
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = key_in(kb, i) ? __builtin_amdgcn_exp2f(s[i] * sl2 - lse2) : 0.0f;
            ds[i] = p * (dp[i] - dq_i);
        }
        __syncthreads();  // the K slab is visible to the whole wave
        mma_slab_t<D>(Ks, ds, acc);
        __syncthreads();  // slab free for the next block
    }
    if (valid) store_row_t<T, D>((T *)a.dq + sample + (size_t)tok * tok_stride, acc, a.scale);
}

// dK and dV of 128 keys: the 4x8 tiles (ty, 4*xg + w) of frame t, wave w
// taking one tile with its K and V rows in registers.  The four waves share
// every 32-query block: Q and dO rows, LSE, D and the window of each query,
// staged once into LDS (row reads for S and dP, transposed reads for dK and
// dV).
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_dkdv_kernel(BwdArgs a, LocalGeom g, int x_groups,
                                                                  int n_units) {
    using T = float;
    using S = Slab<D>;
    constexpr int kSteps = D / 2;
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

    float kf[kSteps], vf[kSteps];
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
                sc = mfma32_f32(lds_frag<D>(Qs, c), kf[c], sc);
                dp = mfma32_f32(lds_frag<D>(Ds, c), vf[c], dp);
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
            mma_slab_t<D>(Ds, p, dv);   // dV^T += dO^T P
            mma_slab_t<D>(Qs, ds, dk);  // dK^T += Q^T dS
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

// dK and dV of 128 consecutive tokens of one (sample, head), bf16.  The
// block's keys come in four groups of 32, and each group has two waves on
// one SIMD (waves g and g + 4), so that the exponentials of one overlap the
// products of the other:
//   wave g      K rows in registers: S = Q K^T, P = exp2(S - LSE) (window
//               mask for local queries), dV^T += dO^T P;
//   wave g + 4  V rows in registers: dP = dO V^T, dS = P (dP - D),
//               dK^T += Q^T dS, one tile behind, with P taken from LDS.
// Every product keeps the key in the lane (B operand: a K or V row, or P or
// dS of the C layout; A operand: 32 query rows read from LDS, row-wise or
// transposed).  Queries come in tiles of 64 slots: every dense query of the
// sample, then, for each frame the block touches, the local queries of the
// box of positions whose windows can reach the block's keys in that frame.
// A key takes only the pairs of the box of its own frame, so no pair is
// counted twice.  The Q and dO rows of a tile are gathered global -> LDS by
// DMA (each lane fetches one 16-byte chunk of a row at its own offset, so a
// slot's row comes from wherever its token sits), chunk-swizzled as in the
// forward dense kernel, in three buffers (tile r+1 in flight while tiles r
// and r-1 are read); a slot without a query reads zeros (its offset is past
// the buffer's range) and has LSE = +inf, so its P and dS are 0.  Slot tokens
// run two tiles ahead; one barrier per tile.
template <int D>
constexpr uint32_t dkdv_lds_bytes() {
    return 6 * (64 * D * 2) + 2 * (4 * 2 * 2 * 64 * 16) + 3 * 64 * 4 + 3 * 64 * 4 + 3 * 64 * 16;
}

template <int D>
__device__ __forceinline__ void bwd_dkdv_bf16(const BwdArgs &a, const LocalGeom &g, int n_kblocks, int unit,
                                              HET_LDS char *lds) {
    constexpr int kTile = 64;                         // query slots per tile
    constexpr int kCpr = D / 8;                       // 16-byte chunks per row
    constexpr int kRowsPerLoad = 64 / kCpr;           // rows per wave DMA (1 KB)
    constexpr int kLoads = kTile / kRowsPerLoad / 8;  // DMAs per wave and tensor
    constexpr int NC = D / 16, NDB = D / 32;
    static_assert(kLoads >= 1, "tile shape");
    // LDS, in bytes: Q tiles [3][kTile][D] and dO tiles likewise (rows
    // chunk-swizzled), P as B-operand chunks [2 buffers][4 groups][2 halves of
    // 32 slots][2 chunks of 16 slots][64 lanes] x 16 B, then the per-slot LSE,
    // D and window records [3][kTile].  Every read below is a per-lane offset
    // fixed for the tile plus a constant.
    constexpr uint32_t kTileB = kTile * D * 2, kHalfB = 32 * D * 2, kChunkB = 16 * D * 2;
    constexpr uint32_t kQ = 0, kG = 3 * kTileB, kP = 6 * kTileB, kPBuf = 4 * 2 * 2 * 64 * 16;
    constexpr uint32_t kLse = kP + 2 * kPBuf, kDd = kLse + 3 * kTile * 4, kWin = kDd + 3 * kTile * 4;
    constexpr uint32_t kLdsBytes = kWin + 3 * kTile * 16;
    static_assert(kG + kTileB <= 65536, "dO reads take the Q offset plus an immediate");
    static_assert(kLdsBytes == dkdv_lds_bytes<D>(), "LDS size");

    const int N = a.n, H = a.heads, HW = g.Hg * g.Wg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
    const int grp = wave & 3;
    const bool role_p = wave < 4;  // S, P, dV (else dP, dS, dK)
    const int kblk = unit % n_kblocks, h = (unit / n_kblocks) % H, b = unit / n_kblocks / H;
    const int key0 = 128 * kblk, key1 = imin(key0 + 128, N);
    const int key = key0 + 32 * grp + col;
    const bool key_ok = key < N;
    const int kt = key / HW, ky = (key / g.Wg) % g.Hg, kx = key % g.Wg;
    const int tok_stride = H * D;
    const size_t sample = (size_t)b * N * tok_stride + (size_t)h * D;
    const __bf16 *qsrc = (const __bf16 *)a.q + sample, *gsrc = (const __bf16 *)a.dout + sample;
    // Bytes from the (sample, head) base to the end of the sample's last row;
    // below 2^32 because every tensor holds fewer than 2^31 elements.
    const uint32_t range = (uint32_t)N * (uint32_t)tok_stride * 2u;
    const size_t row_bh = ((size_t)b * H + h) * N;
    const float sl2 = a.scale * kLog2e;

    // This wave's key operand: K rows (role P) or V rows.
    bf16x8 kv[NC];
    {
        const __bf16 *src = (const __bf16 *)(role_p ? a.k : a.v) + sample + (size_t)(key_ok ? key : 0) * tok_stride +
                            8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) kv[c] = key_ok ? *(const bf16x8 *)(src + 16 * c) : bf16x8{};
    }
    f32x16 acc[NDB];  // dV^T (role P) or dK^T
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    // DMA j of this wave fills slots from (wave*kLoads + j)*kRowsPerLoad on;
    // this lane writes slot dma_slot[j] at chunk position lane%kCpr and so
    // fetches the chunk the swizzle puts there.
    int dma_slot[kLoads], dma_byte[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int s = (wave * kLoads + j) * kRowsPerLoad + lane / kCpr;
        dma_slot[j] = s;
        dma_byte[j] = 16 * ((lane % kCpr) ^ swz<D>(s));
    }
    // A operands (byte offsets in a tile): slot rows (S, dP) at chunk 2c + half
    // of row col, and the transposed reads (dV, dK) with the forward dense
    // kernel's V offsets; the 32-slot half and the 16-slot chunk only move
    // whole swizzle periods, so they are constants.
    const int g16 = lane >> 4, j16 = lane & 15;
    uint32_t r_off[NC], t_off[NDB][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) r_off[c] = 2 * (col * D + 8 * ((2 * c + half) ^ swz<D>(col)));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int lohi = 0; lohi < 2; ++lohi) {
            const int row = 4 * half + (j16 >> 2) + 8 * lohi;
            t_off[db][lohi] =
                2 * (row * D + 8 * ((4 * db + 2 * (g16 & 1) + ((j16 & 3) >> 1)) ^ swz<D>(row)) + 4 * (j16 & 1));
        }
    const uint32_t p_lane = kP + grp * 4096 + lane * 16;  // + buffer, half, chunk
    const uint32_t rec_lane = 16 * half;                  // 4 slots of 4 bytes per half

    auto ld128 = [&](const HET_LDS char *rd, uint32_t off) HET_INLINE -> bf16x8 {
        return *(const HET_LDS bf16x8 *)(rd + off);
    };
    auto ldtr8 = [&](const HET_LDS char *rd, uint32_t lo, uint32_t hi) HET_INLINE -> bf16x8 {
        return concat8(lds_read_tr16((const HET_LDS void *)(rd + lo)), lds_read_tr16((const HET_LDS void *)(rd + hi)));
    };
    constexpr int kA = 4;  // A operands read ahead of their MFMA

    // One wave's products on the tile in buffer cur (both roles): the row
    // product of both 32-slot halves (independent accumulators, A = Q rows
    // for S or dO rows for dP), the element-wise step, then the transposed
    // product of both halves into acc (A = dO^T for dV or Q^T for dK).
    // `elem` turns the two row products into the four B-operand chunks.
    auto tile_products = [&](const HET_LDS char *rd, uint32_t row_base, uint32_t tr_base, auto &&elem) HET_INLINE {
        uint32_t ra[NC], ta[NDB][2];
#pragma unroll
        for (int c = 0; c < NC; ++c) ra[c] = row_base + r_off[c];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            ta[db][0] = tr_base + t_off[db][0];
            ta[db][1] = tr_base + t_off[db][1];
        }
        f32x16 rp[2] = {f32x16{}, f32x16{}};
        bf16x8 ring[kA];
        constexpr int n1 = 2 * NC;  // step i: half i&1, k-chunk i>>1
        auto op1 = [&](int i) HET_INLINE -> bf16x8 { return ld128(rd, ra[i >> 1] + (i & 1) * kHalfB); };
#pragma unroll
        for (int x = 0; x < kA; ++x) ring[x] = op1(x);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < n1; ++i) {
            rp[i & 1] = mfma32_bf16(ring[i % kA], kv[i >> 1], rp[i & 1]);
            if (i + kA < n1) ring[i % kA] = op1(i + kA);
            __builtin_amdgcn_sched_barrier(0);
        }
        constexpr int n3 = 4 * NDB;  // step i: dim block i%NDB, chunk (i/NDB)&1, half i/(2 NDB)
        auto op3 = [&](int i) HET_INLINE -> bf16x8 {
            const int db = i % NDB, c2 = (i / NDB) & 1, qb2 = i / (2 * NDB);
            const uint32_t o = c2 * kChunkB + qb2 * kHalfB;
            return ldtr8(rd, ta[db][0] + o, ta[db][1] + o);
        };
#pragma unroll
        for (int x = 0; x < kA; ++x) ring[x] = op3(x);
        bf16x8 bf[2][2];
        elem(rp, bf);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < n3; ++i) {
            const int db = i % NDB, c2 = (i / NDB) & 1, qb2 = i / (2 * NDB);
            acc[db] = mfma32_bf16(ring[i % kA], bf[qb2][c2], acc[db]);
            if (i + kA < n3) ring[i % kA] = op3(i + kA);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // meta(r, s): token of slot s of tile r, or -1 for a slot without a query.
    auto run = [&](int n_tiles, auto &&meta, auto windowed_tag, bool key_in_part) HET_INLINE {
        constexpr bool windowed = decltype(windowed_tag)::value;
        if (n_tiles <= 0) return;
        int tk_next[kLoads + 1], tk_ahead[kLoads + 1];  // DMA slots, then record slot tid
        auto fetch_meta = [&](int r, int(&dst)[kLoads + 1]) HET_INLINE {
#pragma unroll
            for (int j = 0; j < kLoads; ++j) dst[j] = meta(r, dma_slot[j]);
            dst[kLoads] = tid < kTile ? meta(r, tid) : -1;
        };
        auto issue_dma = [&](HET_LDS char *wr, int buf, const int(&tk)[kLoads + 1]) HET_INLINE {
#pragma unroll
            for (int j = 0; j < kLoads; ++j) {
                // unsigned: a row offset can pass 2^31 bytes (it stays below range)
                const uint32_t voff =
                    tk[j] >= 0 ? (uint32_t)tk[j] * (uint32_t)tok_stride * 2u + (uint32_t)dma_byte[j] : range;
                const uint32_t dst = (wave * kLoads + j) * kRowsPerLoad * D * 2;  // wr: Q buffer buf
                buffer_load_lds16(qsrc, range, (HET_LDS void *)(wr + dst), (int)voff);
                buffer_load_lds16(gsrc, range, (HET_LDS void *)(wr + (kG - kQ) + dst), (int)voff);
            }
        };
        float r_lse = 0.0f, r_d = 0.0f;
        i32x4 r_win = {0, 0, 0, 0};
        auto load_rec = [&](const int(&tk)[kLoads + 1]) HET_INLINE {
            if (tid < kTile) {
                const int t = tk[kLoads];
                r_lse = t >= 0 ? a.lse[row_bh + t] : __builtin_inff();
                r_d = t >= 0 ? a.dsum[row_bh + t] : 0.0f;
                if (windowed && t >= 0) {
                    const int qt = t / HW, qy = (t / g.Wg) % g.Hg, qx = t % g.Wg;
                    r_win[0] = win_lo(qt, g.wt, g.lt, g.T, g.cut) | (win_hi(qt, g.wt, g.lt, g.T, g.cut) << 16);
                    r_win[1] = win_lo(qy, g.wh, g.lh, g.Hg, g.cut) | (win_hi(qy, g.wh, g.lh, g.Hg, g.cut) << 16);
                    r_win[2] = win_lo(qx, g.ww, g.lw, g.Wg, g.cut) | (win_hi(qx, g.ww, g.lw, g.Wg, g.cut) << 16);
                }
            }
        };
        auto store_rec = [&](int buf) HET_INLINE {
            if (tid < kTile) {
                *(HET_LDS float *)(lds + kLse + buf * kTile * 4 + tid * 4) = r_lse;
                *(HET_LDS float *)(lds + kDd + buf * kTile * 4 + tid * 4) = r_d;
                if (windowed) *(HET_LDS i32x4 *)(lds + kWin + buf * kTile * 16 + tid * 16) = r_win;
            }
        };
        // Role P: P = exp2(S - LSE) (0 outside the window), published for
        // the partner wave, and dV^T += dO^T P.
        // rd: Q buffer of the tile (its dO buffer sits kG - kQ bytes above)
        auto compute_p = [&](const HET_LDS char *rd, int cur, int pb) HET_INLINE {
            tile_products(rd, 0, kG - kQ, [&](const f32x16(&sc)[2], bf16x8(&pf)[2][2]) HET_INLINE {
#pragma unroll
                for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        u32x4 wp;
#pragma unroll
                        for (int g2 = 0; g2 < 2; ++g2) {
                            // register 4*g4 + e: slot 32*qb2 + 8*g4 + 4*half + e
                            const int g4 = 2 * c2 + g2;
                            const f32x4 l4 =
                                *(const HET_LDS f32x4 *)(lds + kLse + cur * kTile * 4 + rec_lane + 4 * (32 * qb2 + 8 * g4));
                            float p[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb2][4 * g4 + e], sl2, -l4[e]));
                                if constexpr (windowed) {
                                    const i32x4 w = *(const HET_LDS i32x4 *)(lds + kWin + cur * kTile * 16 +
                                                                            16 * (32 * qb2 + 8 * g4 + 4 * half + e));
                                    auto inside = [](int cc, int ww) HET_INLINE {
                                        return cc >= (ww & 0xffff) && cc < (ww >> 16);
                                    };
                                    const bool in =
                                        key_in_part && inside(kt, w[0]) && inside(ky, w[1]) && inside(kx, w[2]);
                                    p[e] = in ? p[e] : 0.0f;
                                }
                            }
                            wp[2 * g2] = pack_bf16x2(p[0], p[1]);
                            wp[2 * g2 + 1] = pack_bf16x2(p[2], p[3]);
                        }
                        pf[qb2][c2] = __builtin_bit_cast(bf16x8, wp);
                        *(HET_LDS bf16x8 *)(lds + p_lane + pb * kPBuf + qb2 * 2048 + c2 * 1024) = pf[qb2][c2];
                    }
            });
        };
        // Role dS: dS = P (dP - D) with the partner's P, and dK^T += Q^T dS.
        auto compute_ds = [&](const HET_LDS char *rd, int cur, int pb) HET_INLINE {
            tile_products(rd, kG - kQ, 0, [&](const f32x16(&dp)[2], bf16x8(&sf)[2][2]) HET_INLINE {
#pragma unroll
                for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        const bf16x8 pf = ld128(lds, p_lane + pb * kPBuf + qb2 * 2048 + c2 * 1024);
                        u32x4 ws;
#pragma unroll
                        for (int g2 = 0; g2 < 2; ++g2) {
                            const int g4 = 2 * c2 + g2;
                            const f32x4 d4 =
                                *(const HET_LDS f32x4 *)(lds + kDd + cur * kTile * 4 + rec_lane + 4 * (32 * qb2 + 8 * g4));
                            float s[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) s[e] = (float)pf[4 * g2 + e] * (dp[qb2][4 * g4 + e] - d4[e]);
                            ws[2 * g2] = pack_bf16x2(s[0], s[1]);
                            ws[2 * g2 + 1] = pack_bf16x2(s[2], s[3]);
                        }
                        sf[qb2][c2] = __builtin_bit_cast(bf16x8, ws);
                    }
            });
        };

        fetch_meta(0, tk_next);
        if (n_tiles > 1) fetch_meta(1, tk_ahead);
        __syncthreads();  // the previous run is done with the buffers
        issue_dma(lds + kQ, 0, tk_next);
        load_rec(tk_next);
        store_rec(0);
        // Iteration r: role P on tile r (buffer r % 3, P buffer r % 2), role
        // dS on tile r - 1.
        int cur = 0;
        for (int r = 0; r <= n_tiles; ++r) {
            const int nxt = cur == 2 ? 0 : cur + 1, prv = cur == 0 ? 2 : cur - 1;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();  // tile r, its records and P of tile r-1 in LDS; tile r-2 done
            // The DMA into buffer nxt and the reads of buffers cur and prv go
            // through pointers declared not to alias (their bytes are
            // disjoint), so the compiler does not wait for the DMA before the
            // transposed reads.
            auto iter = [&](HET_LDS char *__restrict__ wr, const HET_LDS char *__restrict__ rd) HET_INLINE {
                if (r + 1 < n_tiles) {
#pragma unroll
                    for (int j = 0; j <= kLoads; ++j) tk_next[j] = tk_ahead[j];
                    issue_dma(wr, nxt, tk_next);
                    load_rec(tk_next);
                    if (r + 2 < n_tiles) fetch_meta(r + 2, tk_ahead);
                }
                if (role_p) {
                    if (r < n_tiles) compute_p(rd, cur, r & 1);
                } else if (r > 0) {
                    compute_ds(rd, prv, (r - 1) & 1);
                }
            };
            iter(lds + kQ + nxt * kTileB, lds + kQ + (role_p ? cur : prv) * kTileB);
            if (r + 1 < n_tiles) store_rec(nxt);
            cur = nxt;
        }
    };

    // Every dense query of the sample sees every key.
    const int cnt = a.counts[2 * b];
    const int32_t *didx = a.dense_idx + (size_t)b * N;
    run((cnt + kTile - 1) / kTile,
        [&](int r, int s) HET_INLINE -> int {
            const int i = kTile * r + s;
            return i < cnt ? didx[i] : -1;
        },
        std::false_type{}, true);
    // Local queries, per frame the block touches: the box of positions whose
    // windows can hold a key of the block in that frame (rows y0..y1 of the
    // frame; columns x0..x1 when the block stays in one row, else all).
    // (When the band kernel has taken the local queries, their part is in
    // dk_part / dv_part and is added below.)
    const uint8_t *mb = a.mask + (size_t)b * N;
    for (int f = key0 / HW; !a.dk_part && f <= (key1 - 1) / HW; ++f) {
        const int lo = imax(key0, f * HW) - f * HW, hi = imin(key1, (f + 1) * HW) - 1 - f * HW;
        const int y0 = lo / g.Wg, y1 = hi / g.Wg;
        const int x0 = y0 == y1 ? lo % g.Wg : 0, x1 = y0 == y1 ? hi % g.Wg : g.Wg - 1;
        int pt0, pt1, py0, py1, px0, px1;
        inverse_window(f, f, g.wt, g.lt, g.T, g.cut, pt0, pt1);
        inverse_window(y0, y1, g.wh, g.lh, g.Hg, g.cut, py0, py1);
        inverse_window(x0, x1, g.ww, g.lw, g.Wg, g.cut, px0, px1);
        const int nby = py1 - py0 + 1, nbx = px1 - px0 + 1;
        const int total = (pt1 - pt0 + 1) * nby * nbx;
        run((total + kTile - 1) / kTile,
            [&](int r, int s) HET_INLINE -> int {
                const int e = kTile * r + s;
                if (e >= total) return -1;
                const int tk = ((pt0 + e / (nby * nbx)) * g.Hg + py0 + (e / nbx) % nby) * g.Wg + px0 + e % nbx;
                return mb[tk] != 0 ? tk : -1;
            },
            std::true_type{}, kt == f);
    }

    if (key_ok) {
        if (a.dk_part) {
            const float *src = (role_p ? a.dv_part : a.dk_part) + (((size_t)b * N + key) * H + h) * D + 4 * half;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 pv = *(const f32x4 *)(src + db * 32 + 8 * i4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[db][4 * i4 + e] += pv[e];
                }
        }
        __bf16 *dst = (__bf16 *)(role_p ? a.dv : a.dk) + sample + (size_t)key * tok_stride;
        store_row_t<__bf16, D>(dst, acc, role_p ? 1.0f : a.scale);
    }
}

// Local part of dK and dV (bf16) for grids that local_band_fits accepts
// (windows at most 9 wide along the columns).  Workgroup = the
// four 4x8 key tiles (ty, 4*xg .. 4*xg+3) of frame t, two waves per tile on
// one SIMD, as in the dense pass (K side: S, P, dV; V side: dP, dS, dK one
// band behind, P through LDS).  The queries whose windows can hold a key of
// the tiles form a box (frames x rows x columns: the inverse windows of the
// tiles' extent per axis).  It is streamed through LDS in bands of two box
// rows of one frame: each box row is a run of consecutive tokens, so every
// lane's DMA offset from the band's first token is fixed.  From each band a
// tile takes the 16 columns x 2 rows of queries whose windows can reach it:
// one 32 x 32 block.  A query sees a key when it is local and its position
// lies, per axis, in the key's inverse window (computed once per lane).
// Output: the fp32 partial dK (without the softmax scale) and dV of every
// key of the tiles, which the dense pass adds before it stores dK and dV.
constexpr int kLbCols = 40;  // LDS rows per box row of a band

// Whether the band form holds the grid: every 8-column key tile takes its
// queries from at most 16 columns, and every group of four tiles from at most
// kLbCols.  A key tile's columns span 8 + k - 1 positions away from a border;
// where windows are shifted inside the grid, the positions that see a key
// near the border reach up to (k - 1) / 2 further, so the spans are taken
// from the inverse windows tile by tile.
static bool local_band_fits(const LocalGeom &g) {
    for (int tx = 0; tx < g.tiles_x; ++tx) {
        int c0, c1;
        inverse_window(tx * kBwdQX, imin(tx * kBwdQX + kBwdQX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut, c0, c1);
        if (c1 - c0 + 1 > 16) return false;
        if (tx % 4 == 0) {
            const int tx1 = imin(tx + 3, g.tiles_x - 1);
            inverse_window(tx * kBwdQX, imin(tx1 * kBwdQX + kBwdQX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut, c0, c1);
            if (c1 - c0 + 1 > kLbCols) return false;
        }
    }
    return true;
}

template <int D>
__global__ __launch_bounds__(512) void bwd_dkdv_local_band_kernel(BwdArgs a, LocalGeom g, int x_groups,
                                                                  int n_units) {
    constexpr int kCpr = D / 8;
    constexpr int kTokPerLoad = 64 / kCpr;                 // rows per wave DMA (1 KB)
    constexpr int kBandRows = 2 * kLbCols;
    constexpr int kLoadsTot = kBandRows / kTokPerLoad;     // wave DMAs per tensor and band
    constexpr int kLoadsPerWave = (kLoadsTot + 7) / 8;
    static_assert(kBandRows % kTokPerLoad == 0, "band rows in whole DMAs");
    constexpr int NC = D / 16, NDB = D / 32;
    constexpr uint32_t kBufB = kBandRows * D * 2;
    constexpr uint32_t kQ = 0, kG = 3 * kBufB, kP = 6 * kBufB, kPBuf = 4 * 2 * 64 * 16;
    constexpr uint32_t kLse = kP + 2 * kPBuf, kDd = kLse + 3 * 4 * 32 * 4;
    constexpr uint32_t kLdsBytes = kDd + 3 * 4 * 32 * 4;
    __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
    HET_LDS char *lds = (HET_LDS char *)smem;

    const int unit = blockIdx.x;
    if (unit >= n_units) return;
    const int N = a.n, H = a.heads;
    int rest = unit;
    const int xg = rest % x_groups;
    rest /= x_groups;
    const int ty = rest % g.tiles_y;
    rest /= g.tiles_y;
    const int t = rest % g.T;
    rest /= g.T;
    const int h = rest % H, b = rest / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
    const int grp = wave & 3;
    const bool role_p = wave < 4;
    const int tok_stride = H * D;
    const size_t sample = (size_t)b * N * tok_stride + (size_t)h * D;
    const size_t row_bh = ((size_t)b * H + h) * N;
    const float sl2 = a.scale * kLog2e;

    // The box of query positions (uniform).
    const int tx0 = 4 * xg, tx1 = imin(tx0 + 3, g.tiles_x - 1);
    int pt0, pt1, py0, py1, px0, px1;
    inverse_window(t, t, g.wt, g.lt, g.T, g.cut, pt0, pt1);
    inverse_window(ty * kBwdQY, imin(ty * kBwdQY + kBwdQY - 1, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut, py0, py1);
    inverse_window(tx0 * kBwdQX, imin(tx1 * kBwdQX + kBwdQX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut, px0, px1);
    const int C = px1 - px0 + 1;  // <= kLbCols
    const int nb_f = (py1 - py0 + 2) / 2, n_bands = (pt1 - pt0 + 1) * nb_f;
    // Columns of the box from which tile g' takes its 16 query columns.
    auto tile_cw = [&](int gg) HET_INLINE -> int {
        const int tx = imin(tx0 + gg, g.tiles_x - 1);
        int c0, c1;
        inverse_window(tx * kBwdQX, imin(tx * kBwdQX + kBwdQX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut, c0, c1);
        return c0 - px0;
    };
    const int cw = tile_cw(grp);

    // This lane's key and the intervals of query positions that see it.
    const int tx = tx0 + grp;
    const int ky = ty * kBwdQY + col / kBwdQX, kx = tx * kBwdQX + col % kBwdQX;
    const bool key_ok = tx < g.tiles_x && ky < g.Hg && kx < g.Wg;
    const int key = key_ok ? (t * g.Hg + ky) * g.Wg + kx : 0;
    int it0, it1, iy0, iy1, ix0, ix1;
    inverse_window(t, t, g.wt, g.lt, g.T, g.cut, it0, it1);
    inverse_window(imin(ky, g.Hg - 1), imin(ky, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut, iy0, iy1);
    inverse_window(imin(kx, g.Wg - 1), imin(kx, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut, ix0, ix1);

    bf16x8 kv[NC];
    {
        const __bf16 *src = (const __bf16 *)(role_p ? a.k : a.v) + sample + (size_t)key * tok_stride + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) kv[c] = key_ok ? *(const bf16x8 *)(src + 16 * c) : bf16x8{};
    }
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    // Slot j (< 32) of this tile's block: box row j/16 of the band, column
    // cw + j%16 (clamped to the LDS rows; a clamped slot is outside every
    // key's interval, so it is masked).
    auto slot_row = [&](int j) HET_INLINE -> int { return (j >> 4) * kLbCols + imin(cw + (j & 15), kLbCols - 1); };
    const int g16 = lane >> 4, j16 = lane & 15;
    uint32_t r_off[NC], t_off[2][NDB][2];
    {
        const int R = slot_row(col);
#pragma unroll
        for (int c = 0; c < NC; ++c) r_off[c] = 2 * (R * D + 8 * ((2 * c + half) ^ swz<D>(R)));
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int lohi = 0; lohi < 2; ++lohi) {
                const int Rt = slot_row(16 * c2 + 4 * half + (j16 >> 2) + 8 * lohi);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    t_off[c2][db][lohi] =
                        2 * (Rt * D + 8 * ((4 * db + 2 * (g16 & 1) + ((j16 & 3) >> 1)) ^ swz<D>(Rt)) + 4 * (j16 & 1));
            }
    }
    // DMA: wave load i (= wave + 8j) fills band rows i*kTokPerLoad ..; row R
    // = rr*kLbCols + c holds box row rr, column c; columns past the box get
    // an offset beyond any descriptor's range and read as zeros.
    int dma_voff[kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
        const int i = wave + 8 * j;
        const int R = i * kTokPerLoad + lane / kCpr;
        const int rr = R / kLbCols, c = R % kLbCols;
        dma_voff[j] = c < C ? 2 * ((rr * g.Wg + c) * tok_stride + 8 * ((lane % kCpr) ^ swz<D>(R))) : 0x7ffffff0;
    }
    const __bf16 *qbase = (const __bf16 *)a.q + sample, *gbase = (const __bf16 *)a.dout + sample;
    // A band is named by its frame f and its row of bands rb (box rows
    // py0 + 2 rb and the next); the loop advances both by counters.
    auto next_band = [&](int &f, int &rb) HET_INLINE {
        if (++rb == nb_f) {
            rb = 0;
            ++f;
        }
    };
    auto issue_dma = [&](HET_LDS char *wr, int f, int rb) HET_INLINE {
        const int tok0 = (f * g.Hg + py0 + 2 * rb) * g.Wg + px0;
        const uint32_t bytes = (uint32_t)(N - tok0) * (uint32_t)tok_stride * 2u;
        const __bf16 *qp = qbase + (size_t)tok0 * tok_stride, *gp = gbase + (size_t)tok0 * tok_stride;
#pragma unroll
        for (int j = 0; j < kLoadsPerWave; ++j) {
            const int i = wave + 8 * j;
            if (i < kLoadsTot) {
                const uint32_t dst = i * kTokPerLoad * D * 2;
                buffer_load_lds16(qp, bytes, (HET_LDS void *)(wr + dst), dma_voff[j]);
                buffer_load_lds16(gp, bytes, (HET_LDS void *)(wr + (kG - kQ) + dst), dma_voff[j]);
            }
        }
    };
    // Records of a band, per tile and slot: LSE (+inf for a slot without a
    // local query in the box) and D.  Thread tid < 128 owns slot tid%32 of
    // tile tid/32.
    const int rec_g = (tid >> 5) & 3, rec_j = tid & 31;
    const int rec_cw = tile_cw(rec_g);
    const uint8_t *mb = a.mask + (size_t)b * N;
    float r_lse = 0.0f, r_d = 0.0f;
    auto load_rec = [&](int f, int rb) HET_INLINE {
        if (tid < 128) {
            const int y = py0 + 2 * rb + (rec_j >> 4);
            const int c = rec_cw + (rec_j & 15);
            const bool in_box = y <= py1 && c < C;
            const int tk = in_box ? (f * g.Hg + y) * g.Wg + px0 + c : 0;
            const bool ok = in_box && mb[tk] != 0;
            r_lse = ok ? a.lse[row_bh + tk] : __builtin_inff();
            r_d = ok ? a.dsum[row_bh + tk] : 0.0f;
        }
    };
    auto store_rec = [&](int buf) HET_INLINE {
        if (tid < 128) {
            *(HET_LDS float *)(lds + kLse + (buf * 128 + tid) * 4) = r_lse;
            *(HET_LDS float *)(lds + kDd + (buf * 128 + tid) * 4) = r_d;
        }
    };
    const uint32_t p_lane = kP + grp * 2048 + lane * 16;           // + buffer, chunk
    const uint32_t rec_lane = (grp * 32 + 4 * half) * 4;           // + buffer, 8*(i/4) slots
    // Window test of register i (slot 8(i/4) + 4*half + i%4): the band's
    // frame and the slot's row and column against this key's intervals.
    auto in_win = [&](int f, int rb, int i) HET_INLINE -> bool {
        const int y = py0 + 2 * rb + (i >> 3);
        const int x = px0 + cw + 8 * ((i >> 2) & 1) + 4 * half + (i & 3);
        return f >= it0 && f <= it1 && y >= iy0 && y <= iy1 && x >= ix0 && x <= ix1;
    };

    auto ld128 = [&](const HET_LDS char *rd, uint32_t off) HET_INLINE -> bf16x8 {
        return *(const HET_LDS bf16x8 *)(rd + off);
    };
    constexpr int kA = 4;
    // One block: row product (A = slot rows), element step, transposed
    // product into acc (A = the other tensor's slots read transposed).
    auto block = [&](const HET_LDS char *rd, uint32_t row_base, uint32_t tr_base, auto &&elem) HET_INLINE {
        f32x16 rp = f32x16{};
        bf16x8 ring[kA];
        auto op1 = [&](int i) HET_INLINE -> bf16x8 { return ld128(rd, row_base + r_off[i]); };
#pragma unroll
        for (int x = 0; x < kA; ++x) ring[x] = op1(x);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            rp = mfma32_bf16(ring[i % kA], kv[i], rp);
            if (i + kA < NC) ring[i % kA] = op1(i + kA);
            __builtin_amdgcn_sched_barrier(0);
        }
        constexpr int n3 = 2 * NDB;  // step i: dim block i%NDB, chunk i/NDB
        auto op3 = [&](int i) HET_INLINE -> bf16x8 {
            const int db = i % NDB, c2 = i / NDB;
            return concat8(lds_read_tr16((const HET_LDS void *)(rd + tr_base + t_off[c2][db][0])),
                           lds_read_tr16((const HET_LDS void *)(rd + tr_base + t_off[c2][db][1])));
        };
#pragma unroll
        for (int x = 0; x < kA; ++x) ring[x] = op3(x);
        bf16x8 bf[2];
        elem(rp, bf);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < n3; ++i) {
            acc[i % NDB] = mfma32_bf16(ring[i % kA], bf[i / NDB], acc[i % NDB]);
            if (i + kA < n3) ring[i % kA] = op3(i + kA);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto compute_p = [&](const HET_LDS char *rd, int bf, int brb, int cur, int pb) HET_INLINE {
        block(rd, 0, kG - kQ, [&](const f32x16 &sc, bf16x8(&pf)[2]) HET_INLINE {
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                u32x4 wp;
#pragma unroll
                for (int g2 = 0; g2 < 2; ++g2) {
                    const int g4 = 2 * c2 + g2;
                    const f32x4 l4 = *(const HET_LDS f32x4 *)(lds + kLse + cur * 512 + rec_lane + 32 * g4);
                    float p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[4 * g4 + e], sl2, -l4[e]));
                        p[e] = in_win(bf, brb, 4 * g4 + e) ? pe : 0.0f;
                    }
                    wp[2 * g2] = pack_bf16x2(p[0], p[1]);
                    wp[2 * g2 + 1] = pack_bf16x2(p[2], p[3]);
                }
                pf[c2] = __builtin_bit_cast(bf16x8, wp);
                *(HET_LDS bf16x8 *)(lds + p_lane + pb * kPBuf + c2 * 1024) = pf[c2];
            }
        });
    };
    auto compute_ds = [&](const HET_LDS char *rd, int cur, int pb) HET_INLINE {
        block(rd, kG - kQ, 0, [&](const f32x16 &dp, bf16x8(&sf)[2]) HET_INLINE {
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const bf16x8 pf = ld128(lds, p_lane + pb * kPBuf + c2 * 1024);
                u32x4 ws;
#pragma unroll
                for (int g2 = 0; g2 < 2; ++g2) {
                    const int g4 = 2 * c2 + g2;
                    const f32x4 d4 = *(const HET_LDS f32x4 *)(lds + kDd + cur * 512 + rec_lane + 32 * g4);
                    float s[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[e] = (float)pf[4 * g2 + e] * (dp[4 * g4 + e] - d4[e]);
                    ws[2 * g2] = pack_bf16x2(s[0], s[1]);
                    ws[2 * g2 + 1] = pack_bf16x2(s[2], s[3]);
                }
                sf[c2] = __builtin_bit_cast(bf16x8, ws);
            }
        });
    };

    // Iteration r: K side on band r, V side on band r-1 (three band
    // buffers, two P buffers, records three deep, one barrier per band).
    issue_dma(lds + kQ, pt0, 0);
    load_rec(pt0, 0);
    store_rec(0);
    int cur = 0;
    int c_f = pt0, c_rb = 0, n_f = pt0, n_rb = 0;  // bands r and r + 1
    next_band(n_f, n_rb);
    for (int r = 0; r <= n_bands; ++r) {
        const int nxt = cur == 2 ? 0 : cur + 1, prv = cur == 0 ? 2 : cur - 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // band r, its records and P of band r-1 in LDS; band r-2 done
        auto iter = [&](HET_LDS char *__restrict__ wr, const HET_LDS char *__restrict__ rd) HET_INLINE {
            if (r + 1 < n_bands) {
                issue_dma(wr, n_f, n_rb);
                load_rec(n_f, n_rb);
            }
            if (role_p) {
                if (r < n_bands) compute_p(rd, c_f, c_rb, cur, r & 1);
            } else if (r > 0) {
                compute_ds(rd, prv, (r - 1) & 1);
            }
        };
        iter(lds + kQ + nxt * kBufB, lds + kQ + (role_p ? cur : prv) * kBufB);
        if (r + 1 < n_bands) store_rec(nxt);
        cur = nxt;
        next_band(c_f, c_rb);
        next_band(n_f, n_rb);
    }

    // fp32 partials: dV (K side) and dK without the scale (V side).
    if (key_ok) {
        float *dst = (role_p ? a.dv_part : a.dk_part) + (((size_t)b * N + key) * H + h) * D + 4 * half;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *(f32x4 *)(dst + db * 32 + 8 * i4) =
                    f32x4{acc[db][4 * i4], acc[db][4 * i4 + 1], acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]};
    }
}

// The dense rows' dQ (workgroups 0 .. n_dq-1) and dK/dV (the rest) in one
// launch: the two are independent given the LSE, so the dK/dV workgroups
// fill the CUs that the last round of dQ workgroups leaves idle.
template <int D>
__global__ __launch_bounds__(512) void bwd_dq_dkdv_bf16_kernel(BwdArgs a, LocalGeom g, int n_dq, int n_kblocks,
                                                               int n_kv) {
    constexpr uint32_t kBytes = dq_dense_lds_bytes<D>() > dkdv_lds_bytes<D>() ? dq_dense_lds_bytes<D>()
                                                                                : dkdv_lds_bytes<D>();
    __shared__ __attribute__((aligned(1024))) char smem[kBytes];
    HET_LDS char *lds = (HET_LDS char *)smem;
    const int bid = blockIdx.x;
    if (bid < n_dq) bwd_dq_dense_bf16<D>(a, bid, lds);
    else if (bid - n_dq < n_kv) bwd_dkdv_bf16<D>(a, g, n_kblocks, bid - n_dq, lds);
}

size_t backward_workspace_bytes(int batch, int heads, int n, int head_dim, bool bf16) {
    size_t bytes = 2 * (size_t)batch * heads * n * sizeof(float) + dense_lse_workspace_bytes(kBwdMaxLseGroups);
    if (bf16) bytes += 2 * (size_t)batch * n * heads * head_dim * sizeof(float);  // local dK, dV parts
    return bytes;
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

    // bf16: the rows' LSE comes from the forward kernels in their
    // statistics-only forms (dense rows: the persistent dense kernel; local
    // rows: the band kernel), and the local rows' dQ from the band kernel's
    // gradient form.
    AttnArgs fa{};
    fa.q = a.q;
    fa.k = a.k;
    fa.v = a.v;
    fa.mask = a.mask;
    fa.grid_t = a.grid_t;
    fa.grid_h = a.grid_h;
    fa.grid_w = a.grid_w;
    fa.win_t = a.win_t;
    fa.win_h = a.win_h;
    fa.win_w = a.win_w;
    fa.cut = a.cut;
    fa.dense_idx = a.dense_idx;
    fa.counts = a.counts;
    fa.batch = a.batch;
    fa.n = a.n;
    fa.heads = a.heads;
    fa.head_dim = a.head_dim;
    fa.bf16 = a.bf16;
    fa.scale = a.scale;
    fa.max_dense = a.max_dense;
    fa.dense_exact = a.dense_exact;
    fa.workspace = a.lse_part;
    fa.cu_count = a.cu_count;
    const long rows = (long)a.batch * a.n * a.heads;
    const int dense_units = a.batch * a.heads * ((a.max_dense + 32 * kBwdWaves - 1) / (32 * kBwdWaves));
    const int tile_units = a.batch * a.heads * g.T * g.tiles_y * g.tiles_x;
    const int x_groups = (g.tiles_x + kBwdWaves - 1) / kBwdWaves;
    const int key_units = a.batch * a.heads * g.T * g.tiles_y * x_groups;
    const bool sr16 = g.slot_row == 16;
    const int n_kblocks = (a.n + 127) / 128;
    const int kblock_units = a.batch * a.heads * n_kblocks;
    // bf16: D, the rows' LSE (dense, local), the local rows' dQ, then the
    // dense rows' dQ together with dK/dV in one launch.
    auto bf16_path = [&](auto d_tag) -> hipError_t {
        constexpr int D_ = decltype(d_tag)::value;
        constexpr int kRowsPerBlock = 4 * (64 / (D_ * 2 / 16));
        hipLaunchKernelGGL((bwd_prep_kernel<__bf16, D_>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                           dim3(256), 0, stream, (const __bf16 *)a.o, (const __bf16 *)a.dout, a.dsum, rows, a.n,
                           a.heads);
        hipError_t e = hipSuccess;
        if (!a.lse_given) {
            if (dense_units > 0) e = launch_dense_lse(fa, a.lse, stream);
            if (e == hipSuccess) e = launch_local_lse(fa, a.lse, stream);
        }
        if (e == hipSuccess) e = launch_local_dq(fa, a.dout, a.lse, a.dsum, a.dq, stream);
        if (e != hipSuccess) return e;
        // Local part of dK/dV by key tiles over query bands when the tiles'
        // query columns fit its slots (windows up to 9 wide, less near a
        // shifted border); else the dense pass runs over the local queries.
        BwdArgs a2 = a;
        if (local_band_fits(g)) {
            hipLaunchKernelGGL((bwd_dkdv_local_band_kernel<D_>), dim3((unsigned)key_units), dim3(512), 0, stream, a, g,
                               x_groups, key_units);
        } else {
            a2.dk_part = a2.dv_part = nullptr;
        }
        hipLaunchKernelGGL((bwd_dq_dkdv_bf16_kernel<D_>), dim3((unsigned)(dense_units + kblock_units)), dim3(512), 0,
                           stream, a2, g, dense_units, n_kblocks, kblock_units);
        return hipGetLastError();
    };
    // fp32: the staged-block kernels, each with its own LSE pass.
    auto f32_path = [&](auto d_tag) -> hipError_t {
        constexpr int D_ = decltype(d_tag)::value;
        constexpr int kRowsPerBlock = 4 * (64 / (D_ * 4 / 16));
        hipLaunchKernelGGL((bwd_prep_kernel<float, D_>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                           dim3(256), 0, stream, (const float *)a.o, (const float *)a.dout, a.dsum, rows, a.n,
                           a.heads);
        if (dense_units > 0)
            hipLaunchKernelGGL((bwd_dq_dense_kernel<D_>), dim3(dense_units), dim3(64 * kBwdWaves), 0, stream,
                               a, dense_units);
        if (sr16)
            hipLaunchKernelGGL((bwd_dq_kernel<D_, false, 16>), dim3(tile_units), dim3(64), 0, stream, a, g,
                               tile_units);
        else
            hipLaunchKernelGGL((bwd_dq_kernel<D_, false, 32>), dim3(tile_units), dim3(64), 0, stream, a, g,
                               tile_units);
        hipLaunchKernelGGL((bwd_dkdv_kernel<D_>), dim3(key_units), dim3(64 * kBwdWaves), 0, stream, a, g,
                           x_groups, key_units);
        return hipGetLastError();
    };
    using D128 = std::integral_constant<int, 128>;
    using D64 = std::integral_constant<int, 64>;
    if (a.bf16) return a.head_dim == 128 ? bf16_path(D128{}) : bf16_path(D64{});
    return a.head_dim == 128 ? f32_path(D128{}) : f32_path(D64{});
}

}  // namespace hetattn
