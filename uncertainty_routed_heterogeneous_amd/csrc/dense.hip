// dense.hip -- dense softmax attention for the gathered dense tokens.
//
// [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
// Video Diffusion" (HetA-DiT): dense attention of §3.1.1 Eq. 2 for the tokens
// with m_i = 0 (§3.2.2 Eqs. 12-13).  This is the rho*N^2*d_h term of the cost
// model (§3.2.2 Eq. 14) and the dominant cost of the layer.
//
// One workgroup = 4 waves = 128 gathered queries of one (sample, head); each
// wave owns 32 queries.  Per key tile of BN keys:
//   S^T = K Q^T      MFMA, A = K tile (LDS), B = Q (registers, loaded once)
//   online softmax   fp32, base 2, per query = per lane (lane l%32)
//   O^T += V^T P^T   MFMA, A = V tile read transposed from LDS, B = P
// Computing the transposed products keeps every per-query quantity (running
// max, row sum, output column) in the lane that owns the query, so the
// softmax needs one cross-half exchange per tile and no LDS round trip.
// K/V tiles for step j+1 are fetched into registers while step j computes.
#include "common.hpp"
#include "kernels.hpp"

namespace hetattn {

constexpr int kDenseThreads = 256;
constexpr int kDenseBM = 128;

template <typename T, int D, int BN>
struct DenseTile {
    static constexpr int kPadK = (sizeof(T) == 2) ? 8 : 4;
    static constexpr int kPadV = (sizeof(T) == 2) ? 16 : 4;
    static constexpr int kPitchK = D + kPadK;     // elements
    static constexpr int kPitchV = D + kPadV;
    static constexpr int kVec = 16 / sizeof(T);   // elements per 16-byte load
    static constexpr int kChunksPerRow = D / kVec;
    static constexpr int kRowsPerPass = kDenseThreads / kChunksPerRow;
    static constexpr int kPasses = BN / kRowsPerPass;
    static_assert(kPasses * kRowsPerPass == BN, "tile load shape");
};

// ---------------------------------------------------------------- bf16 ----
// K and V tiles move global -> LDS by DMA (global_load_lds_dwordx4: each wave
// writes one contiguous 1 KB run, lane l at byte 16*l), double-buffered in
// four separate LDS arrays so that reads of one buffer never wait on DMA into
// another.  Rows are unpadded; the 16-byte chunk c of key row r is stored at
// chunk c ^ swz<D>(r).  The LDS has 64 banks of 4 bytes (256 B per cycle):
// a 16-lane ds_read_b128 of 16 consecutive rows at one chunk (K, A operand)
// and a 32-lane transposed read of 4 consecutive rows x 4 consecutive chunks
// (V) then both touch every bank exactly once.
//
// Per iteration kt (one barrier):
//   wait for own DMA, barrier      K(kt+1), V(kt) now in LDS; previous reads done
//   DMA K(kt+2), V(kt+1)           into the buffers freed by the barrier
//   S(kt+1) = K(kt+1) Q^T          MFMA, overlaps the softmax of S(kt) below
//   P = softmax(S(kt)), O^T += V(kt)^T P^T
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);  // 16 chunks per row
    else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);              // 8 chunks, 2 rows per 256 B
}

template <int D>
struct DenseBf16Geom {
    static constexpr int BN = 64;                  // keys per tile
    static constexpr int kCpr = D / 8;             // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kCpr; // rows per wave DMA (1 KB)
    static constexpr int kLoadsPerWave = BN / kRowsPerLoad / 4;
    static constexpr int kTileElems = BN * D;
};

template <int D>
__device__ __forceinline__ const HET_LDS void *lds_chunk(const __bf16 *buf, int row, int chunk) {
    return (const HET_LDS void *)(buf + row * D + 8 * (chunk ^ swz<D>(row)));
}

template <int D>
__global__ __launch_bounds__(kDenseThreads, 2) void dense_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ o, const int32_t *__restrict__ dense_idx,
    const int32_t *__restrict__ counts, int N, int H, float scale_log2, int tiles_per_bh,
    int n_units) {
    using G = DenseBf16Geom<D>;
    constexpr int BN = G::BN;
    __shared__ __attribute__((aligned(1024))) __bf16 K0[G::kTileElems];
    __shared__ __attribute__((aligned(1024))) __bf16 K1[G::kTileElems];
    __shared__ __attribute__((aligned(1024))) __bf16 V0[G::kTileElems];
    __shared__ __attribute__((aligned(1024))) __bf16 V1[G::kTileElems];

    const int unit = xcd_remap(blockIdx.x, gridDim.x);
    if (unit >= n_units) return;
    const int tile = unit % tiles_per_bh, bh = unit / tiles_per_bh;
    const int h = bh % H, b = bh / H;
    const int n_dense = counts[2 * b];
    if (tile * kDenseBM >= n_dense) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int tok_stride = H * D;
    const __bf16 *kb = k + (size_t)b * N * tok_stride + (size_t)h * D;
    const __bf16 *vb = v + (size_t)b * N * tok_stride + (size_t)h * D;

    // Gathered query of this lane (col = query within the wave's 32).
    const int qrow = tile * kDenseBM + wave * 32 + col;
    const bool q_valid = qrow < n_dense;
    const int tok = q_valid ? dense_idx[(size_t)b * N + qrow] : 0;
    bf16x8 qf[D / 16];
    {
        const __bf16 *qp = q + ((size_t)b * N + tok) * tok_stride + (size_t)h * D + 8 * half;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) qf[c] = q_valid ? *(const bf16x8 *)(qp + 16 * c) : bf16x8{};
    }

    // DMA geometry: load j of this wave fills tile rows r0_j .. r0_j + kRowsPerLoad.
    int dma_row[G::kLoadsPerWave], dma_off[G::kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < G::kLoadsPerWave; ++j) {
        const int r0 = (wave * G::kLoadsPerWave + j) * G::kRowsPerLoad;
        const int r = r0 + lane / G::kCpr, p = lane % G::kCpr;
        dma_row[j] = r;
        dma_off[j] = 8 * (p ^ swz<D>(r));
    }
    const int n_tiles = (N + BN - 1) / BN;
    auto dma = [&](const __bf16 *src, __bf16 *dst, int kt) {
        const int key0 = kt * BN;
        const bool ragged = key0 + BN > N;
#pragma unroll
        for (int j = 0; j < G::kLoadsPerWave; ++j) {
            const int key = ragged ? imin(key0 + dma_row[j], N - 1) : key0 + dma_row[j];
            const __bf16 *gp = src + (size_t)key * tok_stride + dma_off[j];
            __bf16 *lp = dst + (wave * G::kLoadsPerWave + j) * G::kRowsPerLoad * D;
            __builtin_amdgcn_global_load_lds((const void *)gp, (HET_LDS void *)lp, 16, 0, 0);
        }
    };

    // S^T = K Q^T for the two 32-key blocks of a tile (raw scores).
    auto qk = [&](const __bf16 *Kt, f32x16 (&s)[2]) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x16{};
            const int row = blk * 32 + col;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 a = *(const HET_LDS bf16x8 *)lds_chunk<D>(Kt, row, 2 * c + half);
                s[blk] = mfma32_bf16(a, qf[c], s[blk]);
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_ref = -__builtin_inff();  // reference max, log2 units
    float l_part = 0.0f;

    // Transposed V read: lane j16 of each 16-lane group points at tile row
    // (base + 4*half + j16/4), element column 16*(g16&1) + 4*(j16&3) of a
    // 32-column slab, i.e. chunk 2*(g16&1) + (j16&3)/2, byte 8*(j16&1).
    const int g16 = lane >> 4, j16 = lane & 15;
    const int v_row_off = 4 * half + (j16 >> 2);
    const int v_chunk_off = 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int v_elem_off = 4 * (j16 & 1);

    // softmax(S(kt)) and O^T += V(kt)^T P^T.
    auto softmax_pv = [&](f32x16 (&s)[2], const __bf16 *Vt, int kt) {
        if (kt == n_tiles - 1 && kt * BN + BN > N) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kt * BN + blk * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    if (key >= N) s[blk][i] = -__builtin_inff();
                }
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[blk][i]);
        mx = half_pair_max(mx) * scale_log2;
        const bool grow = mx > m_ref + kRescaleSlack;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_ref;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
            m_ref = m_new;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }
        const float neg_m = -m_ref;
        // P as the B operand: chunk c of block blk = registers 8c..8c+7,
        // i.e. keys 16c + 8(j/4) + 4*half + j%4 (j < 8) of the block.
        bf16x8 pf[2][2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4 w;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][8 * c + 2 * j], scale_log2, neg_m));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][8 * c + 2 * j + 1], scale_log2, neg_m));
                    l_part += p0 + p1;
                    w[j] = pack_bf16x2(p0, p1);
                }
                pf[blk][c] = __builtin_bit_cast(bf16x8, w);
            }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int row = blk * 32 + 16 * c + v_row_off;
                    const int chunk = 4 * db + v_chunk_off;
                    const bf16x4 lo = lds_read_tr16((const HET_LDS void *)(Vt + row * D + 8 * (chunk ^ swz<D>(row)) + v_elem_off));
                    const bf16x4 hi = lds_read_tr16((const HET_LDS void *)(Vt + (row + 8) * D + 8 * (chunk ^ swz<D>(row + 8)) + v_elem_off));
                    oacc[db] = mfma32_bf16(concat8(lo, hi), pf[blk][c], oacc[db]);
                }
    };

    // Prologue: K(0), V(0), K(1) in flight; S(0) from K(0).
    dma(kb, K0, 0);
    dma(vb, V0, 0);
    if (n_tiles > 1) dma(kb, K1, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    f32x16 s_cur[2], s_nxt[2];
    qk(K0, s_cur);

    // One step: Kc holds K(kt+1), Kn receives K(kt+2), Vc holds V(kt), Vn receives V(kt+1).
    auto step = [&](int kt, const __bf16 *Kc, __bf16 *Kn, const __bf16 *Vc, __bf16 *Vn) {
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        if (kt + 2 < n_tiles) dma(kb, Kn, kt + 2);
        if (kt + 1 < n_tiles) {
            dma(vb, Vn, kt + 1);
            qk(Kc, s_nxt);
        }
        softmax_pv(s_cur, Vc, kt);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) s_cur[blk] = s_nxt[blk];
    };
    for (int kt = 0; kt < n_tiles; kt += 2) {
        step(kt, K1, K0, V0, V1);
        if (kt + 1 < n_tiles) step(kt + 1, K0, K1, V1, V0);
    }

    if (!q_valid) return;
    const float inv_l = 1.0f / half_pair_sum(l_part);
    __bf16 *op = o + ((size_t)b * N + tok) * tok_stride + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = db * 32 + 8 * i4 + 4 * half;
            u32x2 w;
            w[0] = pack_bf16x2(oacc[db][4 * i4 + 0] * inv_l, oacc[db][4 * i4 + 1] * inv_l);
            w[1] = pack_bf16x2(oacc[db][4 * i4 + 2] * inv_l, oacc[db][4 * i4 + 3] * inv_l);
            *(u32x2 *)(op + d) = w;
        }
    }
}

// ----------------------------------------------------------------- f32 ----
// Same structure with v_mfma_f32_32x32x2_f32 (k = 2 per instruction) and a
// 32-key tile; used for fp32 inputs, where bf16 rounding would not meet the
// fp32 tolerance.
template <int D>
__global__ __launch_bounds__(kDenseThreads) void dense_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ o, const int32_t *__restrict__ dense_idx,
    const int32_t *__restrict__ counts, int N, int H, float scale_log2) {
    constexpr int BN = 32;
    using Tl = DenseTile<float, D, BN>;
    __shared__ __attribute__((aligned(16))) float Ks[BN * Tl::kPitchK];
    __shared__ __attribute__((aligned(16))) float Vs[BN * Tl::kPitchV];

    const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int n_dense = counts[2 * b];
    if (tile * kDenseBM >= n_dense) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const size_t tok_stride = (size_t)H * D;
    const float *kb = k + (size_t)b * N * tok_stride + (size_t)h * D;
    const float *vb = v + (size_t)b * N * tok_stride + (size_t)h * D;

    const int qrow = tile * kDenseBM + wave * 32 + col;
    const bool q_valid = qrow < n_dense;
    const int tok = q_valid ? dense_idx[(size_t)b * N + qrow] : 0;
    float qf[D / 2];
    {
        const float *qp = q + ((size_t)b * N + tok) * tok_stride + (size_t)h * D + half;
#pragma unroll
        for (int c = 0; c < D / 2; ++c) qf[c] = q_valid ? qp[2 * c] : 0.0f;
    }

    u32x4 kreg[Tl::kPasses], vreg[Tl::kPasses];
    const int ld_row = tid / Tl::kChunksPerRow, ld_chunk = tid % Tl::kChunksPerRow;
    auto fetch = [&](int kt) {
#pragma unroll
        for (int p = 0; p < Tl::kPasses; ++p) {
            const int key = kt * BN + p * Tl::kRowsPerPass + ld_row;
            if (key < N) {
                kreg[p] = *(const u32x4 *)(kb + (size_t)key * tok_stride + ld_chunk * Tl::kVec);
                vreg[p] = *(const u32x4 *)(vb + (size_t)key * tok_stride + ld_chunk * Tl::kVec);
            } else {
                kreg[p] = u32x4{0, 0, 0, 0};
                vreg[p] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int p = 0; p < Tl::kPasses; ++p) {
            const int r = p * Tl::kRowsPerPass + ld_row;
            *(u32x4 *)(Ks + r * Tl::kPitchK + ld_chunk * Tl::kVec) = kreg[p];
            *(u32x4 *)(Vs + r * Tl::kPitchV + ld_chunk * Tl::kVec) = vreg[p];
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;

    const int n_tiles = (N + BN - 1) / BN;
    fetch(0);
    stash();
    __syncthreads();
    for (int kt = 0; kt < n_tiles; ++kt) {
        if (kt + 1 < n_tiles) fetch(kt + 1);

        f32x16 s = f32x16{};
        const float *krow = Ks + col * Tl::kPitchK + half;
#pragma unroll
        for (int c = 0; c < D / 2; ++c) s = mfma32_f32(krow[2 * c], qf[c], s);

        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = s[i] * scale_log2;
            const int key = kt * BN + 8 * (i / 4) + 4 * half + (i % 4);
            if (key >= N) x = -__builtin_inff();
            s[i] = x;
            mx = fmaxf(mx, x);
        }
        mx = half_pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
            l_part += s[i];
        }
        // MFMA i: both halves contribute register i = key 8(i/4) + 4*half + i%4.
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = Vs[(8 * (i / 4) + 4 * half + (i % 4)) * Tl::kPitchV + db * 32 + col];
                oacc[db] = mfma32_f32(a, s[i], oacc[db]);
            }
        }

        __syncthreads();
        if (kt + 1 < n_tiles) {
            stash();
            __syncthreads();
        }
    }

    if (!q_valid) return;
    const float inv_l = 1.0f / half_pair_sum(l_part);
    float *op = o + ((size_t)b * N + tok) * tok_stride + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = db * 32 + 8 * i4 + 4 * half;
            f32x4 w = {oacc[db][4 * i4 + 0] * inv_l, oacc[db][4 * i4 + 1] * inv_l,
                       oacc[db][4 * i4 + 2] * inv_l, oacc[db][4 * i4 + 3] * inv_l};
            *(f32x4 *)(op + d) = w;
        }
    }
}

hipError_t launch_dense(const AttnArgs &a, hipStream_t stream) {
    if (a.max_dense <= 0) return hipSuccess;
    const dim3 grid((a.max_dense + kDenseBM - 1) / kDenseBM, a.heads, a.batch);
    const float sl2 = a.scale * kLog2e;
    if (a.bf16) {
        auto q = (const __bf16 *)a.q, k = (const __bf16 *)a.k, v = (const __bf16 *)a.v;
        auto o = (__bf16 *)a.o;
        const int tiles = (a.max_dense + kDenseBM - 1) / kDenseBM;
        const int units = tiles * a.heads * a.batch;
        const dim3 g1d((units + 7) / 8 * 8);
        if (a.head_dim == 128)
            hipLaunchKernelGGL(dense_bf16_kernel<128>, g1d, dim3(kDenseThreads), 0, stream, q, k, v, o,
                               a.dense_idx, a.counts, a.n, a.heads, sl2, tiles, units);
        else
            hipLaunchKernelGGL(dense_bf16_kernel<64>, g1d, dim3(kDenseThreads), 0, stream, q, k, v, o,
                               a.dense_idx, a.counts, a.n, a.heads, sl2, tiles, units);
    } else {
        auto q = (const float *)a.q, k = (const float *)a.k, v = (const float *)a.v;
        auto o = (float *)a.o;
        if (a.head_dim == 128)
            hipLaunchKernelGGL(dense_f32_kernel<128>, grid, dim3(kDenseThreads), 0, stream, q, k, v, o,
                               a.dense_idx, a.counts, a.n, a.heads, sl2);
        else
            hipLaunchKernelGGL(dense_f32_kernel<64>, grid, dim3(kDenseThreads), 0, stream, q, k, v, o,
                               a.dense_idx, a.counts, a.n, a.heads, sl2);
    }
    return hipGetLastError();
}

}  // namespace hetattn
