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

template <int D>
__global__ __launch_bounds__(kDenseThreads, 2) void dense_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ o, const int32_t *__restrict__ dense_idx,
    const int32_t *__restrict__ counts, int N, int H, float scale_log2, int tiles_per_bh,
    int n_units) {
    constexpr int BN = 64;
    using Tl = DenseTile<__bf16, D, BN>;
    __shared__ __attribute__((aligned(16))) __bf16 Ks[BN * Tl::kPitchK];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[BN * Tl::kPitchV];

    const int unit = xcd_remap(blockIdx.x, gridDim.x);
    if (unit >= n_units) return;
    const int tile = unit % tiles_per_bh, bh = unit / tiles_per_bh;
    const int h = bh % H, b = bh / H;
    const int n_dense = counts[2 * b];
    if (tile * kDenseBM >= n_dense) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const size_t tok_stride = (size_t)H * D;
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
        for (int c = 0; c < D / 16; ++c) {
            qf[c] = q_valid ? *(const bf16x8 *)(qp + 16 * c) : bf16x8{};
        }
    }

    // Register staging of one K/V tile.
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
    float m_ref = -__builtin_inff();  // reference max, log2 units
    float l_part = 0.0f;

    // Transposed-read coordinates of V (see the O^T update below).
    const int g16 = lane >> 4, j16 = lane & 15;
    const int v_key_off = 4 * half + (j16 >> 2);
    const int v_col_off = 16 * (g16 & 1) + 4 * (j16 & 3);

    const int n_tiles = (N + BN - 1) / BN;
    fetch(0);
    stash();
    __syncthreads();
    for (int kt = 0; kt < n_tiles; ++kt) {
        if (kt + 1 < n_tiles) fetch(kt + 1);

        // ---- S^T = K Q^T for two 32-key blocks (raw scores)
        f32x16 s[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x16{};
            const __bf16 *krow = Ks + (blk * 32 + col) * Tl::kPitchK + 8 * half;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const bf16x8 a = *(const bf16x8 *)(krow + 16 * c);
                s[blk] = mfma32_bf16(a, qf[c], s[blk]);
            }
        }
        if (kt == n_tiles - 1 && (kt + 1) * BN > N) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kt * BN + blk * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    if (key >= N) s[blk][i] = -__builtin_inff();
                }
        }

        // ---- online softmax (base 2, lazy rescale)
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

        // P as the B operand of O^T += V^T P^T: chunk c of block blk = registers 8c..8c+7,
        // i.e. keys 16c + 8(j/4) + 4*half + j%4 (j < 8) of the block.
        bf16x8 pf[2][2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
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
        }

        // ---- O^T += V^T P^T.  A operand rows = d, k = the 8 keys above; read
        // transposed from the row-major V tile: lane j of each 16-lane group
        // points at key (base + j/4), columns 4*(j%4) .. +3 of its 16-column slab.
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const __bf16 *base = Vs + (blk * 32 + 16 * c + v_key_off) * Tl::kPitchV + db * 32 + v_col_off;
                    const bf16x4 lo = lds_read_tr16((const HET_LDS void *)base);
                    const bf16x4 hi = lds_read_tr16((const HET_LDS void *)(base + 8 * Tl::kPitchV));
                    oacc[db] = mfma32_bf16(concat8(lo, hi), pf[blk][c], oacc[db]);
                }
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
