// local.hip -- softmax attention over a 3D window for the local tokens.
//
// [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
// Video Diffusion" (HetA-DiT): local attention of §3.1.1 Eq. 3 over a fixed
// 3D neighbourhood of the latent grid (§5.1, "predefined 3D neighborhood")
// for the tokens with m_i = 1 (§3.2.2 Eqs. 12-13).  This is the
// (1-rho)*N*M*d_h term of the cost model (§3.2.2 Eq. 14).
//
// Query tiles are 32 grid positions of one frame of one (sample, head).
// Because the window is shifted rather than cut at the border, the union of
// a tile's windows is a box (frames x rows x columns); it is walked in key
// blocks of 32 slots, each block holding 32/SR box rows of SR column slots,
// so every key block is one 32x32 MFMA tile, and per (query, key) a mask
// keeps only the query's own window.  Dense tokens inside a tile ride along
// and are not stored.
//
// local_band_kernel (bf16, the layer's local kernel and its statistics and
// gradient forms): 8-wave workgroups share one key box streamed through LDS
// in bands by buffer DMA; see its comment below.
// local_f32_kernel (fp32 inputs, for fp32 parity): one wave per 4x8 tile, K
// rows straight from global memory into the MFMA, V through a per-wave LDS
// slab.
#include "common.hpp"
#include "kernels.hpp"

namespace hetattn {

constexpr int kLocalQY = 4;
constexpr int kLocalQX = 8;

// fp32 form: one wave = one query tile of 4 (h) x 8 (w) grid positions at
// one t, v_mfma_f32_32x32x2_f32.  The tiles are ordered (sample, head, t, y,
// x) and dealt to XCDs in contiguous runs, so that neighbouring tiles, whose
// key boxes overlap, share one L2.  The next key block's K and V are fetched
// into registers while the current block computes; slots outside the box
// load a clamped in-grid address and are zeroed (V) or masked (scores), so
// no load is predicated.
template <int D, int SR>
__global__ __launch_bounds__(64) void local_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v, float *__restrict__ o,
    const uint8_t *__restrict__ mask, int N, int H, float scale_log2, LocalGeom g, int n_units) {
    constexpr int rpb = 32 / SR;                  // box rows per key block
    constexpr int kVec = 4;                       // floats per 16-byte load
    constexpr int kChunks = D / kVec;             // 16-byte chunks per row
    constexpr int kStage = 32 * kChunks / 64;     // V chunks staged per lane per block
    constexpr int kPitchV = D + 4;
    constexpr int kKRegs = D / 2;
    __shared__ __attribute__((aligned(16))) float Vs[32 * kPitchV];

    const int unit = xcd_remap(blockIdx.x, gridDim.x);
    if (unit >= n_units) return;
    const int tx = unit % g.tiles_x;
    int rest = unit / g.tiles_x;
    const int ty = rest % g.tiles_y;
    rest /= g.tiles_y;
    const int t = rest % g.T;
    rest /= g.T;
    const int h = rest % H, b = rest / H;

    const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
    const int ybase = ty * kLocalQY, xbase = tx * kLocalQX;

    // The query of this lane (col = query within the tile).
    const int y = ybase + col / kLocalQX, x = xbase + col % kLocalQX;
    const bool in_grid = y < g.Hg && x < g.Wg;
    const int tok = in_grid ? (t * g.Hg + y) * g.Wg + x : 0;
    const bool is_local = in_grid && mask[(size_t)b * N + tok] != 0;
    if (!__any(is_local)) return;

    // Window of this query, and the union box of the tile.
    const int t0 = win_lo(t, g.wt, g.lt, g.T, g.cut);
    const int nt = win_hi(t, g.wt, g.lt, g.T, g.cut) - t0;
    const int ylo = win_lo(imin(y, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut);
    const int yhi = win_hi(imin(y, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut);
    const int qxlo = win_lo(imin(x, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut);
    const int qxhi = win_hi(imin(x, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut);
    const int ylast = imin(ybase + kLocalQY - 1, g.Hg - 1), xlast = imin(xbase + kLocalQX - 1, g.Wg - 1);
    const int uy0 = win_lo(ybase, g.wh, g.lh, g.Hg, g.cut);
    const int ux0 = win_lo(xbase, g.ww, g.lw, g.Wg, g.cut);
    const int ny = win_hi(ylast, g.wh, g.lh, g.Hg, g.cut) - uy0;
    const int nx = win_hi(xlast, g.ww, g.lw, g.Wg, g.cut) - ux0;
    const int rows = nt * ny;
    const int n_blocks = (rows + rpb - 1) / rpb;

    const size_t tok_stride = (size_t)H * D;
    const float *kbase = k + (size_t)b * N * tok_stride + (size_t)h * D;
    const float *vbase = v + (size_t)b * N * tok_stride + (size_t)h * D;

    // Box row r -> token of its first column (rows past the box clamp to the
    // last row).  r is the same for the whole wave, so this runs on the SALU.
    auto row_token = [&](int r) HET_INLINE -> int {
        r = imin(r, rows - 1);
        const int tt = t0 + r / ny, yy = uy0 + r % ny;
        return (tt * g.Hg + yy) * g.Wg + ux0;
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;

    // Staging of one block: this lane's K row (A operand) and its share of V rows.
    float kf[kKRegs], kn[kKRegs];
    u32x4 vst[kStage];
    bool vok[kStage];
    // Slot s = rr*SR + xo of a block lies in box row rr of the block; slots
    // past the row (xo >= nx) or past the box load a clamped in-box address.
    auto fetch = [&](int kb, float *kdst) HET_INLINE {
        const int rt0 = row_token(kb * rpb), rt1 = row_token(kb * rpb + 1);
        const bool ok0 = kb * rpb < rows, ok1 = rpb > 1 && kb * rpb + 1 < rows;
        const int jk = ((col / SR) ? rt1 : rt0) + imin(col % SR, nx - 1);
        const float *kp = kbase + (size_t)jk * tok_stride;
#pragma unroll
        for (int c = 0; c < kKRegs; ++c) kdst[c] = kp[2 * c + half];
        // Lane stages slot (P*it + lane/kChunks), chunk lane%kChunks, P = 64/kChunks;
        // P*it % SR + P - 1 < SR, so the slot's row (P*it)/SR is known per it.
        constexpr int P = 64 / kChunks;
#pragma unroll
        for (int it = 0; it < kStage; ++it) {
            const int rr = (P * it) / SR;
            const int xo = (P * it) % SR + lane / kChunks;
            const int jv = (rr ? rt1 : rt0) + imin(xo, nx - 1);
            vok[it] = (rr ? ok1 : ok0) && xo < nx;
            vst[it] = *(const u32x4 *)(vbase + (size_t)jv * tok_stride + kVec * (lane % kChunks));
        }
    };
    auto stage_v = [&]() HET_INLINE {
#pragma unroll
        for (int it = 0; it < kStage; ++it) {
            const int e = lane + 64 * it, s = e / kChunks, ch = e % kChunks;
            const u32x4 val = vok[it] ? vst[it] : u32x4{0, 0, 0, 0};
            *(u32x4 *)(Vs + s * kPitchV + kVec * ch) = val;
        }
    };

    // Query operand.
    float qf[kKRegs];
    {
        const float *qp = q + ((size_t)b * N + tok) * tok_stride + (size_t)h * D;
#pragma unroll
        for (int c = 0; c < kKRegs; ++c) qf[c] = is_local ? qp[2 * c + half] : 0.0f;
    }

    fetch(0, kf);
    for (int kb = 0; kb < n_blocks; ++kb) {
        stage_v();
#pragma unroll
        for (int c = 0; c < kKRegs; ++c) kn[c] = kf[c];
        if (kb + 1 < n_blocks) fetch(kb + 1, kf);

        // S^T = K Q^T for this block.
        f32x16 s = f32x16{};
#pragma unroll
        for (int c = 0; c < kKRegs; ++c) s = mfma32_f32(kn[c], qf[c], s);

        // Keep only keys inside this query's window.  Register i holds slot
        // 8(i/4) + 4*half + i%4 of the block: box row (i/4 >= 2 && SR == 16),
        // column 8*((i/4) % (SR/8)) + 4*half + i%4.
        const int r0 = kb * rpb;
        const int yy0 = uy0 + imin(r0, rows - 1) % ny, yy1 = uy0 + imin(r0 + 1, rows - 1) % ny;
        const bool y_in0 = r0 < rows && yy0 >= ylo && yy0 < yhi;
        const bool y_in1 = rpb > 1 && r0 + 1 < rows && yy1 >= ylo && yy1 < yhi;
        // Columns of the query's window relative to the box, intersected with the box.
        const int xlo = qxlo - ux0, xhi = imin(qxhi - ux0, nx);
        float mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int xo = 8 * ((i / 4) % (SR / 8)) + 4 * half + (i % 4);
            const bool y_in = (SR == 16 && i >= 8) ? y_in1 : y_in0;
            const bool ok = y_in && xo >= xlo && xo < xhi;
            const float xv = ok ? s[i] : -__builtin_inff();
            s[i] = xv;
            mx = fmaxf(mx, xv);
        }
        // Online softmax in base 2 with a lazily moved reference max (see the
        // dense kernel): the reference moves only when a block's max exceeds
        // it by more than kRescaleSlack.  A block may hold none of this
        // query's keys (mx = -inf); the reference then stays put.
        mx = half_pair_max(mx) * scale_log2;
        const bool grow = mx > m_run + kRescaleSlack;
        if (__any(grow)) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            m_run = m_new;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        }
        const float m_use = (m_run == -__builtin_inff()) ? 0.0f : m_run;
        const float neg_m = -m_use;

        __syncthreads();  // V slab of this block visible to the whole wave
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], scale_log2, neg_m));
            l_part += s[i];
        }
        // MFMA i: both halves contribute register i = key 8(i/4) + 4*half + i%4.
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = Vs[(8 * (i / 4) + 4 * half + (i % 4)) * kPitchV + db * 32 + col];
                oacc[db] = mfma32_f32(a, s[i], oacc[db]);
            }
        }
        __syncthreads();  // slab free for the next block
    }

    if (!is_local) return;
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

// ------------------------------------------------------------ bf16 path ----
// One workgroup = WV waves = NF query frames x NW x-tiles of QY (h)
// x QX (w) = 32 queries, all on the rows ybase .. ybase+QY-1 (QY = 4 or 8,
// chosen per window: the tile whose key box takes the fewest 32-key blocks
// per frame).  The forward and statistics forms take one frame and 8
// x-tiles where that fills the waves about as well as 4, so that every wave
// has work in every band; else, and always in the gradient form (whose
// smaller box keeps its buffers' offsets within the LDS instructions'
// immediates), two frames (t, t+1) and 4 x-tiles.  The tiles of a
// workgroup share one key box: the frames [F0, F1) that the frames' windows
// cover x ny rows x C columns (the union of the tiles' column windows).  The box goes through LDS in bands of rpb = 32/SR rows of one
// frame (one MFMA key block per wave and band), double-buffered: the DMA of
// band i+1 runs while the waves work on band i.  Every K/V row of the box is
// read from L2 once per workgroup instead of once per tile.  A wave takes
// from each band the SR columns of its own tile's box (clamped at the edge of
// the workgroup box; such slots are masked) and skips bands outside its
// frame's window.
// Waves per workgroup (WV) and x-tiles per workgroup (NW): 8 and 8 (one
// query frame), 4 and 4 (one frame, two workgroups a CU) or 8 and 4 (two
// frames); the workgroup's query frames are WV / NW.

template <int D, int SR, int QX, int NW, int WV>
struct BandGeom {
    static constexpr int rpb = 32 / SR;                          // box rows per band
    static constexpr int kCpr = D / 8;                           // 16-byte chunks per token row
    static constexpr int kTokPerLoad = 64 / kCpr;                // token rows per wave DMA (1 KB)
    static constexpr int kMaxLw = SR == 16 ? 16 - QX + 1 : kLocalMaxWinW;
    // LDS rows per box row: the widest workgroup box, in whole DMA loads.
    static constexpr int kCb = (NW * QX + kMaxLw - 1 + kTokPerLoad - 1) / kTokPerLoad * kTokPerLoad;
    static_assert(kCb % kTokPerLoad == 0, "a DMA load's rows stay in one box row");
    static constexpr int kBandRows = rpb * kCb;
    static constexpr int kLoads = kBandRows / kTokPerLoad;      // DMA loads per tensor and band
    static constexpr int kLoadsPerWave = (kLoads + WV - 1) / WV;
    static constexpr int kBufElems = kBandRows * D;              // one tensor, one buffer
};


// Extra operands of the statistics and gradient forms of the band kernel.
struct BandGrad {
    const __bf16 *dout;  // kMode 2: dL/dO
    float *lse;          // kMode 1: written; kMode 0: written when not null; kMode 2: read
                         // ([b][h][n], log2 units)
    const float *dsum;   // kMode 2: D_i = dO_i . O_i ([b][h][n])
    __bf16 *dq;          // kMode 2: dQ rows of the local tokens
    float scale;         // kMode 2: softmax scale
};

// kMode 0: the layer's output O for the local tokens (and their LSE when
//          gr.lse is given).
// kMode 1: only the row statistics: LSE_i = m_i + log2(l_i) of each local
//          row (no V, no P*V), for the gradient of the layer.
// kMode 2: dQ of the local rows given their LSE and D (the gradient, with
//          the route held fixed): per band S^T = K Q^T and dP^T = V dO^T
//          (K and V rows as A operands), P = exp2(S - LSE) inside the
//          window, dS = P (dP - D), dQ^T += K^T dS^T (K read transposed).
template <int D, int SR, int QY, int kMode, int NW, int WV>
__global__ __launch_bounds__(64 * WV, 2) void local_band_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ o, const uint8_t *__restrict__ mask, int N, int H, float scale_log2, LocalGeom g,
    int n_units, int x_blocks, int t_groups, BandGrad gr) {
    constexpr int QX = 32 / QY;
    constexpr int NF = WV / NW;
    using Bg = BandGeom<D, SR, QX, NW, WV>;
    constexpr int rpb = Bg::rpb, NC = D / 16, NDB = D / 32;
    __shared__ __attribute__((aligned(1024))) __bf16 Kb0[Bg::kBufElems];
    __shared__ __attribute__((aligned(1024))) __bf16 Kb1[Bg::kBufElems];
    __shared__ __attribute__((aligned(1024))) __bf16 Vb0[Bg::kBufElems];
    __shared__ __attribute__((aligned(1024))) __bf16 Vb1[Bg::kBufElems];

    const int unit = xcd_remap(blockIdx.x, gridDim.x);
    if (unit >= n_units) return;  // the whole workgroup
    int rest = unit;
    const int xb = rest % x_blocks;
    rest /= x_blocks;
    const int ty = rest % g.tiles_y;
    rest /= g.tiles_y;
    const int tp = rest % t_groups;
    rest /= t_groups;
    const int h = rest % H, b = rest / H;

    // The wave index as a wave-uniform (scalar) value: the DMA's LDS addresses
    // and the tile of each wave are then scalar too.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int gq = lane >> 4, j16 = lane & 15;

    // Workgroup box (uniform).
    const int ybase = ty * QY;
    const int uy0 = win_lo(ybase, g.wh, g.lh, g.Hg, g.cut);
    const int ny = win_hi(imin(ybase + QY - 1, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut) - uy0;
    const int xt0 = xb * NW, xt1 = imin(xt0 + NW, g.tiles_x) - 1;
    const int ux0 = win_lo(xt0 * QX, g.ww, g.lw, g.Wg, g.cut);
    const int C = win_hi(imin(xt1 * QX + QX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut) - ux0;
    const int tA = NF * tp, tB = imin(tA + NF - 1, g.T - 1);
    const int F0 = win_lo(tA, g.wt, g.lt, g.T, g.cut);
    const int F1 = win_hi(tB, g.wt, g.lt, g.T, g.cut);
    const int nb_f = (ny + rpb - 1) / rpb;
    const int n_bands = (F1 - F0) * nb_f;

    // This wave's tile and this lane's query.
    const int xt = xt0 + wave % NW;
    const int t = tA + wave / NW;
    const bool wave_on = t < g.T && xt < g.tiles_x;
    const int xbase = xt * QX;
    const int y = ybase + col / QX, x = xbase + col % QX;
    const bool in_grid = wave_on && y < g.Hg && x < g.Wg;
    const int tok = in_grid ? (t * g.Hg + y) * g.Wg + x : 0;
    const bool is_local = in_grid && mask[(size_t)b * N + tok] != 0;
    const bool active = __any(is_local);
    // A workgroup whose queries are all dense has nothing to do.
    // (The flags go through the second K buffer, which no DMA fills before
    // the first band's barrier; no other LDS, so that two four-wave
    // workgroups fit a CU.)
    {
        uint32_t *flag = reinterpret_cast<uint32_t *>(Kb1);
        if (lane == 0) flag[wave] = active ? 1u : 0u;
        __syncthreads();
        uint32_t any_local = 0u;
#pragma unroll
        for (int w = 0; w < WV; ++w) any_local |= flag[w];
        if (any_local == 0u) return;
    }
    const int t0 = win_lo(imin(t, g.T - 1), g.wt, g.lt, g.T, g.cut);
    const int t1 = win_hi(imin(t, g.T - 1), g.wt, g.lt, g.T, g.cut);
    const int ylo = win_lo(imin(y, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut);
    const int yhi = win_hi(imin(y, g.Hg - 1), g.wh, g.lh, g.Hg, g.cut);
    const int qxlo = win_lo(imin(x, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut);
    const int qxhi = win_hi(imin(x, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut);
    const int uxw = win_lo(imin(xbase, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut);
    const int nxw = win_hi(imin(xbase + QX - 1, g.Wg - 1), g.ww, g.lw, g.Wg, g.cut) - uxw;
    const int cw = uxw - ux0;  // this tile's box inside the workgroup box

    const size_t tok_stride = (size_t)H * D;
    bf16x8 qf[NC];
    {
        const __bf16 *qp = q + ((size_t)b * N + tok) * tok_stride + (size_t)h * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) qf[c] = is_local ? *(const bf16x8 *)(qp + 16 * c) : bf16x8{};
    }
    const size_t row_bh = ((size_t)b * H + h) * N;
    // kMode 2: this lane's dO row, LSE and D.
    bf16x8 df[kMode == 2 ? NC : 1];
    float lse_i = 0.0f, d_i = 0.0f;
    if constexpr (kMode == 2) {
        const __bf16 *dp_ = gr.dout + ((size_t)b * N + tok) * tok_stride + (size_t)h * D + 8 * half;
#pragma unroll
        for (int c = 0; c < NC; ++c) df[c] = is_local ? *(const bf16x8 *)(dp_ + 16 * c) : bf16x8{};
        lse_i = is_local ? gr.lse[row_bh + tok] : 0.0f;
        d_i = is_local ? gr.dsum[row_bh + tok] : 0.0f;
    }

    // LDS row of key slot s (0..31) of this wave's block: box row s/SR of the
    // band, column cw + s%SR, clamped to the box.
    auto band_row = [&](int s) HET_INLINE -> int {
        const int rr = s / SR, cc = s % SR;
        return rr * Bg::kCb + imin(cw + cc, C - 1);
    };
    int k_off[NC];  // K, A operand: slot col, chunk 2c+half
    {
        const int row = band_row(col);
#pragma unroll
        for (int c = 0; c < NC; ++c) k_off[c] = row * D + 8 * ((2 * c + half) ^ swz<D>(row));
    }
    // V, transposed read of key chunk c2 (slots 16*c2 ..), rows +8*lohi, 32-column slab db.
    int v_off[2][2][NDB];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int lohi = 0; lohi < 2; ++lohi) {
            const int row = band_row(16 * c2 + 4 * half + (j16 >> 2) + 8 * lohi);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                v_off[c2][lohi][db] =
                    row * D + 8 * ((4 * db + 2 * (gq & 1) + ((j16 & 3) >> 1)) ^ swz<D>(row)) + 4 * (j16 & 1);
        }
    // DMA: load i (i = wave + WV*j) fills LDS rows [i*kTokPerLoad, ..);
    // this lane writes row R = i*kTokPerLoad + lane/kCpr at chunk position
    // lane%kCpr.  Row R = rr*kCb + c holds column c of band row rr; the byte
    // offset from the band's first token is fixed per lane.  Columns past
    // the box get an offset beyond any descriptor's range: they read as
    // zeros and cost no memory traffic (no read ever reaches them).
    int dma_voff[Bg::kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < Bg::kLoadsPerWave; ++j) {
        const int i = wave + WV * j;
        const int R = i * Bg::kTokPerLoad + lane / Bg::kCpr;
        const int rr = R / Bg::kCb, c = R % Bg::kCb;
        dma_voff[j] = c < C ? 2 * ((rr * g.Wg + c) * (int)tok_stride + 8 * ((lane % Bg::kCpr) ^ swz<D>(R)))
                            : 0x7ffffff0;
    }
    // Loads whose rows all lie past the box's C columns are not issued (a
    // load's rows are kTokPerLoad consecutive columns of one box row, since
    // kCb is a multiple of kTokPerLoad); no read reaches those LDS rows.
    uint32_t dma_live = 0;
    {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int j = 0; j < Bg::kLoadsPerWave; ++j) {
            const int i = wv + WV * j;
            if (i < Bg::kLoads && (i * Bg::kTokPerLoad) % Bg::kCb < C) dma_live |= 1u << j;
        }
    }
    const __bf16 *kbase = k + (size_t)b * N * tok_stride + (size_t)h * D;
    const __bf16 *vbase = v + (size_t)b * N * tok_stride + (size_t)h * D;
    // Bands go (frame, row of bands) in order; (c_f, c_r) is the band being
    // computed and (d_f, d_r) the next one to fetch, advanced step by step
    // (no division in the loop).
    int c_f = F0, c_r = 0, d_f = F0, d_r = 0;
    auto next_band = [&](int &f, int &r) HET_INLINE {
        if (++r == nb_f) {
            r = 0;
            ++f;
        }
    };
    // The next band -> LDS.  The descriptors end at token N of this sample,
    // so a second band row past the grid reads zeros (its slots are masked).
    auto dma_band = [&](__bf16 *Kd, __bf16 *Vd) HET_INLINE {
        const int f = d_f, yy0 = uy0 + d_r * rpb;
        next_band(d_f, d_r);
        const int tok0 = (f * g.Hg + yy0) * g.Wg + ux0;
        const uint32_t bytes = (uint32_t)((N - tok0) * (int)tok_stride) * 2u;
        const __bf16 *kp = kbase + (size_t)tok0 * tok_stride, *vp = vbase + (size_t)tok0 * tok_stride;
#pragma unroll
        for (int j = 0; j < Bg::kLoadsPerWave; ++j) {
            const int i = wave + WV * j;
            if ((dma_live >> j) & 1u) {
                buffer_load_lds16(kp, bytes, (HET_LDS void *)(Kd + i * Bg::kTokPerLoad * D), dma_voff[j]);
                if constexpr (kMode != 1)
                    buffer_load_lds16(vp, bytes, (HET_LDS void *)(Vd + i * Bg::kTokPerLoad * D), dma_voff[j]);
            }
        }
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    // Columns of this query's window relative to the tile box, inside the box.
    const int xlo = qxlo - uxw, xhi = imin(qxhi - uxw, nxw);

    // Band bi is read from (Kc, Vc) while the DMA of band bi+1 goes to
    // (Kn, Vn).  The buffers are fixed at each call site (the loop is
    // unrolled by two), so the compiler can see that the reads of one buffer
    // do not wait on the DMA into the other.
    auto step = [&](int bi, const __bf16 *Kc, const __bf16 *Vc, __bf16 *Kn, __bf16 *Vn) HET_INLINE {
        // Band bi has landed for every wave, and every wave is done with
        // band bi-1, whose buffers the next DMA refills.
        // A wave waits for the band at the lowest priority and computes it at
        // a raised one, so that on a SIMD shared by two workgroups the wave
        // that has its band goes first.
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        if (bi + 1 < n_bands) dma_band(Kn, Vn);
        __builtin_amdgcn_s_setprio(1);
        const int f = c_f, yy0 = uy0 + c_r * rpb;
        next_band(c_f, c_r);
        if (!active || f < t0 || f >= t1) return;
        // Register i holds slot 8(i/4) + 4*half + i%4 of the block: box row
        // (i/4 >= 2 && SR == 16), column 8*((i/4) % (SR/8)) + 4*half + i%4;
        // in_win(i): that key is inside this query's window.
        const bool y_in0 = yy0 < uy0 + ny && yy0 >= ylo && yy0 < yhi;
        const bool y_in1 = rpb > 1 && yy0 + 1 < uy0 + ny && yy0 + 1 >= ylo && yy0 + 1 < yhi;
        auto in_win = [&](int i) HET_INLINE {
            const int xo = 8 * ((i / 4) % (SR / 8)) + 4 * half + (i % 4);
            const bool y_in = (SR == 16 && i >= 8) ? y_in1 : y_in0;
            return y_in && xo >= xlo && xo < xhi;
        };

        if constexpr (kMode == 2) {
            // S^T and dP^T of the block (K and V rows), then the transposed
            // K reads land while dS is formed.
            bf16x8 ka[NC], va[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                ka[c] = *(const HET_LDS bf16x8 *)(Kc + k_off[c]);
                va[c] = *(const HET_LDS bf16x8 *)(Vc + k_off[c]);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                s = mfma32_bf16(ka[c], qf[c], s);
                dp = mfma32_bf16(va[c], df[c], dp);
            }
            bf16x4 kr[2][2][NDB];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int lohi = 0; lohi < 2; ++lohi)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        kr[c2][lohi][db] = lds_read_tr16((const HET_LDS void *)(Kc + v_off[c2][lohi][db]));
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 sf[2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                u32x4 w;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float d2[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int i = 8 * c2 + 2 * jj + e;
                        const float p =
                            in_win(i) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], scale_log2, -lse_i)) : 0.0f;
                        d2[e] = p * (dp[i] - d_i);
                    }
                    w[jj] = pack_bf16x2(d2[0], d2[1]);
                }
                sf[c2] = __builtin_bit_cast(bf16x8, w);
            }
            // dQ^T += K^T dS^T (accumulated in oacc).
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
                    oacc[db] = mfma32_bf16(concat8(kr[c2][0][db], kr[c2][1][db]), sf[c2], oacc[db]);
            return;
        }

        // All LDS operands of the block are requested up front: the K reads
        // feed the QK product, the V reads land while the softmax runs.
        bf16x8 ka[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[c] = *(const HET_LDS bf16x8 *)(Kc + k_off[c]);
        bf16x4 vr[2][2][kMode == 0 ? NDB : 1];
        if constexpr (kMode == 0) {
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int lohi = 0; lohi < 2; ++lohi)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        vr[c2][lohi][db] = lds_read_tr16((const HET_LDS void *)(Vc + v_off[c2][lohi][db]));
        }
        __builtin_amdgcn_sched_barrier(0);
        // S^T = K Q^T for this wave's key block.
        f32x16 s = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) s = mfma32_bf16(ka[c], qf[c], s);

        // Keep only keys inside this query's window.
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = in_win(i) ? s[i] : -__builtin_inff();
        // Online softmax in base 2 with a lazily moved reference max (see the
        // dense kernel): the reference is set on a query's first block with
        // keys and moves only when a block's exponentials ran large -- with
        // every score <= reference + kRescaleSlack a lane's 16 exponentials
        // sum to at most 16 * 2^kRescaleSlack, so a larger (or non-finite) sum
        // sends the block through the exact max and its exponentials are
        // taken again.  A block may hold none of this query's keys.
        auto rescale = [&]() HET_INLINE {
            float mx = -__builtin_inff();
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
            mx = half_pair_max(mx) * scale_log2;
            const bool grow = mx > m_run + kRescaleSlack;
            if (__builtin_expect(__any(grow), 0)) {
                const float m_new = grow ? mx : m_run;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
                m_run = m_new;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            }
        };
        bf16x8 pf[2];
        auto exps = [&]() HET_INLINE -> float {
            const float neg_m = -((m_run == -__builtin_inff()) ? 0.0f : m_run);
            float tsum = 0.0f;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                u32x4 w;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * c2 + 2 * jj], scale_log2, neg_m));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * c2 + 2 * jj + 1], scale_log2, neg_m));
                    tsum += p0 + p1;
                    if constexpr (kMode == 0) w[jj] = pack_bf16x2(p0, p1);
                }
                if constexpr (kMode == 0) pf[c2] = __builtin_bit_cast(bf16x8, w);
            }
            return tsum;
        };
        constexpr float kBlockSumLimit = 16.0f * (float)(1 << (int)kRescaleSlack);
        if (__builtin_expect(__any(m_run == -__builtin_inff()), 0)) rescale();
        float tsum = exps();
        if (__builtin_expect(__any(!(tsum <= kBlockSumLimit)), 0)) {
            rescale();
            tsum = exps();
        }
        l_part += tsum;
        // O^T += V^T P^T.
        if constexpr (kMode == 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
                    oacc[db] = mfma32_bf16(concat8(vr[c2][0][db], vr[c2][1][db]), pf[c2], oacc[db]);
        }
    };

    dma_band(Kb0, Vb0);
    for (int bi = 0; bi < n_bands; bi += 2) {
        step(bi, Kb0, Vb0, Kb1, Vb1);
        if (bi + 1 < n_bands) step(bi + 1, Kb1, Vb1, Kb0, Vb0);
    }

    if (!is_local) return;
    if constexpr (kMode == 1) {
        const float l_tot = half_pair_sum(l_part);
        if (half == 0) gr.lse[row_bh + tok] = m_run + __builtin_log2f(l_tot);
        return;
    }
    const float l_tot = half_pair_sum(l_part);
    // kMode 0: the row's LSE for the gradient, when asked for.
    if (kMode == 0 && gr.lse != nullptr && half == 0) gr.lse[row_bh + tok] = m_run + __builtin_log2f(l_tot);
    const float mul = kMode == 2 ? gr.scale : 1.0f / l_tot;
    __bf16 *op = (kMode == 2 ? gr.dq : o) + ((size_t)b * N + tok) * tok_stride + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = db * 32 + 8 * i4 + 4 * half;
            u32x2 w;
            w[0] = pack_bf16x2(oacc[db][4 * i4 + 0] * mul, oacc[db][4 * i4 + 1] * mul);
            w[1] = pack_bf16x2(oacc[db][4 * i4 + 2] * mul, oacc[db][4 * i4 + 3] * mul);
            *(u32x2 *)(op + d) = w;
        }
}

namespace {

LocalGeom local_geom(const AttnArgs &a) {
    LocalGeom g;
    g.T = a.grid_t; g.Hg = a.grid_h; g.Wg = a.grid_w;
    g.wt = a.win_t; g.wh = a.win_h; g.ww = a.win_w;
    g.lt = a.win_t < a.grid_t ? a.win_t : a.grid_t;
    g.lh = a.win_h < a.grid_h ? a.win_h : a.grid_h;
    g.lw = a.win_w < a.grid_w ? a.win_w : a.grid_w;
    g.cut = a.cut;
    g.tiles_y = (a.grid_h + kLocalQY - 1) / kLocalQY;
    g.tiles_x = (a.grid_w + kLocalQX - 1) / kLocalQX;
    g.slot_row = kLocalQX + g.lw - 1 <= 16 ? 16 : 32;
    return g;
}

// The band kernel (bf16) in form kMode over every local token.
template <int kMode>
hipError_t launch_band(const AttnArgs &a, const LocalGeom &g, const BandGrad &gr, hipStream_t stream) {
    const float sl2 = a.scale * kLog2e;
    // Tile shape: 4x8 or 8x4 queries, whichever needs fewer 32-key blocks
    // per key frame (box rows / rows per block).
    auto blocks_per_frame = [&](int qy) {
        const int qx = 32 / qy, nx = qx + g.lw - 1, rows = qy + g.lh - 1;
        const int rpb = nx <= 16 ? 2 : 1;
        return nx > 32 ? 1 << 30 : (rows + rpb - 1) / rpb;
    };
    const int qy = blocks_per_frame(8) < blocks_per_frame(4) ? 8 : 4, qx = 32 / qy;
    LocalGeom gb = g;
    gb.tiles_y = (a.grid_h + qy - 1) / qy;
    gb.tiles_x = (a.grid_w + qx - 1) / qx;
    const bool b16 = qx + g.lw - 1 <= 16;
    // Workgroup shape (x-tiles NW, waves WV).  One frame x 4 x-tiles in
    // four-wave workgroups, two to a CU, so that one workgroup's waits (its
    // first loads, the band barrier) overlap the other's work, where at least
    // 3/4 of those waves have a tile; else one frame x 8 x-tiles in eight
    // waves, unless 4 x-tiles in two frames leave clearly fewer waves without
    // a tile (one frame keeps every wave busy in every band).  The gradient
    // form, whose buffers must stay within the LDS instructions' offsets,
    // never takes 8 x-tiles.
    auto filled = [&](int nw) { return (double)gb.tiles_x / (nw * ((gb.tiles_x + nw - 1) / nw)); };
    int shape = 2;  // 0: NW 8, WV 8; 1: NW 4, WV 4; 2: NW 4, WV 8
    if (filled(4) >= 0.75 && (kMode == 2 || filled(4) >= filled(8) - 0.05)) shape = 1;
    else if (kMode != 2 && filled(8) >= filled(4) - 0.05) shape = 0;
    const int NW = shape == 0 ? 8 : 4, WV = shape == 1 ? 4 : 8, NF = WV / NW;
    const int x_blocks = (gb.tiles_x + NW - 1) / NW, t_groups = (g.T + NF - 1) / NF;
    const int band_units = a.batch * a.heads * t_groups * gb.tiles_y * x_blocks;
    const dim3 bgrid((band_units + 7) / 8 * 8), bblock(64 * WV);
#define HET_BAND_LAUNCH_NW(D_, SR_, QY_, NW_, WV_)                                                           \
    hipLaunchKernelGGL((local_band_kernel<D_, SR_, QY_, kMode, NW_, WV_>), bgrid, bblock, 0, stream,         \
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (__bf16 *)a.o, a.mask, \
                       a.n, a.heads, sl2, gb, band_units, x_blocks, t_groups, gr)
#define HET_BAND_LAUNCH(D_, SR_, QY_)                                   \
    do {                                                                \
        if constexpr (kMode != 2) {                                     \
            if (shape == 0) HET_BAND_LAUNCH_NW(D_, SR_, QY_, 8, 8);      \
            else if (shape == 1) HET_BAND_LAUNCH_NW(D_, SR_, QY_, 4, 4); \
            else HET_BAND_LAUNCH_NW(D_, SR_, QY_, 4, 8);                 \
        } else {                                                        \
            if (shape == 1) HET_BAND_LAUNCH_NW(D_, SR_, QY_, 4, 4);      \
            else HET_BAND_LAUNCH_NW(D_, SR_, QY_, 4, 8);                 \
        }                                                               \
    } while (0)
    if (a.head_dim == 128) {
        if (qy == 4) {
            if (b16) HET_BAND_LAUNCH(128, 16, 4); else HET_BAND_LAUNCH(128, 32, 4);
        } else {
            if (b16) HET_BAND_LAUNCH(128, 16, 8); else HET_BAND_LAUNCH(128, 32, 8);
        }
    } else {
        if (qy == 4) {
            if (b16) HET_BAND_LAUNCH(64, 16, 4); else HET_BAND_LAUNCH(64, 32, 4);
        } else {
            if (b16) HET_BAND_LAUNCH(64, 16, 8); else HET_BAND_LAUNCH(64, 32, 8);
        }
    }
#undef HET_BAND_LAUNCH
#undef HET_BAND_LAUNCH_NW
    return hipGetLastError();
}

}  // namespace

hipError_t launch_local(const AttnArgs &a, hipStream_t stream) {
    const LocalGeom g = local_geom(a);
    if (kLocalQX + g.lw - 1 > 32) return hipErrorInvalidValue;  // rejected earlier by the ABI layer
    if (a.bf16) return launch_band<0>(a, g, BandGrad{nullptr, a.lse_out, nullptr, nullptr, 0.0f}, stream);
    const int units = a.batch * a.heads * g.T * g.tiles_y * g.tiles_x;
    const dim3 grid((units + 7) / 8 * 8);
    const float sl2 = a.scale * kLog2e;
#define HET_LOCAL_LAUNCH(D_, SR_)                                                                   \
    hipLaunchKernelGGL((local_f32_kernel<D_, SR_>), grid, dim3(64), 0, stream, (const float *)a.q,  \
                       (const float *)a.k, (const float *)a.v, (float *)a.o, a.mask, a.n, a.heads, sl2, g, units)
    const bool sr16 = g.slot_row == 16;
    if (a.head_dim == 128) {
        if (sr16) HET_LOCAL_LAUNCH(128, 16); else HET_LOCAL_LAUNCH(128, 32);
    } else {
        if (sr16) HET_LOCAL_LAUNCH(64, 16); else HET_LOCAL_LAUNCH(64, 32);
    }
#undef HET_LOCAL_LAUNCH
    return hipGetLastError();
}

hipError_t launch_local_lse(const AttnArgs &a, float *lse, hipStream_t stream) {
    const LocalGeom g = local_geom(a);
    if (!a.bf16 || kLocalQX + g.lw - 1 > 32) return hipErrorInvalidValue;
    return launch_band<1>(a, g, BandGrad{nullptr, lse, nullptr, nullptr, 0.0f}, stream);
}

hipError_t launch_local_dq(const AttnArgs &a, const void *dout, const float *lse, const float *dsum, void *dq,
                           hipStream_t stream) {
    const LocalGeom g = local_geom(a);
    if (!a.bf16 || kLocalQX + g.lw - 1 > 32) return hipErrorInvalidValue;
    return launch_band<2>(a, g,
                          BandGrad{(const __bf16 *)dout, const_cast<float *>(lse), dsum, (__bf16 *)dq, a.scale},
                          stream);
}

}  // namespace hetattn
