// dense.hip -- dense softmax attention for the gathered dense tokens.
//
// [HetA] = "Where Compute Matters: Heterogeneous Attention for Efficient
// Video Diffusion" (HetA-DiT): dense attention of §3.1.1 Eq. 2 for the tokens
// with m_i = 0 (§3.2.2 Eqs. 12-13).  This is the rho*N^2*d_h term of the cost
// model (§3.2.2 Eq. 14) and the dominant cost of the layer.
//
// bf16 path.  One workgroup = 8 waves = 256 gathered queries of one
// (sample, head), 32 per wave.  Per 64-key tile:
//   S^T = K Q^T      MFMA 32x32x16, A = K tile (LDS), B = Q (registers)
//   online softmax   fp32, base 2, per query = per lane (lane l%32)
//   O^T += V^T P^T   MFMA, A = V tile read transposed from LDS, B = P
// Computing the transposed products keeps every per-query quantity (running
// max, row sum, output column) in the lane that owns the query, so the
// softmax needs one cross-half exchange per tile and no LDS round trip.
//
// Ping-pong: waves 0-3 (group 0) and 4-7 (group 1) put one wave of each
// group on every SIMD.  Each wave alternates an MFMA burst (P*V of the
// previous tile, then S of this tile) with a VALU burst (softmax of this
// tile), and the two groups run half a round apart, so while one wave of a
// SIMD computes exponentials the other keeps the matrix unit busy.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace hetattn {

constexpr int kDenseThreads = 256;  // f32 path
constexpr int kDenseBM = 128;       // f32 path: queries per workgroup
constexpr int kDenseThreads16 = 512;  // bf16 path: 8 waves
constexpr int kDenseBM16 = 256;       // bf16 path: queries per workgroup

// ---------------------------------------------------------------- bf16 ----
// K and V tiles move global -> LDS by DMA (buffer_load_dwordx4 ... lds: each
// wave writes one contiguous 1 KB run, lane l at byte 16*l), double-buffered
// in four separate LDS arrays so that reads of one buffer never wait on DMA
// into another.  Rows are unpadded and chunk-swizzled (swz<D>), so the K
// reads (A operand) and the transposed V reads are free of bank conflicts.
//
// Per iteration kt (one barrier):
//   wait for own DMA, barrier      K(kt+1), V(kt) now in LDS; previous reads done
//   DMA K(kt+2), V(kt+1)           into the buffers freed by the barrier
//   S(kt+1) = K(kt+1) Q^T  ||  P(kt) = exp2(S(kt) - m)
//   O^T += V(kt)^T P^T     ||  row max of S(kt+1)
template <int D>
struct DenseBf16Geom {
    static constexpr int BN = 64;                  // keys per tile
    static constexpr int kWaves = 8;
    static constexpr int kCpr = D / 8;             // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / kCpr; // rows per wave DMA (1 KB)
    static constexpr int kLoadsPerWave = BN / kRowsPerLoad / kWaves;
    static constexpr int kTileElems = BN * D;
};

// ------------------------------------------------------ stream-K schedule --
// The dense work is the list of units (sample, head, 256-query tile), each a
// sequence of n_kt key tiles.  The grid is persistent (one workgroup per CU,
// G of them).  Whole units go first, round-robin; the units_sk = units mod G
// left over are flattened unit-major into W = units_sk * n_kt items and
// workgroup w takes items [w*W/G, (w+1)*W/G), so every CU gets the same
// amount of work.  A unit cut between workgroups is finished in pieces: each
// piece stores its partial state (unnormalised O, reference max m, row sum l,
// fp32) in the workspace, and a second kernel merges the pieces of every
// split unit (O = sum 2^(m_s - m) O_s, l = sum 2^(m_s - m) l_s) in workgroup
// order and writes the output.  The kernel boundary orders the two, so no
// workgroup waits for another and no device-scope fence (which on this chip
// writes back a whole L2) is needed inside the persistent kernel.
//
// Workspace: [2G slots][kDenseBM16 queries][D] O partials (each lane's
// accumulators contiguous, in register order), then [2G][2][kDenseBM16]
// (m, l).  Slot 2w holds the piece of workgroup w's first unit, slot 2w+1
// that of its last.
__device__ __forceinline__ int64_t work_begin(int64_t W, int G, int w) { return (int64_t)w * W / G; }
// Workgroup owning item x: the largest w with work_begin(w) <= x.
__device__ __forceinline__ int work_owner(int64_t W, int G, int64_t x) {
    int w = (int)(x * G / W);
    while (w + 1 < G && work_begin(W, G, w + 1) <= x) ++w;
    return w;
}

// kLse: only the row statistics -- no P*V, no V tiles -- and the output is
// LSE_i = m_i + log2(l_i) (log2 units of scale * q.k) in lse[(b*H + h)*N + i]
// for the gradient of the layer; the stream-K pieces then publish (m, l) only.
// !kLse: the output O, and the same LSE too when lse is not null.
template <int D, bool kLse>
__global__ __launch_bounds__(kDenseThreads16) void dense_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    __bf16 *__restrict__ o, const int32_t *__restrict__ dense_idx,
    const int32_t *__restrict__ counts, int B, int N, int H, float scale_log2, int G,
    float *__restrict__ ws_part, float *__restrict__ lse) {
    using Gm = DenseBf16Geom<D>;
    constexpr int BN = Gm::BN;
    constexpr int BM = kDenseBM16;
    constexpr int NC = D / 16;  // k-chunks of QK
    constexpr int NDB = D / 32; // 32-row blocks of O^T
    __shared__ __attribute__((aligned(1024))) __bf16 K0[Gm::kTileElems];
    __shared__ __attribute__((aligned(1024))) __bf16 K1[Gm::kTileElems];
    __shared__ __attribute__((aligned(1024))) __bf16 V0[Gm::kTileElems];
    __shared__ __attribute__((aligned(1024))) __bf16 V1[Gm::kTileElems];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2;  // ping-pong group
    const int half = lane >> 5, col = lane & 31;
    const int tok_stride = H * D;
    const int n_kt = (N + BN - 1) / BN;

    // Units per sample come from the device-side dense counts, so the split is
    // exact in both threshold modes; every workgroup computes the same list.
    int units = 0;
    for (int bb = 0; bb < B; ++bb) units += H * ((counts[2 * bb] + BM - 1) / BM);
    // Whole units first, round-robin: the G workgroups start their units
    // together at key tile 0, and the units of one head run on one XCD, so
    // the K/V stream of a head is fetched once per XCD and shared in its L2.
    // Only the remaining units_sk = units mod G are split stream-K style.
    const int units_dp = units / G * G, units_sk = units - units_dp;
    const int64_t W = (int64_t)units_sk * n_kt;  // stream-K items
    const int w = xcd_remap(blockIdx.x, gridDim.x);
    if (w >= G || units == 0) return;
    int dp_unit = w;
    int64_t x = units_sk ? work_begin(W, G, w) : 0;
    const int64_t x_end = units_sk ? work_begin(W, G, w + 1) : 0;
    const int first_unit = units_sk ? units_dp + (int)(x / n_kt) : -1;  // first stream-K unit

    // DMA geometry: load j of this wave fills tile rows from r0_j on; this
    // lane writes row r0_j + lane/kCpr at chunk position lane%kCpr, so it
    // fetches the chunk that the swizzle puts there.  The loads go through a
    // buffer descriptor whose base is the tile's first key row (scalar, per
    // tile), so each lane's byte offset inside the tile is fixed.
    const int dma_lrow = lane / Gm::kCpr, dma_pos = lane % Gm::kCpr;
    int dma_voff[Gm::kLoadsPerWave];
#pragma unroll
    for (int j = 0; j < Gm::kLoadsPerWave; ++j) {
        const int r = (wave * Gm::kLoadsPerWave + j) * Gm::kRowsPerLoad + dma_lrow;
        dma_voff[j] = 2 * (r * tok_stride + 8 * (dma_pos ^ swz<D>(r)));
    }
    // Transposed V read: lane j16 of each 16-lane group points at tile row
    // base + 4*half + j16/4, element column 16*(g16&1) + 4*(j16&3) of a
    // 32-column slab, i.e. chunk 2*(g16&1) + (j16&3)/2, byte 8*(j16&1).
    const int g16 = lane >> 4, j16 = lane & 15;
    const int v_row_off = 4 * half + (j16 >> 2);
    const int v_chunk_off = 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int v_elem_off = 4 * (j16 & 1);
    // Per-lane element offsets inside a tile, shared by every buffer: the
    // swizzle only sees the low row bits, which the block/step parts of the
    // row index (multiples of 16) leave alone.
    //   K, A operand of chunk c:   row col (+32 per key block), chunk 2c+half
    //   V, slab db, rows +8*lohi:  row v_row_off + 8*lohi (+16*c2 + 32*kbk)
    int k_off[NC], v_off[NDB][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) k_off[c] = col * D + 8 * ((2 * c + half) ^ swz<D>(col));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int lohi = 0; lohi < 2; ++lohi) {
            const int row = v_row_off + 8 * lohi;
            v_off[db][lohi] = row * D + 8 * ((4 * db + v_chunk_off) ^ swz<D>(row)) + v_elem_off;
        }

    // Stream-K pieces of the full length M = W / G visit their key tiles in
    // the order of the tile index mod M (step i takes the tile t of the piece
    // with t = i mod M), so every piece that holds a given key tile of a head
    // reads it in the same round: the pieces of different units start at
    // different tiles (n_kt mod M != 0 in general) but, like the whole units,
    // run side by side on their XCD and share its L2.  Other pieces (the
    // whole units, and the ends of units) keep the natural order.
    const int piece_m = units_sk ? (int)(W / G) : 0;
    for (;;) {
        // ---- next task: a whole unit, then pieces of the stream-K units
        int unit, kt0, kt1;
        int rot_m = 0;  // M when this piece visits its tiles in rotated order
        if (dp_unit < units_dp) {
            unit = dp_unit;
            kt0 = 0;
            kt1 = n_kt;
            dp_unit += G;
        } else if (x < x_end) {
            const int sk = (int)(x / n_kt);
            kt0 = (int)(x - (int64_t)sk * n_kt);
            kt1 = (int)((x_end - (int64_t)sk * n_kt) < n_kt ? (x_end - (int64_t)sk * n_kt) : n_kt);
            x = (int64_t)sk * n_kt + kt1;
            unit = units_dp + sk;
            if (piece_m > 1 && kt1 - kt0 == piece_m) rot_m = piece_m;
        } else {
            break;
        }
        int b = 0, rem = unit, tiles_b = 0;
        for (;;) {
            tiles_b = (counts[2 * b] + BM - 1) / BM;
            if (rem < H * tiles_b) break;
            rem -= H * tiles_b;
            ++b;
        }
        const int h = rem / tiles_b, tile = rem % tiles_b;
        const int n_dense = counts[2 * b];
        const __bf16 *kb = k + (size_t)b * N * tok_stride + (size_t)h * D;
        const __bf16 *vb = v + (size_t)b * N * tok_stride + (size_t)h * D;

        // Gathered query of this lane, as stored: the MFMA forms q.k exactly
        // (bf16 products, fp32 sums), and the softmax scale is applied in fp32
        // with the exponent's FMA, so no rounding of the logits precedes the
        // exponential (the logits of a peaked softmax reach tens of units).
        const int qrow = tile * BM + wave * 32 + col;
        const bool q_valid = qrow < n_dense;
        const int tok = q_valid ? dense_idx[(size_t)b * N + qrow] : 0;
        bf16x8 qf[NC];
        {
            const __bf16 *qp = q + ((size_t)b * N + tok) * tok_stride + (size_t)h * D + 8 * half;
#pragma unroll
            for (int c = 0; c < NC; ++c) qf[c] = q_valid ? *(const bf16x8 *)(qp + 16 * c) : bf16x8{};
        }

        // K or V tile kt -> LDS.  The descriptor covers the rows below N only:
        // a buffer load past its range returns zeros, so the ragged last tile
        // needs no special addressing (its extra keys are masked and their V
        // rows are zero).
        auto dma = [&](const __bf16 *src, __bf16 *dst, int kt) HET_INLINE {
            const int key0 = kt * BN;
            const uint32_t bytes = (uint32_t)((N - key0) * tok_stride) * 2u;
            const __bf16 *base = src + (size_t)key0 * tok_stride;
#pragma unroll
            for (int j = 0; j < Gm::kLoadsPerWave; ++j) {
                const int r0 = (wave * Gm::kLoadsPerWave + j) * Gm::kRowsPerLoad;
                buffer_load_lds16(base, bytes, (HET_LDS void *)(dst + r0 * D), dma_voff[j]);
            }
        };

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
        float m_ref = -__builtin_inff();  // reference max, log2 units (of scale * q.k * log2(e))
        float l_part = 0.0f;
        f32x16 sc[2];                     // S^T = q.k of the current tile: key block x 32 queries
        bf16x8 pf[2][2];                  // P of the current tile as the B operand

        // MFMA burst of round r: O^T += V(r-1)^T P(r-1)^T (steps 0..4*NDB-1),
        // then S(r) = K(r) Q^T (steps 4*NDB..4*NDB+2*NC-1).  The A operand of
        // step i is read from LDS kAhead steps before its MFMA, and
        // sched_barrier keeps the compiler from sinking the reads back.
        constexpr int kPvSteps = 4 * NDB, kQkSteps = 2 * NC, kAhead = 4;
        auto a_operand = [&](int i, const __bf16 *Vt, const __bf16 *Kt) HET_INLINE -> bf16x8 {
            if (i < kPvSteps) {
                const int db = i % NDB, kbk = (i / NDB) >> 1, c2 = (i / NDB) & 1;
                const __bf16 *base = Vt + (kbk * 32 + 16 * c2) * D;
                const bf16x4 lo = lds_read_tr16((const HET_LDS void *)(base + v_off[db][0]));
                const bf16x4 hi = lds_read_tr16((const HET_LDS void *)(base + v_off[db][1]));
                return concat8(lo, hi);
            }
            const int j = i - kPvSteps, kbk = j & 1, c = j >> 1;
            return *(const HET_LDS bf16x8 *)(Kt + kbk * 32 * D + k_off[c]);
        };
        // pv_tag/qk_tag are std::integral_constant<bool, ...>: every index below
        // is a compile-time constant, so the ring stays in registers.
        auto burst_ct = [&](auto pv_tag, auto qk_tag, const __bf16 *Vt, const __bf16 *Kt) HET_INLINE {
            constexpr bool kPv = decltype(pv_tag)::value, kQk = decltype(qk_tag)::value;
            constexpr int i0 = kPv ? 0 : kPvSteps, i1 = kQk ? kPvSteps + kQkSteps : kPvSteps;
            if constexpr (i0 < i1) {
                bf16x8 ring[kAhead];
#pragma unroll
                for (int a = 0; a < kAhead; ++a)
                    if (i0 + a < i1) ring[a] = a_operand(i0 + a, Vt, Kt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = i0; i < i1; ++i) {
                    const bf16x8 a = ring[(i - i0) % kAhead];
                    if (i < kPvSteps) {
                        const int db = i % NDB, kbk = (i / NDB) >> 1, c2 = (i / NDB) & 1;
                        oacc[db] = mfma32_bf16(a, pf[kbk][c2], oacc[db]);
                    } else {
                        // the first k-chunk of a key block starts from zero
                        // (an inline constant, not zeroed registers)
                        const int j = i - kPvSteps, kbk = j & 1, c = j >> 1;
                        sc[kbk] = mfma32_bf16(a, qf[c], c == 0 ? f32x16{} : sc[kbk]);
                    }
                    if (i + kAhead < i1) ring[(i - i0) % kAhead] = a_operand(i + kAhead, Vt, Kt);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // VALU burst of round r: softmax of S(r) into P(r) (lazy rescale, base 2).
        auto softmax = [&](int kt) HET_INLINE {
            if (__builtin_expect(kt == n_kt - 1 && kt * BN + BN > N, 0)) {
                // keys past N in the last tile: branch-free select per element
                const int lim = N - kt * BN - 4 * half;
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key_off = kbk * 32 + 8 * (i / 4) + (i % 4);
                        sc[kbk][i] = key_off < lim ? sc[kbk][i] : -__builtin_inff();
                    }
            }
            // Scores relative to the reference, in log2 units: one fp32 FMA
            // per score, s * scale * log2(e) - m_ref (a piece's first tile
            // is taken against 0).  The reference moves (exactly as a
            // running max would) only on the first tile of a piece and when
            // a tile's exponentials ran large: with every score <=
            // kRescaleSlack a lane's 32 exponentials sum to at most
            // 32 * 2^kRescaleSlack, so a larger sum (or a non-finite one)
            // sends the tile through the exact max and its exponentials are
            // taken again.  Without the max on every tile a score may exceed
            // the reference by up to log2(32) + kRescaleSlack, well inside
            // fp32 and bf16 range.
            {
                const float neg_m = m_ref == -__builtin_inff() ? 0.0f : -m_ref;
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sc[kbk][i] = __builtin_fmaf(sc[kbk][i], scale_log2, neg_m);
            }
            auto rescale = [&]() HET_INLINE {
                float mx = -__builtin_inff();
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kbk][i]);
                mx = half_pair_max(mx);
                const bool first = m_ref == -__builtin_inff();  // first tile of the piece
                const bool grow = first || mx > kRescaleSlack;
                if (__builtin_expect(__any(grow), 0)) {
                    // The new reference and how far it moved.
                    const float m_base = first ? 0.0f : m_ref;
                    const float delta = grow ? mx : 0.0f;
                    const float alpha = first ? 1.0f : __builtin_amdgcn_exp2f(-delta);
                    m_ref = m_base + delta;
                    l_part *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
#pragma unroll
                    for (int kbk = 0; kbk < 2; ++kbk) sc[kbk] -= delta;
                }
            };
            // chunk c2 of key block kb = registers 8*c2 .. 8*c2+7, i.e. keys
            // 16*c2 + 8(j/4) + 4*half + j%4 (j < 8) of the block.
            auto exps = [&]() HET_INLINE -> float {
                float tsum = 0.0f;
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        u32x4 wv;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float p0 = __builtin_amdgcn_exp2f(sc[kbk][8 * c2 + 2 * j]);
                            const float p1 = __builtin_amdgcn_exp2f(sc[kbk][8 * c2 + 2 * j + 1]);
                            tsum += p0 + p1;
                            if constexpr (!kLse) wv[j] = pack_bf16x2(p0, p1);
                        }
                        if constexpr (!kLse) pf[kbk][c2] = __builtin_bit_cast(bf16x8, wv);
                    }
                return tsum;
            };
            constexpr float kTileSumLimit = 32.0f * (float)(1 << (int)kRescaleSlack);
            if (__builtin_expect(__any(m_ref == -__builtin_inff()), 0)) rescale();
            float tsum = exps();
            if (__builtin_expect(__any(!(tsum <= kTileSumLimit)), 0)) {
                rescale();
                tsum = exps();
            }
            l_part += tsum;
        };

        // ---- rounds kt0 .. kt1 of this piece.  Round r holds K(r) and
        // V(r-1) in LDS and fetches K(r+1), V(r):
        //   group 0: burst(r), then softmax(r)
        //   group 1: softmax(r-1), then burst(r)
        // so on every SIMD one wave starts on the matrix unit while the other
        // computes exponentials; only the end of a round is a barrier.
        // The first round has no P*V and the last no QK; in between, K(r)
        // lives in K0 for even r-kt0 and K1 for odd, V(r) likewise.
        // Key tile of round r (rounds kt0 .. kt1-1): kt0 + (r - 2*kt0 mod M),
        // from one remainder per piece and a compare per round.
        const int rot0 = rot_m ? (rot_m - kt0 % rot_m) % rot_m : 0;
        auto tile_at = [&](int r) HET_INLINE -> int {
            if (rot_m == 0) return r;
            const int d = r - kt0 + rot0;
            return kt0 + (d >= rot_m ? d - rot_m : d);
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();  // previous piece is done with the buffers
        dma(kb, K0, tile_at(kt0));
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        // first round r = kt0
        if (kt0 + 1 < kt1) dma(kb, K1, tile_at(kt0 + 1));
        if constexpr (!kLse) dma(vb, V0, tile_at(kt0));
        if (grp == 0) burst_ct(F_{}, T_{}, V1, K0);
        __builtin_amdgcn_s_barrier();
        if (grp == 0) softmax(tile_at(kt0));
        else burst_ct(F_{}, T_{}, V1, K0);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        // rounds kt0+1 .. kt1-1: full bursts
        // (kLse: S-only bursts, and no V tiles.)
        using PV_ = std::integral_constant<bool, !kLse>;
        auto round = [&](int r, const __bf16 *Kc, __bf16 *Kn, const __bf16 *Vp, __bf16 *Vc) HET_INLINE {
            if (r + 1 < kt1) dma(kb, Kn, tile_at(r + 1));
            if constexpr (!kLse) dma(vb, Vc, tile_at(r));
            if (grp == 0) burst_ct(PV_{}, T_{}, Vp, Kc);
            else softmax(tile_at(r - 1));
            if (grp == 0) softmax(tile_at(r));
            else burst_ct(PV_{}, T_{}, Vp, Kc);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_s_barrier();
        };
        for (int r = kt0 + 1; r < kt1; r += 2) {
            round(r, K1, K0, V0, V1);
            if (r + 1 < kt1) round(r + 1, K0, K1, V1, V0);
        }
        // last round r = kt1: P*V of tile kt1-1 only; no DMA is in flight, so
        // the buffer can be picked at run time.
        {
            const __bf16 *Vp = ((kt1 - 1 - kt0) & 1) ? V1 : V0;
            if (grp == 0) burst_ct(PV_{}, F_{}, Vp, K0);
            else softmax(tile_at(kt1 - 1));
            __builtin_amdgcn_s_barrier();
            if (grp == 1) burst_ct(PV_{}, F_{}, Vp, K0);
        }

        const float l_tot = half_pair_sum(l_part);
        if constexpr (kLse) {
            if (kt0 == 0 && kt1 == n_kt) {
                if (q_valid && half == 0) lse[((size_t)b * H + h) * N + tok] = m_ref + __builtin_log2f(l_tot);
                continue;
            }
        }
        __bf16 *op = o + ((size_t)b * N + tok) * tok_stride + (size_t)h * D;
        auto store_out = [&](float inv_l) HET_INLINE {
            if (!q_valid) return;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int d = db * 32 + 8 * i4 + 4 * half;
                    u32x2 wv;
                    wv[0] = pack_bf16x2(oacc[db][4 * i4 + 0] * inv_l, oacc[db][4 * i4 + 1] * inv_l);
                    wv[1] = pack_bf16x2(oacc[db][4 * i4 + 2] * inv_l, oacc[db][4 * i4 + 3] * inv_l);
                    *(u32x2 *)(op + d) = wv;
                }
        };
        if constexpr (!kLse) {
            if (kt0 == 0 && kt1 == n_kt) {
                store_out(1.0f / l_tot);
                // The row's LSE for the gradient, when asked for.
                if (lse != nullptr && q_valid && half == 0)
                    lse[((size_t)b * H + h) * N + tok] = m_ref + __builtin_log2f(l_tot);
                continue;
            }
        }

        // ---- a piece of a split unit: publish the partial state.  Each lane
        // stores its D/2 accumulators contiguously in register order (the
        // lane that merges reads them back in the same order).
        const size_t slot_elems = kLse ? 0 : (size_t)D * BM;  // kLse: no O partials
        const int my_slot = 2 * w + (unit == first_unit ? 0 : 1);
        const int qi = wave * 32 + col;  // query within the unit
        {
            if constexpr (!kLse) {
                f32x4 *dst =
                    (f32x4 *)(ws_part + (size_t)my_slot * slot_elems + (size_t)qi * D + (size_t)half * (D / 2));
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4)
                        dst[db * 4 + i4] = f32x4{oacc[db][4 * i4], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2],
                                                 oacc[db][4 * i4 + 3]};
            }
            float *part_ml = ws_part + (size_t)2 * G * slot_elems + (size_t)my_slot * 2 * BM;
            if (half == 0) {
                part_ml[qi] = m_ref;
                part_ml[BM + qi] = l_tot;
            }
        }
        __syncthreads();
    }
}

// Partial layout helper shared by the persistent kernel and the merge: the
// piece slot of workgroup pw for split unit `unit`.
__device__ __forceinline__ int piece_slot(int64_t W, int G, int n_kt, int units_dp, int unit, int pw) {
    return 2 * pw + (unit == units_dp + (int)(work_begin(W, G, pw) / n_kt) ? 0 : 1);
}

// Merge of the split units.  Workgroup = (split unit, kMergeQ queries);
// thread = (query, 16 consecutive partial floats of it).  Partial float
// half*(D/2) + 16*db + 4*i4 + e of a query holds output column
// 32*db + 8*i4 + 4*half + e (the accumulator order of the MFMA C layout).
// The piece list of the unit (64-bit schedule arithmetic) is worked out by a
// few threads per batch and shared through LDS.
// kLse: the pieces hold (m, l) only and the result is the LSE of each row.
template <int D, bool kLse>
__global__ __launch_bounds__(256) void dense_merge_kernel(
    __bf16 *__restrict__ o, const int32_t *__restrict__ dense_idx, const int32_t *__restrict__ counts,
    int B, int N, int H, int G, const float *__restrict__ ws_part, float *__restrict__ lse) {
    constexpr int BM = kDenseBM16;
    constexpr int kSlices = D / 16;
    constexpr int kMergeQ = 256 / kSlices;
    constexpr int NDB = D / 32;
    constexpr int kMergeBatch = 8;
    __shared__ int s_range[2];
    __shared__ int s_slot[kMergeBatch];
    const int n_kt = (N + DenseBf16Geom<D>::BN - 1) / DenseBf16Geom<D>::BN;
    int units = 0;
    for (int bb = 0; bb < B; ++bb) units += H * ((counts[2 * bb] + BM - 1) / BM);
    const int units_dp = units / G * G, units_sk = units - units_dp;
    const int sk = blockIdx.x / (BM / kMergeQ);
    if (sk >= units_sk) return;  // the whole workgroup
    const int unit = units_dp + sk;
    int b = 0, rem = unit, tiles_b = 0;
    for (;;) {
        tiles_b = (counts[2 * b] + BM - 1) / BM;
        if (rem < H * tiles_b) break;
        rem -= H * tiles_b;
        ++b;
    }
    const int h = rem / tiles_b, tile = rem % tiles_b;
    const int tid = (int)threadIdx.x;
    const int qi = (blockIdx.x % (BM / kMergeQ)) * kMergeQ + tid / kSlices;
    const int slice = tid % kSlices;
    const int qrow = tile * BM + qi;
    const bool q_valid = qrow < counts[2 * b];

    const int64_t W = (int64_t)units_sk * n_kt;
    if (tid == 0) {
        const int64_t ux0 = (int64_t)sk * n_kt;
        s_range[0] = work_owner(W, G, ux0);
        s_range[1] = work_owner(W, G, ux0 + n_kt - 1);
    }
    __syncthreads();
    const int w_first = s_range[0], w_last = s_range[1];
    if (w_first == w_last) return;  // one workgroup ran the whole unit and stored it
    const size_t slot_elems = kLse ? 0 : (size_t)D * BM;
    const float *ml = ws_part + (size_t)2 * G * slot_elems;
    // Pieces come from the non-empty workgroups owning the unit's items,
    // taken kMergeBatch at a time with all their loads in flight (the running
    // max and the sums are rescaled between batches).
    float m_all = -__builtin_inff();
    f32x4 acc[4] = {};
    float l_all = 0.0f;
    for (int pw0 = w_first; pw0 <= w_last; pw0 += kMergeBatch) {
        if (tid < kMergeBatch) {
            const int pw = pw0 + tid;
            const bool ok = pw <= w_last && work_begin(W, G, pw + 1) > work_begin(W, G, pw);
            s_slot[tid] = ok ? piece_slot(W, G, n_kt, units_dp, unit, pw) : -1;
        }
        __syncthreads();
        float mp[kMergeBatch], lp[kMergeBatch];
        f32x4 pv[kMergeBatch][4];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const int ps = s_slot[j];
            const bool ok = ps >= 0 && q_valid;
            const f32x4 *po = (const f32x4 *)(ws_part + (size_t)(ok ? ps : 0) * slot_elems + (size_t)qi * D + 16 * slice);
            mp[j] = ok ? ml[(size_t)ps * 2 * BM + qi] : -__builtin_inff();
            lp[j] = ok ? ml[(size_t)ps * 2 * BM + BM + qi] : 0.0f;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) pv[j][i4] = (ok && !kLse) ? po[i4] : f32x4{};
        }
        __syncthreads();  // s_slot is rewritten by the next batch
        float m_new = m_all;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) m_new = fmaxf(m_new, mp[j]);
        const float r = (m_all == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_all - m_new);
        l_all *= r;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) acc[i4] *= r;
        m_all = m_new;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const float a = (mp[j] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mp[j] - m_all);
            l_all += a * lp[j];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i4][e] += a * pv[j][i4][e];
        }
    }
    if (!q_valid) return;
    const int tok = dense_idx[(size_t)b * N + qrow];
    if constexpr (kLse) {
        if (slice == 0) lse[((size_t)b * H + h) * N + tok] = m_all + __builtin_log2f(l_all);
        return;
    }
    if (lse != nullptr && slice == 0) lse[((size_t)b * H + h) * N + tok] = m_all + __builtin_log2f(l_all);
    const float inv_l = 1.0f / l_all;
    const int half = slice / NDB, db = slice % NDB;
    __bf16 *op = o + ((size_t)b * N + tok) * ((size_t)H * D) + (size_t)h * D;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 wv;
        wv[0] = pack_bf16x2(acc[i4][0] * inv_l, acc[i4][1] * inv_l);
        wv[1] = pack_bf16x2(acc[i4][2] * inv_l, acc[i4][3] * inv_l);
        *(u32x2 *)(op + 32 * db + 8 * i4 + 4 * half) = wv;
    }
}

// The f32 path below uses kDenseBM queries per workgroup and a plain grid;
// K and V tiles are staged in LDS with rows padded against bank conflicts.
template <int D, int BN>
struct DenseTileF32 {
    static constexpr int kPitchK = D + 4;         // elements
    static constexpr int kPitchV = D + 4;
    static constexpr int kVec = 4;                // elements per 16-byte load
    static constexpr int kChunksPerRow = D / kVec;
    static constexpr int kRowsPerPass = kDenseThreads / kChunksPerRow;
    static constexpr int kPasses = BN / kRowsPerPass;
    static_assert(kPasses * kRowsPerPass == BN, "tile load shape");
};

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
    using Tl = DenseTileF32<D, BN>;
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
    auto fetch = [&](int kt) HET_INLINE {
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
    auto stash = [&]() HET_INLINE {
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

int dense_persistent_groups(int cu_count) { return cu_count; }

size_t dense_lse_workspace_bytes(int cu_count) {
    return 2 * (size_t)dense_persistent_groups(cu_count) * 2 * kDenseBM16 * sizeof(float);
}

// Row statistics of the dense rows for the gradient (bf16): the persistent
// kernel and merge in their kLse form; ws holds dense_lse_workspace_bytes().
hipError_t launch_dense_lse(const AttnArgs &a, float *lse, hipStream_t stream) {
    if (a.max_dense <= 0 || !a.bf16) return hipSuccess;
    const float sl2 = a.scale * kLog2e;
    auto q = (const __bf16 *)a.q, k = (const __bf16 *)a.k;
    const int G = dense_persistent_groups(a.cu_count);
    float *ws_part = (float *)a.workspace;
    const dim3 g1d((G + 7) / 8 * 8);
    const int units_ub = a.batch * a.heads * ((a.max_dense + kDenseBM16 - 1) / kDenseBM16);
    const int units_sk_ub = a.dense_exact ? units_ub % G : (units_ub < G ? units_ub : G - 1);
    const int merge_q = 256 / (a.head_dim / 16);
    const dim3 gm((unsigned)units_sk_ub * (kDenseBM16 / merge_q));
    if (a.head_dim == 128) {
        hipLaunchKernelGGL((dense_bf16_kernel<128, true>), g1d, dim3(kDenseThreads16), 0, stream, q, k, nullptr,
                           nullptr, a.dense_idx, a.counts, a.batch, a.n, a.heads, sl2, G, ws_part, lse);
        if (units_sk_ub > 0)
            hipLaunchKernelGGL((dense_merge_kernel<128, true>), gm, dim3(256), 0, stream, nullptr, a.dense_idx,
                               a.counts, a.batch, a.n, a.heads, G, (const float *)ws_part, lse);
    } else {
        hipLaunchKernelGGL((dense_bf16_kernel<64, true>), g1d, dim3(kDenseThreads16), 0, stream, q, k, nullptr,
                           nullptr, a.dense_idx, a.counts, a.batch, a.n, a.heads, sl2, G, ws_part, lse);
        if (units_sk_ub > 0)
            hipLaunchKernelGGL((dense_merge_kernel<64, true>), gm, dim3(256), 0, stream, nullptr, a.dense_idx,
                               a.counts, a.batch, a.n, a.heads, G, (const float *)ws_part, lse);
    }
    return hipGetLastError();
}

// Scratch of het_attn_forward_noalloc: the dense kernel's stream-K partials
// for up to kNoAllocGroups persistent workgroups at head_dim <= 128, held in
// a file-scope device array (one copy per device, allocated by the runtime
// when the library's code object is loaded on that device, held until the
// process ends).  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, looked up
// once per device below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

size_t dense_workspace_bytes(int batch, int heads, int n, int head_dim, bool bf16, int cu_count) {
    if (!bf16) return 0;
    const size_t G = (size_t)dense_persistent_groups(cu_count);
    (void)batch;
    (void)heads;
    (void)n;
    return 2 * G * ((size_t)head_dim * kDenseBM16 + 2 * kDenseBM16) * sizeof(float);
}

hipError_t launch_dense(const AttnArgs &a, hipStream_t stream) {
    if (a.max_dense <= 0) return hipSuccess;
    const float sl2 = a.scale * kLog2e;
    if (a.bf16) {
        auto q = (const __bf16 *)a.q, k = (const __bf16 *)a.k, v = (const __bf16 *)a.v;
        auto o = (__bf16 *)a.o;
        const int G = dense_persistent_groups(a.cu_count);
        float *ws_part = (float *)a.workspace;
        const dim3 g1d((G + 7) / 8 * 8);
        // Split units: units mod G.  Exact when the host knows the dense count
        // (top-rho gives every sample the same count), else at most G - 1; the
        // merge workgroups past the device-side count return at once.
        const int units_ub = a.batch * a.heads * ((a.max_dense + kDenseBM16 - 1) / kDenseBM16);
        const int units_sk_ub = a.dense_exact ? units_ub % G : (units_ub < G ? units_ub : G - 1);
        const int merge_q = 256 / (a.head_dim / 16);
        const dim3 gm((unsigned)units_sk_ub * (kDenseBM16 / merge_q));
        if (a.head_dim == 128) {
            hipLaunchKernelGGL((dense_bf16_kernel<128, false>), g1d, dim3(kDenseThreads16), 0, stream, q, k, v, o,
                               a.dense_idx, a.counts, a.batch, a.n, a.heads, sl2, G, ws_part, a.lse_out);
            if (units_sk_ub > 0)
                hipLaunchKernelGGL((dense_merge_kernel<128, false>), gm, dim3(256), 0, stream, o, a.dense_idx,
                                   a.counts, a.batch, a.n, a.heads, G, (const float *)ws_part, a.lse_out);
        } else {
            hipLaunchKernelGGL((dense_bf16_kernel<64, false>), g1d, dim3(kDenseThreads16), 0, stream, q, k, v, o,
                               a.dense_idx, a.counts, a.batch, a.n, a.heads, sl2, G, ws_part, a.lse_out);
            if (units_sk_ub > 0)
                hipLaunchKernelGGL((dense_merge_kernel<64, false>), gm, dim3(256), 0, stream, o, a.dense_idx,
                                   a.counts, a.batch, a.n, a.heads, G, (const float *)ws_part, a.lse_out);
        }
    } else {
        const dim3 grid((a.max_dense + kDenseBM - 1) / kDenseBM, a.heads, a.batch);
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
