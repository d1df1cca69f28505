// common.hpp -- device helpers shared by the gfx950 kernels of the
// heterogeneous attention library: vector types, MFMA wrappers and the lane
// layouts they imply, bf16 packing and a few cross-lane reductions.
//
// MFMA lane layouts used throughout (wave64, gfx950):
//   v_mfma_f32_32x32x16_bf16   A: lane l holds row l%32, k = 8*(l/32) + j (j < 8)
//                              B: lane l holds col l%32, k = 8*(l/32) + j
//                              C: lane l, reg i -> col l%32, row 8*(i/4) + 4*(l/32) + i%4
//   v_mfma_f32_32x32x2_f32     A: row l%32, k = l/32;  B: col l%32, k = l/32;  C as above
// ds_read_b64_tr_b16: inside each 16-lane group, lane j supplies the address
// of 4 consecutive 16-bit elements M_j; lane i receives M_{4e + i/4}[i%4] as
// element e (e < 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hetattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define HET_LDS __attribute__((address_space(3)))
// Kernel-local lambdas must inline: a lambda left as a call makes its
// by-reference captures addressable, which puts them in scratch memory.
#define HET_INLINE __attribute__((always_inline))

constexpr float kLog2e = 1.4426950408889634f;

// Lazy rescaling of the online softmax: the running reference max only moves
// when a tile's max exceeds it by more than kRescaleSlack (log2 units).
// Probabilities are then at most 2^kRescaleSlack, which bf16 and fp32 hold
// with the same relative precision as values <= 1, and O / l is unchanged
// because both are taken against the same reference.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x16 mfma32_bf16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 of two values, packed (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const bf16x2 r = __builtin_convertvector((f32x2_t){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Value of lane l^32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0] = [x_lo, x_lo], r[1] = [x_hi, x_hi]: the partner is r[1] below lane 32, r[0] above.
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float half_pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const HET_LDS void *p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HET_LDS s16x4 *)p);
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__host__ __device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// Workgroup -> work unit.  The hardware deals consecutive workgroups to the 8
// XCDs round-robin; this remap gives each XCD a contiguous run of units so
// that units sharing K/V (one head, neighbouring tiles) share that XCD's L2.
// nwg must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    const int per_xcd = nwg >> 3;
    return (bid & 7) * per_xcd + (bid >> 3);
}

// Word 3 of a raw buffer descriptor (gfx9 family: 32-bit data format, no
// swizzle); out-of-range loads return zeros.
constexpr int kBufferRsrcWord3 = 0x00020000;

// 16 bytes per lane from base + voff (bytes) into LDS (each wave writes one
// contiguous 1 KB run from lds, lane l at 16*l).  Bytes at or past `bytes`
// from base read as zero.  base, bytes and lds must be wave-uniform.
__device__ __forceinline__ void buffer_load_lds16(const void *base, uint32_t bytes, HET_LDS void *lds,
                                                  int voff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferRsrcWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0);
}

// XOR swizzle of the 16-byte chunks of a bf16 row of D elements held in LDS
// (rows unpadded): chunk c of row r is stored at chunk c ^ swz<D>(r).  The
// LDS has 64 banks of 4 bytes; with this swizzle a 16-lane ds_read_b128 of 16
// consecutive rows at one chunk, and a 32-lane transposed read of 4
// consecutive rows x 4 consecutive chunks, both touch every bank once.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);  // 16 chunks per row
    else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);              // 8 chunks, 2 rows per 256 B
}

// Window start along one axis (shifted inside the grid), see hetattn.h.
__host__ __device__ __forceinline__ int window_start(int pos, int k, int len, int S) {
    int s = pos - (k - 1) / 2;
    s = imin(s, S - len);
    return imax(s, 0);
}

// Window [lo, hi) of position pos along an axis of extent S, for the odd
// window k of effective length len = min(k, S): shifted to stay inside
// [0, S) (cut = 0), or centred on pos and cut at the border (cut = 1).  Both
// ends are non-decreasing in pos, so the union of the windows of the
// positions p0 <= p <= p1 is [lo(p0), hi(p1)), and it is never wider than
// p1 - p0 + len.
__host__ __device__ __forceinline__ int win_lo(int pos, int k, int len, int S, int cut) {
    return cut ? imax(pos - (k - 1) / 2, 0) : window_start(pos, k, len, S);
}
__host__ __device__ __forceinline__ int win_hi(int pos, int k, int len, int S, int cut) {
    return cut ? imin(pos + (k - 1) / 2 + 1, S) : window_start(pos, k, len, S) + len;
}

}  // namespace hetattn
