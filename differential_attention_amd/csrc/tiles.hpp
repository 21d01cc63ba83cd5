// tiles.hpp -- tile geometry and LDS layout helpers shared by the bf16
// attention kernels (prefill forward and its backward pass).
//
// A key tile holds kBN = 64 rows of one head in LDS, row-major, without
// padding; its 16-byte chunks are XOR-swizzled per row so that both the
// operand reads of a key row (ds_read_b128) and the transposing reads of a
// column block (ds_read_b64_tr_b16) hit distinct banks. The same layouts
// serve any [rows][d] tile of width 64 or 128 (keys, queries) and any
// [rows][128] tile (values, output gradients).
#pragma once

#include "common.hpp"

namespace da {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDV = 128;  // value width (both forms)
constexpr int kBN = 64;   // rows per LDS tile

// Row (within a 32-row sub-block) read by the A-operand row m of an MFMA:
// bits 2 and 3 of m swapped, so that the 8 accumulator registers a lane
// holds for one 16-row step cover 8 consecutive rows.
__device__ __forceinline__ int perm_key(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Row offset (within a sub-block, before adding 8 * lane-half) held by
// register r of an accumulator whose A-operand rows were permuted as above.
__device__ __forceinline__ constexpr int key_of_reg(int r) { return 16 * ((r >> 3) & 1) + 4 * ((r >> 2) & 1) + (r & 3); }

// XOR swizzles of the 16-byte chunk index inside a tile row.
//
// Forward tiles are read one way each: K tiles by rows (ds_read_b128, 16
// lanes per pass reading one chunk of 16 different rows of an aligned 16-row
// block) and V tiles transposed (ds_read_b64_tr_b16, 32 lanes per pass reading
// 4 consecutive chunks of 4 consecutive rows that start at a multiple of 4).
// These swizzles keep each pattern on distinct banks and fold into immediate
// LDS offsets (few address registers):
template <int DQK>
__device__ __forceinline__ int k_swz(int row) {
    return DQK == 128 ? (row & 15) : ((row >> 1) & 7);  // row reads
}
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }  // transposed reads

// Backward tiles (K, Q, V, output gradient) are read both ways. Both passes
// touch every bank once when:
//  * 256-byte rows (d 128, and the value / output-gradient tiles): the swizzle
//    is a bijection of the row's 4 low bits (row reads) whose bits 2-3 differ
//    across 4 consecutive rows (transposed reads): 4 (row & 3) + ((row >> 2) & 3).
//  * 128-byte rows (d 64; two rows per 256-byte bank period): a bijection of
//    row bits 1-3 for either row parity (row reads) that differs in bit 2
//    between rows r and r + 2 of a 4-row group (transposed reads):
//    4 ((row >> 1) & 1) + ((row >> 2) & 3).
__device__ __forceinline__ int swz256(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz128(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
template <int DQK>
__device__ __forceinline__ int bk_swz(int row) {
    return DQK == 128 ? swz256(row) : swz128(row);
}
__device__ __forceinline__ int bv_swz(int row) { return swz256(row); }

// the swizzles as function objects (for tr_frag)
template <int DQK>
struct SwzK {
    __device__ __forceinline__ int operator()(int row) const { return k_swz<DQK>(row); }
};
struct SwzV {
    __device__ __forceinline__ int operator()(int row) const { return v_swz(row); }
};
template <int DQK>
struct BSwzK {
    __device__ __forceinline__ int operator()(int row) const { return bk_swz<DQK>(row); }
};
struct BSwzV {
    __device__ __forceinline__ int operator()(int row) const { return bv_swz(row); }
};

__device__ __forceinline__ uint4 ldg16(const __bf16 *p) { return *(const uint4 *)p; }

__device__ __forceinline__ void wait_vmem_all() {
    // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int DQK, bool SHARED_K>
struct Tile {
    static constexpr int kKBytes = kBN * DQK * 2;           // one K tile
    static constexpr int kVBytes = kBN * kDV * 2;           // the V tile
    static constexpr int kNK = SHARED_K ? 1 : 2;            // K tiles per stage
    static constexpr int kStage = kNK * kKBytes + kVBytes;  // bytes per stage
    static constexpr int kKCh = DQK / 8;                    // 16-byte chunks per K row
    static constexpr int kKBlocks = kNK * kKBytes / 1024;   // 1 KB blocks of K per stage
    static constexpr int kBlocks = kStage / 1024;           // 1 KB blocks per stage
    static constexpr int kRowsPerKBlock = 1024 / (2 * DQK);
};

// Byte offset of the 4 b16 values a lane fetches with one ds_read_b64_tr_b16
// for the transposed operand of a 32x32x16 MFMA: A = X^T for a row-major tile
// X [rows][width] (row bytes rb, swizzle swz(row)). sb: 32-row sub-block,
// t: 16-row k step, dc: 32-column block, half: which 4 of the lane's 8 rows.
template <typename Swz>
__device__ __forceinline__ int tr_addr(int lane, int rb, Swz swz, int sb, int t, int dc, int half) {
    const int vi = lane & 15;
    const int hh = lane >> 5;
    const int row = 32 * sb + 16 * t + 8 * hh + 4 * half + (vi >> 2);
    const int col = 32 * dc + 16 * ((lane >> 4) & 1) + 4 * (vi & 3);
    const int c = (col >> 3) ^ swz(row);
    return row * rb + 16 * c + 2 * (col & 7);
}

// Two transposing reads forming one bf16x8 A operand (see tr_addr).
template <typename Swz>
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char *tile, int lane, int rb, Swz swz, int sb, int t,
                                          int dc) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + tr_addr(lane, rb, swz, sb, t, dc, 0)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tile + tr_addr(lane, rb, swz, sb, t, dc, 1)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace da
