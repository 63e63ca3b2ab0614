// attn_tiles.h -- device helpers shared by the attention kernels: operand
// layouts of v_mfma_f32_32x32x16_bf16, LDS swizzles, tile lookup and the
// XCD-aware workgroup renumbering.  Internal; not part of the ABI.
#pragma once

#include "kernels.h"

namespace ringattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kXcds = 8;

// Hardware hands workgroup ids to the 8 XCDs round-robin; give XCD x the
// contiguous logical range [x*n/8, (x+1)*n/8) instead (a bijection for any n),
// so that the workgroups of one head run on one XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// K tile swizzle: piece c (16 bytes) of row r is stored at c ^ k_swizzle(r).
// A K-operand read has 16 lanes in flight reading keys {0..3, 16..19, 4..7,
// 20..23} (+32) at the same piece; the swizzle sends them to 16 distinct
// 16-byte bank groups (64 banks x 4 bytes).
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
    if constexpr (D == 128) {
        return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 1) << 3);
    } else {  // 128-byte rows: two rows share one 256-byte bank window
        return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 4) & 1) << 2);
    }
}

// V tile swizzle: a transposing read has 32 lanes in flight covering rows
// j0..j0+3 (j0 % 4 == 0) and 4 consecutive pieces; XOR on piece bits 2..3
// (D=128) or bit 2 (D=64, two rows per bank window) spreads them over
// distinct bank groups.
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
    if constexpr (D == 128) {
        return 4 * (r & 3);
    } else {
        return 4 * ((r >> 1) & 1);
    }
}

// The 32 rows of each S^T = K Q^T block are assigned to keys with the
// permutation j(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3), which makes each
// 32-lane half of the accumulator hold 16 consecutive keys: lane half h,
// accumulator element v <-> key 16h + v.  Those are exactly the keys the
// half must supply as the B operand (P^T) of O^T = V^T P^T.
__device__ __forceinline__ int key_of_row(int m) {
    return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// Tile t of a chunk table -> chunk c (advanced monotonically from its
// previous value), first K/V row and number of valid rows.
__device__ __forceinline__ void tile_info(const ChunkTable &ct, int t, int &c, int64_t &row0, int &nv) {
    while (t >= ct.tile_start[c + 1]) ++c;
    const int local = t - ct.tile_start[c];
    row0 = ct.row_start[c] + (int64_t)local * kBlockN;
    nv = min(kBlockN, ct.len[c] - local * kBlockN);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 lds_read_b128(const unsigned char *smem, int off) {
    return *(const bf16x8 *)(smem + off);
}

__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char *smem, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(smem + off));
}

}  // namespace ringattn
