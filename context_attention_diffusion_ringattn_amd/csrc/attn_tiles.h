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
typedef __attribute__((address_space(3))) unsigned char lds_byte;

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
// N: keys per tile of the table (the table's tile_start counts N-key tiles).
template <int N = kBlockN>
__device__ __forceinline__ void tile_info(const ChunkTable &ct, int t, int &c, int64_t &row0, int &nv) {
    while (t >= ct.tile_start[c + 1]) ++c;
    const int local = t - ct.tile_start[c];
    row0 = ct.row_start[c] + (int64_t)local * N;
    nv = min(N, ct.len[c] - local * N);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 lds_read_b128(const unsigned char *smem, int off) {
    return *(const bf16x8 *)(smem + off);
}

__device__ __forceinline__ s16x4 lds_read_tr(const unsigned char *smem, int off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(smem + off));
}

// ---- building blocks of the streaming kernels ------------------------------

// Workgroup barrier that neither the compiler's scheduler nor its memory
// optimisations move anything across, and that (unlike __syncthreads) does
// not wait for the in-flight global->LDS loads of later tiles.
__device__ __forceinline__ void wg_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// A value the compiler cannot see through (no instruction is emitted).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
}

// LDS reads at a lane base address plus a constant offset (folded into the
// instruction's 16-bit offset field).
__device__ __forceinline__ bf16x8 lds_b128_at(uint32_t base, uint32_t off) {
    return *(const bf16x8 *)((const lds_byte *)base + off);
}
__device__ __forceinline__ s16x4 lds_tr_at(uint32_t base, uint32_t off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)((lds_byte *)base + off));
}

// Direct global->LDS load of 16 bytes per lane: lane l's 16 bytes from
// gbase + voff land at LDS address lds_dst + 16 l (lds_dst wave-uniform, in
// M0).  Written as inline assembly on purpose: with the builtin in the loop,
// the compiler treats every LDS read as completing out of order and waits for
// all of them before each use; hidden from it, the LDS reads get exact
// counts.  Completion is tracked by vmcnt, which this kernel waits on
// explicitly before the barrier that publishes a tile.  The "memory" clobber
// tells the compiler LDS (and anything else) may change here.
__device__ __forceinline__ void dma_load16(const unsigned char *gbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_dst), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_sched_barrier(0);
}

// The value of lane i ^ 32 (the other half of the wave).
// v_permlane32_swap_b32 exchanges the upper 32 lanes of its first operand
// with the lower 32 lanes of its second: for inputs (a, b) it leaves
// a' = [a_lo, b_lo] and b' = [a_hi, b_hi]; with a = b = x, lane i then holds
// x[i ^ 32] in b' (lower lanes) or a' (upper lanes).  It is issued as inline
// assembly because the compiler's builtin folding drops one of the two
// results when they feed a floating-point max or add.  The s_nop pairs cover
// the VALU-write -> permlane-read hazard before and the permlane-write ->
// VALU-read hazard after, which the hazard recognizer cannot see through
// inline assembly.
__device__ __forceinline__ float other_half(float x, bool upper) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return upper ? a : b;
}

// Epilogue shared by the streaming kernels: one lane's 4*D/32 outputs of
// query row `qrow` (head h, batch b; rows at or past q_end are not written)
// and, from the lower half, its LSE.
//   Final: out = O / l, lse = m*scale + ln l.
//   Partial: the same into K/V-split slot `split` of the workspace.
//   Accum: LSE-merge (out, lse) into the float32 accumulators in place; where
//     the stored lse is -inf the partial is copied, never multiplied.
//   AccumBf16: the same with bf16 accumulators, the partial rounded to bf16.
// With no keys at all the result is out = 0, lse = -inf (merge modes: no-op).
template <int D, int MODE>
__device__ __forceinline__ void write_rows(const AttnArgs &a, const f32x16 (&o)[D / 32], float m_run, float l_tot,
                                           bool any_keys, int b, int h, int64_t qrow, int64_t q_end, int split,
                                           int half) {
    const int64_t HD = (int64_t)a.heads * D;
    if (qrow >= q_end) return;
    if ((MODE == kModeAccum || MODE == kModeAccumBf16) && !any_keys) return;

    float *orow = a.out + ((int64_t)b * a.q_pitch + qrow) * HD + (int64_t)h * D + 4 * half;
    float *lptr = a.lse + ((int64_t)b * a.heads + h) * a.lse_pitch + qrow;
    if (MODE == kModePartial) {
        orow += (int64_t)split * a.split_out_stride;
        lptr += (int64_t)split * a.split_lse_stride;
    }
    const float inv_l = any_keys ? 1.f / l_tot : 0.f;
    const float lse_chunk = any_keys ? fmaf(m_run, a.scale, logf(l_tot)) : -INFINITY;

    if (MODE == kModeAccumBf16) {
        // Accumulators kept in bf16 between steps: the partial is rounded to
        // bf16 (as a bf16-output attention pass returns it), merged in
        // float32 with the stored state, and the result rounded back.
        uint16_t *o16 = (uint16_t *)a.out + ((int64_t)b * a.q_pitch + qrow) * HD + (int64_t)h * D + 4 * half;
        uint16_t *l16 = (uint16_t *)a.lse + ((int64_t)b * a.heads + h) * a.lse_pitch + qrow;
        const float lc = (float)(__bf16)lse_chunk;
        const float la = (float)__builtin_bit_cast(__bf16, *l16);
        float wa, wb, lse_new;
        if (la == -INFINITY) {
            wa = 0.f;
            wb = 1.f;
            lse_new = lc;
        } else {
            lse_new = fmaxf(la, lc) + log1pf(expf(-fabsf(la - lc)));
            wa = expf(la - lse_new);
            wb = expf(lc - lse_new);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint16_t *p = o16 + 32 * db + 8 * g;
                const uint2 cur = *(const uint2 *)p;
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float part = (float)(__bf16)(o[db][4 * g + e] * inv_l);
                    const uint32_t word = e < 2 ? cur.x : cur.y;
                    const uint16_t bits = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
                    const float acc = (float)__builtin_bit_cast(__bf16, bits);
                    r[e] = la == -INFINITY ? part : fmaf(wa, acc, wb * part);
                }
                uint2 res;
                res.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)r[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)r[1]) << 16);
                res.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)r[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)r[3]) << 16);
                *(uint2 *)p = res;
            }
        }
        if (half == 0) *l16 = __builtin_bit_cast(uint16_t, (__bf16)lse_new);
    } else if (MODE == kModeAccum) {
        const float la = *lptr;
        float wa, wb, lse_new;
        if (la == -INFINITY) {
            wa = 0.f;
            wb = 1.f;
            lse_new = lse_chunk;
        } else {
            lse_new = fmaxf(la, lse_chunk) + log1pf(expf(-fabsf(la - lse_chunk)));
            wa = expf(la - lse_new);
            wb = expf(lse_chunk - lse_new);
        }
        wb *= inv_l;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 *p = (f32x4 *)(orow + 32 * db + 8 * g);
                const f32x4 cur = f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
                f32x4 res = cur * wb;
                if (la != -INFINITY) res += wa * (*p);
                *p = res;
            }
        }
        if (half == 0) *lptr = lse_new;
    } else {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                *(f32x4 *)(orow + 32 * db + 8 * g) =
                    f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]} * inv_l;
            }
        }
        if (half == 0) *lptr = lse_chunk;
    }
}

// The final (or split-partial) output of one wave's 32 rows, staged through
// LDS so that every global store writes whole 128-byte row segments.  In the
// MFMA layout an f32x4 store covers 32 bytes of each of 32 rows; here the
// wave writes its rows to `scratch` (kStageRowFloats floats per row, padded
// against bank conflicts), then each store instruction covers eight rows of
// 32 consecutive floats.  The LDS exchange stays inside the wave (LDS
// operations of one wave complete in order), so every lane takes part and
// only the global accesses of rows at or past q_end are skipped.  `row0` is
// the wave's first query row, `scratch` an LDS byte address of
// 32 * kStageRowFloats * 4 bytes that no other wave touches.
// Accum (the ring step's in-place LSE merge into the float32 accumulator):
// each lane works out its row's weights from the stored and the new LSE, as
// write_rows does, scales its outputs by the new side's weight before
// staging them, and leaves the stored side's weight (and whether the stored
// LSE is -inf) in the row's padding words; the read-back lanes then read the
// accumulator in the same whole row segments they write.
constexpr int kStageRowFloats = 36;
constexpr uint32_t kStageBytes = 32u * kStageRowFloats * 4u;

template <int D, int MODE>
__device__ __forceinline__ void write_rows_staged(const AttnArgs &a, const f32x16 (&o)[D / 32], float m_run,
                                                  float l_tot, bool any_keys, int b, int h, int64_t row0,
                                                  int64_t q_end, int split, int lane, uint32_t scratch) {
    static_assert(MODE == kModeFinal || MODE == kModePartial || MODE == kModeAccum, "float32 modes");
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    typedef __attribute__((address_space(3))) float lds_f32;
    if (MODE == kModeAccum && !any_keys) return;  // merging an empty partial changes nothing
    const int col = lane & 31, half = lane >> 5;
    const int64_t HD = (int64_t)a.heads * D;
    float *obase = a.out + ((int64_t)b * a.q_pitch + row0) * HD + (int64_t)h * D;
    float *lptr = a.lse + ((int64_t)b * a.heads + h) * a.lse_pitch + row0 + col;
    if (MODE == kModePartial) {
        obase += (int64_t)split * a.split_out_stride;
        lptr += (int64_t)split * a.split_lse_stride;
    }
    const float inv_l = any_keys ? 1.f / l_tot : 0.f;
    const float lse_chunk = any_keys ? fmaf(m_run, a.scale, logf(l_tot)) : -INFINITY;
    const int rr = lane >> 3;       // read-back row within a group of eight
    const int c4 = 4 * (lane & 7);  // read-back first column
    const int64_t rows_left = q_end - row0;
    float w_self = inv_l;  // this lane's row: weight of the new partial's outputs
    float wa_rd[4];        // read-back rows 8k + rr: weight of the stored side
    bool copy_rd[4];       // ... and whether the stored LSE is -inf (copy, never multiply)
    if constexpr (MODE == kModeAccum) {
        const float la = col < rows_left ? *lptr : -INFINITY;
        float wa = 0.f, wb = 1.f, lse_new = lse_chunk;
        if (la != -INFINITY) {
            lse_new = fmaxf(la, lse_chunk) + log1pf(expf(-fabsf(la - lse_chunk)));
            wa = expf(la - lse_new);
            wb = expf(lse_chunk - lse_new);
        }
        w_self = wb * inv_l;
        if (half == 0) {
            *(lds_f32 *)(uintptr_t)(scratch + (uint32_t)(col * kStageRowFloats + 32) * 4u) = wa;
            *(lds_f32 *)(uintptr_t)(scratch + (uint32_t)(col * kStageRowFloats + 33) * 4u) =
                la == -INFINITY ? 1.f : 0.f;
            if (col < rows_left) *lptr = lse_new;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t rw = scratch + (uint32_t)((8 * k + rr) * kStageRowFloats) * 4u;
            wa_rd[k] = *(lds_f32 *)(uintptr_t)(rw + 32 * 4u);
            copy_rd[k] = *(lds_f32 *)(uintptr_t)(rw + 33 * 4u) != 0.f;
        }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t at = scratch + (uint32_t)(col * kStageRowFloats + 8 * g + 4 * half) * 4u;
            *(lds_f32x4 *)(uintptr_t)at =
                f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]} * w_self;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 8 * k + rr;
            f32x4 v = *(lds_f32x4 *)(uintptr_t)(scratch + (uint32_t)(r * kStageRowFloats + c4) * 4u);
            if (r < rows_left) {
                f32x4 *p = (f32x4 *)(obase + (int64_t)r * HD + 32 * db + c4);
                if constexpr (MODE == kModeAccum) {
                    if (!copy_rd[k]) v += wa_rd[k] * (*p);
                }
                *p = v;
            }
        }
    }
    if (MODE != kModeAccum && half == 0 && col < rows_left) *lptr = lse_chunk;
}

}  // namespace ringattn
