// attn_fwd.hip -- ring-shard attention kernel for gfx950 (CDNA4).
//
// One workgroup owns 128 query rows of one (batch, head) and sweeps a range
// of K/V tiles (64 rows each) with an online softmax.  A tile never straddles
// two ring chunks, so each chunk is its own non-causal attention pass (context
// parallelism guide, "Paralelisme konteks", section "Ring Attention"), and at
// every tile boundary the running float32 (max, sum, output) state is the
// log-sum-exp merge of the partials seen so far (Parallelism API page,
// ContextParallelConfig.convert_to_fp32).  The epilogue either writes the
// normalised output and LSE, writes them into a split slot of the workspace,
// or LSE-merges them into float32 accumulators in place (one ring step).
//
// Mapping onto CDNA4:
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.  Computing the
//    transposed products puts one query row in each lane column (lane % 32), so
//    the row max / row sum are in-lane reductions plus one exchange between
//    the two 32-lane halves, and the probabilities P come out of the first
//    MFMA already in the register layout the second MFMA takes as its B
//    operand (no LDS round trip for P).
//  * The 32 rows of each S^T block are assigned to keys with the permutation
//    j(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3), which makes each lane half hold
//    16 consecutive keys: lane half h, accumulator element v <-> key 16h + v.
//  * Q lives in registers for the whole sweep (B operand of S^T).
//  * K and V tiles go from HBM/L2 straight into LDS with global_load_lds_dwordx4
//    (no VGPR staging), row-major, 16-byte pieces XOR-swizzled per row.  Each
//    wave-wide load writes 1 KiB of LDS linearly by lane, so the swizzle is
//    applied on the global side: lane p of a row fetches the piece that must
//    live at position p.
//  * The K operand is one 16-byte LDS read per lane.  The V^T operand is read
//    with ds_read_b64_tr_b16, which transposes a 4-key x 16-column block per
//    16-lane group, so V needs no transpose on its way into LDS.
//  * Two LDS stages: the loads of tile t+1 are issued before the MFMAs of tile
//    t; one barrier per tile.  The loop is unrolled by two so every LDS offset
//    is an immediate.
//  * Workgroups are renumbered so consecutive (q-tile, head) work lands on the
//    same XCD and shares that XCD's L2 for the head's K/V.
#include "attn_tiles.h"

#include <math.h>

#include <type_traits>

namespace ringattn {
namespace {

template <int D>
struct Geo {
    static constexpr int ROW = D * 2;                        // bytes per K/V row in LDS
    static constexpr int KCH = D / 8;                        // 16-byte pieces per row
    static constexpr int TILE = kBlockN * ROW;               // bytes of one K (or V) tile
    static constexpr int STAGE = 2 * TILE;                   // K tile then V tile
    static constexpr int ROWS_PER_LOAD = 1024 / ROW;         // rows one wave-wide 16-byte load fills
    static constexpr int LOADS_PER_WAVE = TILE / 1024 / 4;   // per tensor per tile, 4 waves
    static_assert(LOADS_PER_WAVE * 4 * 1024 == TILE, "tile split over waves");
};

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const AttnArgs a) {
    using G = Geo<D>;
    // Two separate LDS objects (not one array) so the compiler can tell that
    // the transposing reads of one stage never alias the in-flight direct
    // loads into the other, and does not wait for those loads early.
    __shared__ __attribute__((aligned(1024))) unsigned char stage0[G::STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char stage1[G::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;   // query row within the wave's 32 rows
    const int half = lane >> 5;  // which 32-lane half

    // ---- work assignment ------------------------------------------------
    int w = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = w % a.n_qtiles;
    w /= a.n_qtiles;
    const int h = w % a.heads;
    w /= a.heads;
    const int b = w % a.batch;
    const int split = w / a.batch;
    const int t_lo = (int)((int64_t)split * a.ct.n_tiles / a.n_splits);
    const int t_hi = (int)((int64_t)(split + 1) * a.ct.n_tiles / a.n_splits);

    const int64_t HD = (int64_t)a.heads * D;
    const uint32_t row_stride = (uint32_t)(HD * 2);  // bytes between consecutive K/V rows
    const unsigned char *kbase = (const unsigned char *)(a.k + (int64_t)b * a.kv_rows * HD + (int64_t)h * D);
    const unsigned char *vbase = (const unsigned char *)(a.v + (int64_t)b * a.kv_rows * HD + (int64_t)h * D);

    // ---- Q operand (registers for the whole sweep) --------------------------
    const int64_t qrow = (int64_t)qt * kBlockM + wave * 32 + col;
    const int64_t qrow_ld = qrow < a.q_len ? qrow : a.q_len - 1;
    const uint16_t *qp = a.q + ((int64_t)b * a.q_pitch + qrow_ld) * HD + (int64_t)h * D + 8 * half;
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * s));

    // ---- per-lane constants of the direct global->LDS loads ---------------
    // Load i of this wave fills tile rows [r0, r0 + ROWS_PER_LOAD); lane -> row
    // r0 + lane / KCH at LDS piece lane % KCH.
    int ld_row[G::LOADS_PER_WAVE];
    int ld_kpiece[G::LOADS_PER_WAVE];
    int ld_vpiece[G::LOADS_PER_WAVE];
#pragma unroll
    for (int i = 0; i < G::LOADS_PER_WAVE; ++i) {
        const int r = (wave * G::LOADS_PER_WAVE + i) * G::ROWS_PER_LOAD + lane / G::KCH;
        const int p = lane % G::KCH;
        ld_row[i] = r;
        ld_kpiece[i] = (p ^ k_swizzle<D>(r)) * 16;
        ld_vpiece[i] = (p ^ v_swizzle<D>(r)) * 16;
    }

    auto issue_loads = [&](int t, int &c, auto stage_tag) {
        int64_t row0;
        int nv;
        tile_info(a.ct, t, c, row0, nv);
        const unsigned char *kt = kbase + row0 * (int64_t)row_stride;
        const unsigned char *vt = vbase + row0 * (int64_t)row_stride;
        unsigned char *kdst = decltype(stage_tag)::value ? stage1 : stage0;
        unsigned char *vdst = kdst + G::TILE;
#pragma unroll
        for (int i = 0; i < G::LOADS_PER_WAVE; ++i) {
            // rows past the chunk's end re-read its last row: finite data that
            // the softmax masks (K) or weights by exactly zero (V)
            const uint32_t rr = (uint32_t)min(ld_row[i], nv - 1) * row_stride;
            const int lds_off = (wave * G::LOADS_PER_WAVE + i) * 1024;
            __builtin_amdgcn_global_load_lds((const void *)(kt + rr + ld_kpiece[i]), (lds_void *)(kdst + lds_off), 16,
                                             0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(vt + rr + ld_vpiece[i]), (lds_void *)(vdst + lds_off), 16,
                                             0, 0);
        }
    };

    // ---- per-lane LDS read offsets ------------------------------------------
    // K operand: row key_of_row(col) (+32 for the second key block), piece
    // 2*st + half.
    const int krow = key_of_row(col);
    int koff[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) koff[st] = krow * G::ROW + (((2 * st + half) ^ k_swizzle<D>(krow)) << 4);
    // V^T operand via transposing reads: lane s of 16-lane group g reads row
    // j0 + s/4 at columns d0 + 4*(s%4) .. +3, d0 = 32*db + 16*(g%2); the group
    // then holds columns d0 .. d0+15 of rows j0 .. j0+3, one column per lane.
    const int s16 = lane & 15;
    const int grp = lane >> 4;
    int voff[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int r = 16 * half + (s16 >> 2);
        const int piece = 4 * db + 2 * (grp & 1) + ((s16 & 3) >> 1);
        voff[db] = G::TILE + r * G::ROW + ((piece ^ v_swizzle<D>(r)) << 4) + ((s16 & 1) << 3);
    }

    // ---- sweep --------------------------------------------------------------
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = -INFINITY;  // running row max of the raw scores q.k
    float l_part = 0.f;       // this lane's share of the running row sum
    const float sl2 = a.scale_log2e;
    int c_cmp = 0, c_ld = 0;

    auto compute_tile = [&](auto stage_tag, int t) {
        const unsigned char *smem = decltype(stage_tag)::value ? stage1 : stage0;
        constexpr int SOFF = 0;
        int64_t row0_unused;
        int nv;
        tile_info(a.ct, t, c_cmp, row0_unused, nv);

        // S^T = K Q^T for two 32-key blocks, interleaved so the two
        // accumulation chains hide each other's latency
        f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const bf16x8 k0 = lds_read_b128(smem, koff[st] + SOFF);
            const bf16x8 k1 = lds_read_b128(smem, koff[st] + SOFF + 32 * G::ROW);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qreg[st], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qreg[st], s1, 0, 0, 0);
        }

        // ragged chunk tail: keys past the chunk's true length get -inf
        if (nv < kBlockN) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (16 * half + v >= nv) s0[v] = -INFINITY;
                if (32 + 16 * half + v >= nv) s1[v] = -INFINITY;
            }
        }

        // online softmax
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {  // wave-uniform: rescale only when a row max moved
            const float alpha = fast_exp2((m_run - m_new) * sl2);
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            m_run = m_new;
        }
        const float mc = m_run * sl2;
        bf16x8 pb[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p0 = fast_exp2(fmaf(s0[e], sl2, -mc));
            const float p1 = fast_exp2(fmaf(s0[8 + e], sl2, -mc));
            const float p2 = fast_exp2(fmaf(s1[e], sl2, -mc));
            const float p3 = fast_exp2(fmaf(s1[8 + e], sl2, -mc));
            l_part += (p0 + p1) + (p2 + p3);
            pb[0][e] = (__bf16)p0;
            pb[1][e] = (__bf16)p1;
            pb[2][e] = (__bf16)p2;
            pb[3][e] = (__bf16)p3;
        }

        // O^T += V^T P^T; step st covers keys 32*(st>>1) + 16*half + 8*(st&1) + 0..7
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int jrow = 32 * (st >> 1) + 8 * (st & 1);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const s16x4 lo = lds_read_tr(smem, voff[db] + SOFF + jrow * G::ROW);
                const s16x4 hi = lds_read_tr(smem, voff[db] + SOFF + (jrow + 4) * G::ROW);
                const s16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb[st], o[db], 0, 0,
                                                                 0);
            }
        }
    };

    const int n_t = t_hi - t_lo;
    constexpr std::integral_constant<int, 0> kStage0{};
    constexpr std::integral_constant<int, 1> kStage1{};
    if (n_t > 0) issue_loads(t_lo, c_ld, kStage0);
    __syncthreads();
    for (int t = t_lo; t < t_hi; t += 2) {
        if (t + 1 < t_hi) issue_loads(t + 1, c_ld, kStage1);
        compute_tile(kStage0, t);
        __syncthreads();
        if (t + 1 >= t_hi) break;
        if (t + 2 < t_hi) issue_loads(t + 2, c_ld, kStage0);
        compute_tile(kStage1, t + 1);
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------------
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (qrow >= a.q_len) return;
    const bool any_keys = n_t > 0;
    if (MODE == kModeAccum && !any_keys) return;

    float *orow = a.out + ((int64_t)b * a.q_pitch + qrow) * HD + (int64_t)h * D + 4 * half;
    float *lptr = a.lse + ((int64_t)b * a.heads + h) * a.lse_pitch + qrow;
    if (MODE == kModePartial) {
        orow += (int64_t)split * a.split_out_stride;
        lptr += (int64_t)split * a.split_lse_stride;
    }
    const float inv_l = any_keys ? 1.f / l_tot : 0.f;
    const float lse_chunk = any_keys ? fmaf(m_run, a.scale, logf(l_tot)) : -INFINITY;

    if (MODE == kModeAccum) {
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

template <int D>
hipError_t launch_attn_d(const AttnArgs &a, EpilogueMode mode, hipStream_t stream) {
    const int64_t grid = (int64_t)a.n_qtiles * a.heads * a.batch * a.n_splits;
    switch (mode) {
        case kModeFinal:
            hipLaunchKernelGGL((attn_fwd_kernel<D, kModeFinal>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
            break;
        case kModePartial:
            hipLaunchKernelGGL((attn_fwd_kernel<D, kModePartial>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
            break;
        case kModeAccum:
            hipLaunchKernelGGL((attn_fwd_kernel<D, kModeAccum>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs &a, int head_dim, EpilogueMode mode, hipStream_t stream) {
    if (head_dim == 128) return launch_attn_d<128>(a, mode, stream);
    return launch_attn_d<64>(a, mode, stream);
}

}  // namespace ringattn
