// attn_w3.hip -- ring-shard attention kernel for gfx950 with 128 query rows
// per workgroup: three workgroups per compute unit, or (for launches of at
// most one workgroup per compute unit) one workgroup of two key groups.
//
// Same computation as attn_pp.hip (one non-causal softmax-attention sweep of
// a query block over K/V tiles; the running float32 (max, sum, output) state
// is the log-sum-exp merge of the partials seen so far -- context
// parallelism guide "Paralelisme konteks", section "Ring Attention";
// Parallelism API page, ContextParallelConfig.convert_to_fp32), organised
// around instruction-issue parallelism:
//
//  * One workgroup = 4 waves = 128 query rows of one (batch, head), one wave
//    per SIMD; three workgroups share a compute unit, so every SIMD runs
//    three independent waves.  A wave's own stream (MFMAs, LDS reads, the
//    softmax VALU work) is serial; three of them keep the matrix pipe fed,
//    and while one workgroup waits at its barrier the other two run.
//  * K/V tiles of 32 keys (8 KB each for D = 128) stream through three LDS
//    stages (48 KB per workgroup) by direct global->LDS loads issued two
//    tiles ahead; one workgroup barrier per tile.
//  * Per tile and wave: S^T = K Q^T as 8 MFMAs on one 32-key block (Q in
//    registers), the online softmax on 16 scores per lane (exact running max,
//    float32 row sums), O^T += V^T P^T as 8 MFMAs with V^T from transposing
//    LDS reads.
//  * At most 168 VGPRs per wave, so that three waves fit a SIMD.
//  * Key groups (KG = 2): when a launch has no more workgroups than compute
//    units, a CU would hold one 4-wave workgroup, one wave per SIMD.  Then
//    the workgroup runs 8 waves in two key groups over the same 128 rows:
//    group g sweeps tiles t_lo + g, t_lo + g + 2, ... with its own three
//    stages, and at the end the second group hands its partial state to the
//    first through LDS, which merges the two by their row maxima (the LSE
//    merge of two partials of the same rows) before the epilogue.
#include "attn_tiles.h"

#include <math.h>

#include <type_traits>

namespace ringattn {
namespace {

constexpr int kW3Waves = 4;
constexpr int kW3BlockM = 32 * kW3Waves;  // 128 query rows per workgroup
constexpr int kW3BlockN = 32;             // keys per tile
constexpr int kW3Stages = 3;

typedef __attribute__((address_space(3))) float lds_float;

template <int D, int KG>
struct W3Geo {
    static constexpr int WAVES = kW3Waves * KG;           // KG key groups of 4 row waves
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int GROUP_LDS = 2 * kW3Stages * kW3BlockN * D * 2;  // one key group's stages
    // with two key groups, the second hands its state to the first past the
    // first group's staging slices: D/2 + 2 words per lane of 4 waves
    static constexpr int XBASE = kW3Waves * kStageBytes;
    static constexpr int XWORDS = D / 32 * 16 + 2;
    static constexpr int LDS_BYTES = KG == 1 ? GROUP_LDS
                                     : (KG * GROUP_LDS > XBASE + XWORDS * 4 * 64 * kW3Waves
                                            ? KG * GROUP_LDS
                                            : XBASE + XWORDS * 4 * 64 * kW3Waves);
    static constexpr int ROW = D * 2;                     // bytes per K/V row
    static constexpr int KCH = D / 8;                     // 16-byte pieces per row
    static constexpr int TILE = kW3BlockN * ROW;          // bytes of one K (or V) tile
    static constexpr int RPL = 1024 / ROW;                // rows one wave-wide 16-byte load fills
    static constexpr int LPW = TILE / 1024 / kW3Waves;    // loads per wave, per tensor, per tile
    static constexpr int VM_PER_TILE = 2 * LPW;           // vmcnt events per wave per tile
    static_assert(LPW >= 1 && LPW * kW3Waves * 1024 == TILE, "tile split over waves");
};

template <int D, int MODE, bool CHUNKED, int KG>
__global__ __launch_bounds__((W3Geo<D, KG>::THREADS)) __attribute__((amdgpu_waves_per_eu(KG == 1 ? 3 : 2, KG == 1 ? 3 : 2)))
void attn_w3_kernel(const AttnArgs a) {
    using G = W3Geo<D, KG>;
    // Per key group, three stages: V tiles in [0, 3*TILE), K tiles in
    // [3*TILE, 6*TILE) of the group's region.
    __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave_id / kW3Waves;   // key group: tiles t_lo + kg, t_lo + kg + KG, ...
    const int wave = wave_id % kW3Waves; // row wave: query rows 32 wave .. 32 wave + 31
    const uint32_t lds_all = (uint32_t)(uintptr_t)(lds_byte *)smem;
    const uint32_t lds0 = lds_all + (uint32_t)kg * G::GROUP_LDS;
    constexpr uint32_t kKRegion = kW3Stages * G::TILE;
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
    const int T = t_hi - t_lo;
    const int len0 = a.ct.len[0];  // packed layout: the whole key range

    const int64_t HD = (int64_t)a.heads * D;
    const uint32_t row_stride = (uint32_t)(HD * 2);
    const unsigned char *kbase = (const unsigned char *)(a.k + (int64_t)b * a.kv_rows * HD + (int64_t)h * D);
    const unsigned char *vbase = (const unsigned char *)(a.v + (int64_t)b * a.kv_rows * HD + (int64_t)h * D);

    int c_ld = 0, c_sm = 0;  // chunk cursors of the two tile walks (chunked layout)
    auto tile_at = [&](int t, int &c, int64_t &row0, int &nv) __attribute__((always_inline)) {
        if constexpr (CHUNKED) {
            tile_info<kW3BlockN>(a.ct, t, c, row0, nv);
        } else {
            row0 = (int64_t)t * kW3BlockN;
            nv = min(kW3BlockN, len0 - t * kW3BlockN);
        }
    };

    // ---- Q operand (registers for the whole sweep) --------------------------
    const int64_t qrow = (int64_t)qt * kW3BlockM + wave * 32 + col;
    const int64_t qrow_ld = qrow < a.q_len ? qrow : a.q_len - 1;
    const uint16_t *qp = a.q + ((int64_t)b * a.q_pitch + qrow_ld) * HD + (int64_t)h * D + 8 * half;
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * s));

    // ---- direct global->LDS loads ---------------------------------------------
    // Load i of this wave fills tile rows [r0, r0 + RPL); lane -> row
    // r0 + lane / KCH at LDS piece lane % KCH, fetched from the swizzled piece.
    int ld_row[G::LPW];
    uint32_t ld_k[G::LPW], ld_v[G::LPW];
#pragma unroll
    for (int i = 0; i < G::LPW; ++i) {
        const int r = (wave * G::LPW + i) * G::RPL + lane / G::KCH;
        const int p = lane % G::KCH;
        ld_row[i] = r;
        ld_k[i] = (uint32_t)r * row_stride + (uint32_t)((p ^ k_swizzle<D>(r)) * 16);
        ld_v[i] = (uint32_t)r * row_stride + (uint32_t)((p ^ v_swizzle<D>(r)) * 16);
    }
    const int lds_slot = wave * G::LPW * 1024;
    auto issue_loads = [&](auto s, int t) __attribute__((always_inline)) {
        constexpr uint32_t S = decltype(s)::value;
        int64_t row0;
        int nv;
        tile_at(t, c_ld, row0, nv);
        const unsigned char *kt = kbase + row0 * (int64_t)row_stride;
        const unsigned char *vt = vbase + row0 * (int64_t)row_stride;
        const uint32_t kdst = lds0 + kKRegion + S * G::TILE + lds_slot;
        const uint32_t vdst = lds0 + S * G::TILE + lds_slot;
#pragma unroll
        for (int i = 0; i < G::LPW; ++i) {
            uint32_t ok = ld_k[i], ov = ld_v[i];
            if (nv < kW3BlockN) {
                // rows past the tile's valid rows re-read its last valid row:
                // finite data that the softmax masks (K) or weights by zero (V)
                const uint32_t back = (uint32_t)(ld_row[i] - min(ld_row[i], nv - 1)) * row_stride;
                ok -= back;
                ov -= back;
            }
            dma_load16(kt, ok, kdst + i * 1024);
            dma_load16(vt, ov, vdst + i * 1024);
        }
    };

    // ---- per-lane LDS read offsets ------------------------------------------
    // K operand: row key_of_row(col) of the 32-key tile, piece 2*st + half.
    const int krow = key_of_row(col);
    uint32_t kb[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
        kb[st] = opaque(lds0 + kKRegion + krow * G::ROW + (((2 * st + half) ^ k_swizzle<D>(krow)) << 4));
    // V^T operand via transposing reads: lane s of 16-lane group g reads row
    // 16*half + 8*st + s/4 (+4) at columns d0 + 4*(s%4) .. +3.
    const int s16 = lane & 15;
    const int g16 = lane >> 4;
    uint32_t vb[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int r = 16 * half + (s16 >> 2);
        const int piece = 4 * db + 2 * (g16 & 1) + ((s16 & 3) >> 1);
        vb[db] = opaque(lds0 + r * G::ROW + ((piece ^ v_swizzle<D>(r)) << 4) + ((s16 & 1) << 3));
    }

    // ---- sweep state --------------------------------------------------------
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = -INFINITY;     // running row max of the raw scores q.k
    float l0 = 0.f, l1 = 0.f;    // this lane's share of the running row sum
    const float sl2 = a.scale_log2e;
    constexpr int kDsRead = 0x100, kMfma = 0x008;

    // One tile in stage S: scores, online softmax, PV.  on_max() runs once
    // the row maxima are known: the step issues its tile loads there, where
    // the wait for the load unit to take them overlaps the max chain's
    // latency instead of holding up the step's first instructions.
    auto compute = [&](auto stage, int t, auto &&on_max) __attribute__((always_inline)) {
        constexpr uint32_t S = decltype(stage)::value;
        constexpr uint32_t KS = S * G::TILE, VS = S * G::TILE;
        // S^T = K Q^T: one 32-key block, lane half h holds keys 16h + v
        f32x16 s = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128_at(kb[st], KS), qreg[st], s, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
#pragma unroll
        for (int i = 0; i < D / 16 - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kMfma, 2, 0);

        int64_t row0_unused;
        int nv;
        tile_at(t, c_sm, row0_unused, nv);
        if (nv < kW3BlockN) {  // ragged tile: keys past the valid rows get -inf
            const int lim = nv - 16 * half;
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (v >= lim) s[v] = -INFINITY;
        }
        float mx = fmaxf(s[0], s[1]);
#pragma unroll
        for (int v = 2; v < 16; v += 2) mx = fmaxf(fmaxf(mx, s[v]), s[v + 1]);
        mx = fmaxf(mx, other_half(mx, half != 0));
        on_max();
        if (__any(mx > m_run)) {  // wave-uniform; rare once the row maxima settle
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2((m_run - m_new) * sl2);
            l0 *= alpha;
            l1 *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            m_run = m_new;
        }
        const float mc = m_run * sl2;
        bf16x8 pb[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p0 = fast_exp2(fmaf(s[e], sl2, -mc));
            const float p1 = fast_exp2(fmaf(s[8 + e], sl2, -mc));
            l0 += p0;  // float32 row sums: with a peaked softmax one term dominates
            l1 += p1;
            pb[0][e] = (__bf16)p0;
            pb[1][e] = (__bf16)p1;
        }
        // O^T += V^T P^T; step st covers keys 16*half + 8*st + 0..7
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const s16x4 lo = lds_tr_at(vb[db], VS + 8 * st * G::ROW);
                const s16x4 hi = lds_tr_at(vb[db], VS + (8 * st + 4) * G::ROW);
                const s16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb[st], o[db], 0, 0,
                                                                 0);
            }
        }
        constexpr int NPV = 2 * (D / 32);
        __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 1);
#pragma unroll
        for (int i = 0; i < NPV - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 1);
            __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(kMfma, 2, 1);
    };

    // ---- sweep: step j is tile t_lo + KG j + kg of each key group, in stage
    // j % 3; loads issued two steps ahead ------------------------------------
    // A group's step-j tile's loads are issued during step j-2 (into
    // the stage that its step j-3 used, released by the barrier at the end of
    // step j-3) and waited for before the barrier at the end of step j-1,
    // which publishes them to the whole workgroup.  The groups step together;
    // a group past its last tile only takes part in the barriers.
    const int Tg = (T - kg + KG - 1) / KG;   // this group's tiles
    const int Ts = (T + KG - 1) / KG;        // steps (the first group's tiles)
    auto tile_of = [&](int j) __attribute__((always_inline)) { return t_lo + KG * j + kg; };
    constexpr std::integral_constant<int, 0> I0{};
    constexpr std::integral_constant<int, 1> I1{};
    constexpr std::integral_constant<int, 2> I2{};
    if (Tg > 0) issue_loads(I0, tile_of(0));
    if (Tg > 1) issue_loads(I1, tile_of(1));
    wait_vmcnt<0>();
    wg_barrier();
    auto step = [&](auto sc, auto sl, int j) __attribute__((always_inline)) -> bool {
        if (j >= Ts) return false;
        auto loads = [&]() __attribute__((always_inline)) {
            if (j + 2 < Tg) issue_loads(sl, tile_of(j + 2));
        };
        __builtin_amdgcn_sched_barrier(0);
        if (j < Tg) compute(sc, tile_of(j), loads);
        else loads();
        __builtin_amdgcn_sched_barrier(0);
        if (j + 2 < Tg) wait_vmcnt<G::VM_PER_TILE>();
        else wait_vmcnt<0>();
        wg_barrier();
        return true;
    };
    for (int j = 0;; j += 3) {  // unrolled by three so that every stage index is a constant
        if (!step(I0, I2, j)) break;
        if (!step(I1, I0, j + 1)) break;
        if (!step(I2, I1, j + 2)) break;
    }

    float l_lane = l0 + l1;
    if constexpr (KG == 2) {
        // The second key group hands its partial state (O, the row max, this
        // lane's share of the row sum) through LDS, past the staging slices
        // of the first group's epilogue; the first group merges it with its
        // own by their maxima (the LSE merge of two partials of the same rows).
        constexpr int kWords = G::XWORDS;
        constexpr uint32_t kXBase = G::XBASE;
        const uint32_t xa = lds_all + kXBase + (uint32_t)(wave * 64 + lane) * 4;
        auto xat = [&](int k) __attribute__((always_inline)) { return (lds_float *)(uintptr_t)(xa + (uint32_t)k * 64 * kW3Waves * 4); };
        if (kg == 1) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) *xat(db * 16 + v) = o[db][v];
            *xat(kWords - 2) = m_run;
            *xat(kWords - 1) = l_lane;
        }
        wg_barrier();
        if (kg == 1) return;
        const float m1 = *xat(kWords - 2);
        const float l1s = *xat(kWords - 1);
        const float m = fmaxf(m_run, m1);
        // a side still at -inf (no keys) has nothing to add: its factor is
        // never formed from -inf - -inf
        const float a0 = m_run == m ? 1.f : fast_exp2((m_run - m) * sl2);
        const float a1 = m1 == m ? 1.f : fast_exp2((m1 - m) * sl2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[db][v] = o[db][v] * a0 + *xat(db * 16 + v) * a1;
        l_lane = l_lane * a0 + l1s * a1;
        m_run = m;
    }

    // ---- epilogue -------------------------------------------------------------
    const float l_tot = l_lane + other_half(l_lane, half != 0);
    if constexpr (MODE == kModeFinal || MODE == kModePartial) {
        // every wave passed the barrier after the last tile: the stages are free.
        // (The Accum merge keeps the direct per-lane form here: staged, it
        // measured 2 % slower on the Flux-like ring steps and no faster on
        // Ring Anything's.)
        static_assert(kW3Waves * kStageBytes <= G::GROUP_LDS, "staging fits the stages");
        write_rows_staged<D, MODE>(a, o, m_run, l_tot, T > 0, b, h, qrow - col, a.q_len, split, lane,
                                   lds0 + (uint32_t)wave * kStageBytes);
    } else {
        write_rows<D, MODE>(a, o, m_run, l_tot, T > 0, b, h, qrow, a.q_len, split, half);
    }
}

template <int D, bool CHUNKED, int KG>
hipError_t launch_w3_dc(const AttnArgs &a, EpilogueMode mode, hipStream_t stream) {
    const int64_t grid = (int64_t)a.n_qtiles * a.heads * a.batch * a.n_splits;
    constexpr int kW3Threads = W3Geo<D, KG>::THREADS;
    switch (mode) {
        case kModeFinal:
            hipLaunchKernelGGL((attn_w3_kernel<D, kModeFinal, CHUNKED, KG>), dim3((unsigned)grid), dim3(kW3Threads), 0,
                               stream, a);
            break;
        case kModePartial:
            hipLaunchKernelGGL((attn_w3_kernel<D, kModePartial, CHUNKED, KG>), dim3((unsigned)grid), dim3(kW3Threads),
                               0, stream, a);
            break;
        case kModeAccum:
            hipLaunchKernelGGL((attn_w3_kernel<D, kModeAccum, CHUNKED, KG>), dim3((unsigned)grid), dim3(kW3Threads), 0,
                               stream, a);
            break;
        case kModeAccumBf16:
            hipLaunchKernelGGL((attn_w3_kernel<D, kModeAccumBf16, CHUNKED, KG>), dim3((unsigned)grid),
                               dim3(kW3Threads), 0, stream, a);
            break;
    }
    return hipGetLastError();
}

template <int KG>
hipError_t launch_w3_kg(const AttnArgs &a, int head_dim, EpilogueMode mode, bool chunked, hipStream_t stream) {
    if (head_dim == 128)
        return chunked ? launch_w3_dc<128, true, KG>(a, mode, stream) : launch_w3_dc<128, false, KG>(a, mode, stream);
    return chunked ? launch_w3_dc<64, true, KG>(a, mode, stream) : launch_w3_dc<64, false, KG>(a, mode, stream);
}

}  // namespace

hipError_t launch_attn_w3(const AttnArgs &a, int head_dim, int key_groups, EpilogueMode mode, bool chunked,
                          hipStream_t stream) {
    return key_groups == 2 ? launch_w3_kg<2>(a, head_dim, mode, chunked, stream)
                           : launch_w3_kg<1>(a, head_dim, mode, chunked, stream);
}

}  // namespace ringattn
