// attn_pp.hip -- 8-wave ping-pong ring-shard attention kernel for gfx950.
//
// One non-causal softmax-attention sweep of a query block over K/V tiles,
// the running float32 (max, sum, output) state being the log-sum-exp merge of
// the partials seen so far (context parallelism guide "Paralelisme konteks",
// section "Ring Attention"; Parallelism API page,
// ContextParallelConfig.convert_to_fp32), organised for large query shards:
//
//  * One workgroup = 8 waves = 256 query rows of one (batch, head); each wave
//    owns 32 rows.  Every K/V tile brought into LDS is used by all 256 rows.
//  * Waves 0-3 (group A) and 4-7 (group B) share the four SIMDs pairwise and
//    run the same loop one phase apart.  A wave alternates an MFMA phase
//    (O^T += V^T P^T for tile t-1, then S^T = K Q^T for tile t) and a softmax
//    phase (tile t).  While group A issues MFMAs, group B does its softmax on
//    the VALU, and the other way round; workgroup barriers separate the
//    phases and the MFMA phase runs at raised wave priority so the matrix
//    pipe is fed first.  The MFMA phase is one software pipeline over both
//    products, the LDS reads of the next four MFMAs always in flight.
//  * K/V tiles stream through a ring of four LDS stages by direct
//    global->LDS loads, issued two tiles ahead; each wave waits only for its
//    own loads of the next tile before the barrier that publishes it.
//  * Softmax: row max by max3 + one cross-half lane swap; O and the row sum
//    are rescaled only when some row's max moved (wave-uniform branch).  The
//    running max is kept exact, so the largest probability of a row is
//    exactly 1 and its bf16 rounding in the PV product is exact -- with a
//    peaked softmax that one term carries the row.
//  * Packed K/V (one contiguous key range) needs no chunk table in the loop;
//    the padded Ring Anything buffer (chunks at a fixed stride) walks the
//    chunk table and never lets a tile straddle two chunks.
#include "attn_tiles.h"

#include <math.h>

#include <type_traits>

#ifdef RINGATTN_CYCLE_COUNTERS
// Measurement build only (build.py --cycles): per workgroup, the engine
// cycles (s_memtime) and 100 MHz reference ticks (s_memrealtime) its first
// wave spent in the sweep, between the barrier after the prologue and the
// barrier before the epilogue, and the sweep's tile count.
constexpr int kCycleSlots = 8192;
__device__ unsigned long long ringattn_cycle_log[kCycleSlots * 4];
extern "C" int ringattn_cycle_log_read(void *dst, size_t bytes) {
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(ringattn_cycle_log), bytes, 0, hipMemcpyDeviceToHost);
}
extern "C" int ringattn_cycle_log_slots() { return kCycleSlots; }
#endif

namespace ringattn {
namespace {

constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;
constexpr int kPPBlockM = 32 * kPPWaves;  // 256 query rows per workgroup

template <int D>
struct PPGeo {
    static constexpr int ROW = D * 2;                    // bytes per K/V row
    static constexpr int KCH = D / 8;                    // 16-byte pieces per row
    static constexpr int TILE = kBlockN * ROW;           // bytes of one K (or V) tile
    static constexpr int STAGE = 2 * TILE;               // K tile then V tile
    static constexpr int RPL = 1024 / ROW;               // rows one wave-wide 16-byte load fills
    static constexpr int LPW = TILE / 1024 / kPPWaves;   // loads per wave, per tensor, per tile
    static constexpr int VM_PER_TILE = 2 * LPW;          // vmcnt events per wave per tile
    static_assert(LPW >= 1 && LPW * kPPWaves * 1024 == TILE, "tile split over waves");
};

template <int D, int MODE, bool CHUNKED, bool MULTI>
__global__ __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_pp_kernel(const AttnArgs a) {
    using G = PPGeo<D>;
    // Four LDS stages: V tiles in [0, 4*TILE), K tiles in [4*TILE, 8*TILE).
    __shared__ __attribute__((aligned(1024))) unsigned char smem[8 * G::TILE];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_byte *)smem;
    constexpr uint32_t kKRegion = 4 * G::TILE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;   // 0: leads, 1: trails by one phase
    const int col = lane & 31;   // query row within the wave's 32 rows
    const int half = lane >> 5;  // which 32-lane half

    // ---- work assignment ------------------------------------------------
    int w = xcd_remap(blockIdx.x, gridDim.x);
    int qt, h, b, split, t_lo, t_hi, len0;
    int64_t q_first = 0, q_end = a.q_len, kv_first = 0;
    if constexpr (MULTI) {
        // one ring step of several ranks: find this tile's rank
        const int total = a.rank_qtile_start[a.n_ranks];
        const int g = w % total;
        w /= total;
        h = w % a.heads;
        b = w / a.heads;
        int r = 0;
        while (g >= a.rank_qtile_start[r + 1]) ++r;
        qt = g - a.rank_qtile_start[r];
        q_first = a.rank_q_begin[r];
        q_end = q_first + a.rank_q_len[r];
        kv_first = a.ct.row_start[r];
        len0 = a.ct.len[r];
        split = 0;
        t_lo = 0;
        t_hi = (len0 + kBlockN - 1) / kBlockN;
    } else {
        qt = w % a.n_qtiles;
        w /= a.n_qtiles;
        h = w % a.heads;
        w /= a.heads;
        b = w % a.batch;
        split = w / a.batch;
        t_lo = (int)((int64_t)split * a.ct.n_tiles / a.n_splits);
        t_hi = (int)((int64_t)(split + 1) * a.ct.n_tiles / a.n_splits);
        len0 = a.ct.len[0];  // packed layout: the whole key range
    }
    const int T = t_hi - t_lo;

    const int64_t HD = (int64_t)a.heads * D;
    const uint32_t row_stride = (uint32_t)(HD * 2);  // bytes between consecutive K/V rows
    const unsigned char *kbase = (const unsigned char *)(a.k + ((int64_t)b * a.kv_rows + kv_first) * HD + (int64_t)h * D);
    const unsigned char *vbase = (const unsigned char *)(a.v + ((int64_t)b * a.kv_rows + kv_first) * HD + (int64_t)h * D);

    int c_ld = 0, c_sm = 0;  // chunk cursors of the two tile walks (chunked layout)
    auto tile_at = [&](int t, int &c, int64_t &row0, int &nv) __attribute__((always_inline)) {
        if constexpr (CHUNKED) {
            tile_info(a.ct, t, c, row0, nv);
        } else {
            row0 = (int64_t)t * kBlockN;
            nv = min(kBlockN, len0 - t * kBlockN);
        }
    };

    // ---- Q operand (registers for the whole sweep) --------------------------
    const int64_t qrow = q_first + (int64_t)qt * kPPBlockM + wave * 32 + col;
    const int64_t qrow_ld = qrow < q_end ? qrow : q_end - 1;
    const uint16_t *qp = a.q + ((int64_t)b * a.q_pitch + qrow_ld) * HD + (int64_t)h * D + 8 * half;
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * s));

    // ---- per-lane constants of the direct global->LDS loads ---------------
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
            if (nv < kBlockN) {
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
    // K operand: row key_of_row(col) (+32 for the second key block), piece
    // 2*st + half.  The base registers are opaque to the compiler so that the
    // stage and block offsets become instruction immediates.
    const int krow = key_of_row(col);
    uint32_t kb[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
        kb[st] = opaque(lds0 + kKRegion + krow * G::ROW + (((2 * st + half) ^ k_swizzle<D>(krow)) << 4));
    // V^T operand via transposing reads: lane s of 16-lane group g reads row
    // j0 + s/4 at columns d0 + 4*(s%4) .. +3, d0 = 32*db + 16*(g%2); the group
    // then holds columns d0 .. d0+15 of rows j0 .. j0+3, one column per lane.
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
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    bf16x8 pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = bf16x8{};
    float m_run = -INFINITY;                 // running row max of the raw scores q.k
    float l0 = 0.f, l1 = 0.f, l2 = 0.f, l3 = 0.f;  // this lane's share of the running row sum
    const float sl2 = a.scale_log2e;

    // The MFMA phase: O^T += V^T P^T for the previous tile (V in stage sv)
    // and S^T = K Q^T for the current one (K in stage sk), as one software
    // pipeline over its MFMAs, numbered m = 0 .. NPV+NQK-1.  m < NPV: PV
    // step st = m / (D/32) (keys 32*(st>>1) + 16*half + 8*(st&1) + 0..7)
    // for output block db = m % (D/32), A operand V^T from two transposing
    // reads.  m >= NPV: QK step (m-NPV)/2 for key block (m-NPV)%2, A operand
    // K from one 16-byte read; the two key blocks' chains interleave.  The A
    // operand of MFMA m sits in ring[m % kRing], and MFMA m is followed by
    // the reads for MFMA m + kRing, so kRing MFMAs' reads stay in flight and
    // the reads of the first QK operands go out under the last PV MFMAs.
    // A scheduling fence after each MFMA and its reads keeps this order.
    constexpr int NPV = 4 * (D / 32);
    constexpr int NQK = 2 * (D / 16);
    constexpr int kRing = 4;
    static_assert(NPV % kRing == 0 && NQK >= kRing, "ring slots line up across the two products");
    bf16x8 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = bf16x8{};
    auto read_op = [&](int m, uint32_t VS, uint32_t KS) __attribute__((always_inline)) -> bf16x8 {
        if (m < NPV) {
            const int st = m / (D / 32), db = m % (D / 32);
            const int jrow = 32 * (st >> 1) + 8 * (st & 1);
            const s16x4 lo = lds_tr_at(vb[db], VS + jrow * G::ROW);
            const s16x4 hi = lds_tr_at(vb[db], VS + (jrow + 4) * G::ROW);
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        const int q = m - NPV;
        return lds_b128_at(kb[q >> 1], KS + (q & 1) * 32 * G::ROW);
    };
    auto mfma_at = [&](int m) __attribute__((always_inline)) {
        const bf16x8 op = ring[m % kRing];
        if (m < NPV) {
            const int st = m / (D / 32), db = m % (D / 32);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pb[st], o[db], 0, 0, 0);
        } else {
            const int q = m - NPV;
            if (q & 1) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[q >> 1], s1, 0, 0, 0);
            else s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qreg[q >> 1], s0, 0, 0, 0);
        }
    };
    // PV of the tile in stage sv.  Its last kRing MFMAs carry the reads of
    // the first QK operands (K in stage sk) whether or not a QK follows:
    // keeping the PV code on one path keeps the output accumulators in the
    // same registers on every step.
    auto pv_pipe = [&](auto sv, auto sk) __attribute__((always_inline)) {
        constexpr uint32_t VS = decltype(sv)::value * G::TILE;
        constexpr uint32_t KS = decltype(sk)::value * G::TILE;
#pragma unroll
        for (int m = 0; m < kRing; ++m) ring[m] = read_op(m, VS, KS);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NPV; ++m) {
            mfma_at(m);
            ring[m % kRing] = read_op(m + kRing, VS, KS);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // QK of the tile in stage sk; `first`: no PV precedes it in this phase,
    // so it reads its own first operands.
    auto qk_pipe = [&](auto sk, auto first) __attribute__((always_inline)) {
        constexpr uint32_t KS = decltype(sk)::value * G::TILE;
        if constexpr (decltype(first)::value) {
#pragma unroll
            for (int m = NPV; m < NPV + kRing; ++m) ring[m % kRing] = read_op(m, 0, KS);
        }
        s0 = f32x16{};
        s1 = f32x16{};
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = NPV; m < NPV + NQK; ++m) {
            mfma_at(m);
            if (m + kRing < NPV + NQK) ring[m % kRing] = read_op(m + kRing, 0, KS);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Online softmax of the scores of tile t (in s0, s1) -> probabilities pb.
    // on_max() runs once the row maxima are known (the softmax phase issues
    // its tile loads there, see below).
    auto softmax = [&](int t, auto &&on_max) __attribute__((always_inline)) {
        int64_t row0_unused;
        int nv;
        tile_at(t, c_sm, row0_unused, nv);
        if (nv < kBlockN) {  // ragged tile: keys past the valid rows get -inf
            // this lane's keys are 16*half + v (block 0) and 32 + 16*half + v
            const int lim0 = nv - 16 * half;
            const int lim1 = lim0 - 32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (v >= lim0) s0[v] = -INFINITY;
                if (v >= lim1) s1[v] = -INFINITY;
            }
        }
        // two independent max3 chains, one per 32-key block
        float ma = fmaxf(s0[0], s0[1]);
        float mb = fmaxf(s1[0], s1[1]);
#pragma unroll
        for (int v = 2; v < 16; v += 2) {
            ma = fmaxf(fmaxf(ma, s0[v]), s0[v + 1]);
            mb = fmaxf(fmaxf(mb, s1[v]), s1[v + 1]);
        }
        float mx = fmaxf(ma, mb);
        mx = fmaxf(mx, other_half(mx, half != 0));
        on_max();
        if (__any(mx > m_run)) {  // wave-uniform; rare once the row maxima settle
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2((m_run - m_new) * sl2);
            l0 *= alpha;
            l1 *= alpha;
            l2 *= alpha;
            l3 *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            m_run = m_new;
        }
        const float mc = m_run * sl2;
        // the row sum is taken over the float32 probabilities: with a peaked
        // softmax one term dominates it, and its bf16 rounding (2^-9
        // relative) would go straight into the LSE
        // In chunks of eight independent scores: their eight fmas, then the
        // eight exps, then the sums and the bf16 packing.  Left to itself
        // the compiler pairs each fma with its exp through one temporary
        // register, and the softmax wave (alone on its SIMD's vector unit in
        // this phase) waits on every pair.
#pragma unroll
        for (int e0 = 0; e0 < 8; e0 += 2) {
            float x[2][4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                x[k][0] = fmaf(s0[e0 + k], sl2, -mc);
                x[k][1] = fmaf(s0[8 + e0 + k], sl2, -mc);
                x[k][2] = fmaf(s1[e0 + k], sl2, -mc);
                x[k][3] = fmaf(s1[8 + e0 + k], sl2, -mc);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[k][i] = fast_exp2(x[k][i]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                l0 += x[k][0];
                l1 += x[k][1];
                l2 += x[k][2];
                l3 += x[k][3];
                pb[0][e0 + k] = (__bf16)x[k][0];
                pb[1][e0 + k] = (__bf16)x[k][1];
                pb[2][e0 + k] = (__bf16)x[k][2];
                pb[3][e0 + k] = (__bf16)x[k][3];
            }
        }
    };

    // ---- ping-pong sweep ------------------------------------------------------
    // Step j = MFMA phase (PV of tile j-1, QK of tile j) + softmax phase of
    // tile j; group B runs one phase behind group A, so phase k of the
    // workgroup is A's step-(k/2) MFMA phase and B's softmax phase, then the
    // other way round.  Tile j lives in stage j % 4.  Its loads are issued in
    // the softmax phases of step j-2 (phase 2j-3 by A, 2j-2 by B) and waited
    // for before the barrier that ends phase 2j-1; K(j) is first read in
    // phase 2j.  V(j) is last read in phase 2j+3 (B's MFMA phase of step
    // j+1); the loads of tile j+4 into the same stage are issued from phase
    // 2j+5 on.  Barriers per wave: 2 per step + 2 (the trailing group's
    // first, the leading group's last), for both groups.
    constexpr std::integral_constant<int, 0> I0{};
    constexpr std::integral_constant<int, 1> I1{};
    constexpr std::integral_constant<int, 2> I2{};
    constexpr std::integral_constant<int, 3> I3{};
    constexpr std::true_type FIRST{};
    constexpr std::false_type AFTER_PV{};
    if (T > 0) issue_loads(I0, t_lo);
    if (T > 1) issue_loads(I1, t_lo + 1);
    wait_vmcnt<0>();
    wg_barrier();
#ifdef RINGATTN_CYCLE_COUNTERS
    const unsigned long long cyc0 = __builtin_amdgcn_s_memtime();
    const unsigned long long ref0 = __builtin_amdgcn_s_memrealtime();
#endif
    if (grp == 1) wg_barrier();

    // The softmax phase of step j, with the waits and barriers around it.
    // Each group issues its share of the loads of tile j+2 in its softmax
    // phase -- never in the MFMA phase, where a stalled vector-memory issue
    // would idle the matrix pipe.  The loads go out once the row maxima are
    // known: the four waves of a group issue them together and each stalls
    // until the load unit takes its requests, a stall that there overlaps
    // the latency of the dependent max chain instead of delaying the phase's
    // first vector instruction.  Before the barrier that publishes tile j+1,
    // group B (end of its MFMA phase) has no later loads in flight and waits
    // for all; group A (end of its softmax phase) may leave the loads of
    // tile j+2 in flight.
    auto softmax_phase = [&](auto sl, int j) __attribute__((always_inline)) {
        if (grp == 1) wait_vmcnt<0>();
        wg_barrier();
        softmax(t_lo + j, [&]() __attribute__((always_inline)) {
            if (j + 2 < T) issue_loads(sl, t_lo + j + 2);
        });
        if (grp == 0) {
            if (j + 2 < T) wait_vmcnt<G::VM_PER_TILE>();
            else wait_vmcnt<0>();
        }
        wg_barrier();
    };
    // Step j >= 1 (j % 4 == J): the MFMA phase -- PV of tile j-1, then for
    // j < T the QK of tile j -- then, for j < T, the softmax phase of tile j.
    auto step = [&](auto jc, int j) __attribute__((always_inline)) -> bool {
        constexpr int J = decltype(jc)::value;
        constexpr std::integral_constant<int, J> SK{};
        constexpr std::integral_constant<int, (J + 3) % 4> SV{};
        constexpr std::integral_constant<int, (J + 2) % 4> SL{};
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        pv_pipe(SV, SK);
        if (j < T) qk_pipe(SK, AFTER_PV);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (j >= T) return false;
        softmax_phase(SL, j);
        return true;
    };
    if (T > 0) {
        // step 0: the QK of tile 0 alone, then its softmax phase
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        qk_pipe(I0, FIRST);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        softmax_phase(I2, 0);
        for (int j = 1;; j += 4) {  // unrolled by four so that every stage index is a constant
            if (!step(I1, j)) break;
            if (!step(I2, j + 1)) break;
            if (!step(I3, j + 2)) break;
            if (!step(I0, j + 3)) break;
        }
    }
    if (grp == 0) wg_barrier();  // both groups pass the same number of barriers
#ifdef RINGATTN_CYCLE_COUNTERS
    {
        const unsigned long long cyc1 = __builtin_amdgcn_s_memtime();
        const unsigned long long ref1 = __builtin_amdgcn_s_memrealtime();
        if (tid == 0 && blockIdx.x < (unsigned)kCycleSlots) {
            ringattn_cycle_log[blockIdx.x * 4 + 0] = cyc1 - cyc0;
            ringattn_cycle_log[blockIdx.x * 4 + 1] = ref1 - ref0;
            ringattn_cycle_log[blockIdx.x * 4 + 2] = (unsigned long long)T;
            ringattn_cycle_log[blockIdx.x * 4 + 3] = 0;
        }
    }
#endif

    // ---- epilogue -------------------------------------------------------------
    const float l_lane = (l0 + l1) + (l2 + l3);
    const float l_tot = l_lane + other_half(l_lane, half != 0);
    if constexpr (D == 128 && (MODE == kModeFinal || MODE == kModePartial || MODE == kModeAccum)) {
        // The K stages are free: the last QK phase ended before the barrier
        // both groups passed on their way here.  (The trailing group's last
        // MFMA phase still reads the first K operands of a QK that does not
        // run; those values feed no MFMA, so what they read does not matter.)
        // The V stages are not: waves of the trailing group may still read V
        // of the last tile, with no barrier after it.  At D = 64 the K stages
        // cannot hold the slices of all eight waves, so that head dim keeps
        // the direct stores.
        static_assert(kPPWaves * kStageBytes <= 4 * G::TILE, "staging fits the K stages");
        write_rows_staged<D, MODE>(a, o, m_run, l_tot, T > 0, b, h, qrow - col, q_end, split, lane,
                                   lds0 + kKRegion + (uint32_t)wave * kStageBytes);
    } else {
        write_rows<D, MODE>(a, o, m_run, l_tot, T > 0, b, h, qrow, q_end, split, half);
    }
}

template <int D, bool CHUNKED>
hipError_t launch_pp_dc(const AttnArgs &a, EpilogueMode mode, hipStream_t stream) {
    const int64_t grid = (int64_t)a.n_qtiles * a.heads * a.batch * a.n_splits;
    switch (mode) {
        case kModeFinal:
            hipLaunchKernelGGL((attn_pp_kernel<D, kModeFinal, CHUNKED, false>), dim3((unsigned)grid), dim3(kPPThreads), 0,
                               stream, a);
            break;
        case kModePartial:
            hipLaunchKernelGGL((attn_pp_kernel<D, kModePartial, CHUNKED, false>), dim3((unsigned)grid), dim3(kPPThreads), 0,
                               stream, a);
            break;
        case kModeAccum:
            hipLaunchKernelGGL((attn_pp_kernel<D, kModeAccum, CHUNKED, false>), dim3((unsigned)grid), dim3(kPPThreads), 0,
                               stream, a);
            break;
        case kModeAccumBf16:
            hipLaunchKernelGGL((attn_pp_kernel<D, kModeAccumBf16, CHUNKED, false>), dim3((unsigned)grid), dim3(kPPThreads),
                               0, stream, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_pp_multi(const AttnArgs &a, int head_dim, hipStream_t stream) {
    const int64_t grid = (int64_t)a.rank_qtile_start[a.n_ranks] * a.heads * a.batch;
    if (head_dim == 128)
        hipLaunchKernelGGL((attn_pp_kernel<128, kModeAccum, false, true>), dim3((unsigned)grid), dim3(kPPThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((attn_pp_kernel<64, kModeAccum, false, true>), dim3((unsigned)grid), dim3(kPPThreads), 0,
                           stream, a);
    return hipGetLastError();
}

hipError_t launch_attn_pp(const AttnArgs &a, int head_dim, EpilogueMode mode, bool chunked, hipStream_t stream) {
    if (head_dim == 128) return chunked ? launch_pp_dc<128, true>(a, mode, stream) : launch_pp_dc<128, false>(a, mode, stream);
    return chunked ? launch_pp_dc<64, true>(a, mode, stream) : launch_pp_dc<64, false>(a, mode, stream);
}

}  // namespace ringattn
