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
//  * K tiles are stored row-major in LDS with a 16-byte-granular XOR swizzle
//    so the A-operand reads (16 bytes per lane) are bank-conflict free.
//  * V tiles are transposed on their way into LDS (4 rows x 8 columns per
//    thread, repacked in registers) so the A operand of O^T = V^T P^T is one
//    16-byte LDS read per lane, also XOR-swizzled.
//  * Two LDS stages: the global loads of tile t+1 are issued before the MFMAs
//    of tile t and written to the other stage after them; one barrier per tile.
//  * Workgroups are renumbered so consecutive (q-tile, head) work lands on the
//    same XCD and shares that XCD's L2 for the head's K/V.
#include "kernels.h"

#include <math.h>

namespace ringattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;

// Hardware hands workgroup ids to the 8 XCDs round-robin; give XCD x the
// contiguous logical range [x*n/8, (x+1)*n/8) instead (a bijection for any n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int q = n / kXcds, r = n % kXcds;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// K tile: row-major [64][D] bf16, 16-byte piece `ch` of row `row` stored at
// piece ch ^ k_swizzle(row).  For the rows one A-operand read touches
// together (lanes 0..15 read keys 0..3, 16..19, 4..7, 20..23) the swizzle is a
// bijection onto distinct pieces.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
    if constexpr (D == 128) {
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    } else {
        return (row & 3) | (((row >> 4) & 1) << 2);
    }
}

// V^T tile: row-major [D][64] bf16 (128 bytes per d-row, 8 pieces of 8 keys),
// piece p of row d stored at p ^ v_swizzle(d).
__device__ __forceinline__ int v_swizzle(int d) { return (d ^ (d >> 3)) & 7; }

// Key index of S^T row m (see header comment).
__device__ __forceinline__ int key_of_row(int m) {
    return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

__device__ __forceinline__ void tile_info(const ChunkTable &ct, int t, int &c, int64_t &row0, int &nv) {
    while (t >= ct.tile_start[c + 1]) ++c;
    const int local = t - ct.tile_start[c];
    row0 = ct.row_start[c] + (int64_t)local * kBlockN;
    nv = min(kBlockN, ct.len[c] - local * kBlockN);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const AttnArgs a) {
    constexpr int KCH = D / 8;                               // 16-byte pieces per K row
    constexpr int K_BYTES = kBlockN * D * 2;
    constexpr int V_BYTES = D * kBlockN * 2;
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int K_PER_THREAD = kBlockN * KCH / kThreads;   // 4 (D=128) or 2 (D=64)
    constexpr int V_UNITS = (kBlockN / 4) * KCH;             // 4-row x 8-column units
    static_assert(K_PER_THREAD * kThreads == kBlockN * KCH, "K tile split");
    static_assert(V_UNITS <= kThreads, "V tile split");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

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
    const uint16_t *kbase = a.k + (int64_t)b * a.kv_rows * HD + (int64_t)h * D;
    const uint16_t *vbase = a.v + (int64_t)b * a.kv_rows * HD + (int64_t)h * D;

    // ---- Q operand (registers for the whole sweep) --------------------------
    const int64_t qrow = (int64_t)qt * kBlockM + wave * 32 + col;
    const int64_t qrow_ld = qrow < a.q_len ? qrow : a.q_len - 1;
    const uint16_t *qp = a.q + ((int64_t)b * a.q_len + qrow_ld) * HD + (int64_t)h * D + 8 * half;
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * s));

    // ---- global -> register staging of one K/V tile -----------------------
    u32x4 kst[K_PER_THREAD];
    u32x4 vst[4];
    const bool v_active = tid < V_UNITS;
    const int v_dc = tid % KCH;  // 8-column group of d
    const int v_jg = tid / KCH;  // 4-row group of keys

    auto load_tile = [&](int64_t row0, int nv) {
#pragma unroll
        for (int r = 0; r < K_PER_THREAD; ++r) {
            const int idx = tid + r * kThreads;
            const int row = idx / KCH, ch = idx % KCH;
            kst[r] = u32x4{0u, 0u, 0u, 0u};
            if (row < nv) kst[r] = *(const u32x4 *)(kbase + (row0 + row) * HD + ch * 8);
        }
        if (v_active) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 4 * v_jg + e;
                vst[e] = u32x4{0u, 0u, 0u, 0u};
                if (row < nv) vst[e] = *(const u32x4 *)(vbase + (row0 + row) * HD + v_dc * 8);
            }
        }
    };

    auto store_tile = [&](unsigned char *stage) {
        unsigned char *Ks = stage;
        unsigned char *Vs = stage + K_BYTES;
#pragma unroll
        for (int r = 0; r < K_PER_THREAD; ++r) {
            const int idx = tid + r * kThreads;
            const int row = idx / KCH, ch = idx % KCH;
            *(u32x4 *)(Ks + row * (D * 2) + ((ch ^ k_swizzle<D>(row)) << 4)) = kst[r];
        }
        if (v_active) {
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int k = dd >> 1;
                uint32_t lo, hi;
                if (dd & 1) {  // odd column: high halves
                    lo = (vst[0][k] >> 16) | (vst[1][k] & 0xffff0000u);
                    hi = (vst[2][k] >> 16) | (vst[3][k] & 0xffff0000u);
                } else {       // even column: low halves
                    lo = (vst[0][k] & 0xffffu) | (vst[1][k] << 16);
                    hi = (vst[2][k] & 0xffffu) | (vst[3][k] << 16);
                }
                const int d = v_dc * 8 + dd;
                *(u32x2 *)(Vs + d * (kBlockN * 2) + (((v_jg >> 1) ^ v_swizzle(d)) << 4) + ((v_jg & 1) << 3)) =
                    u32x2{lo, hi};
            }
        }
    };

    // ---- sweep --------------------------------------------------------------
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m_run = -INFINITY;  // running row max of the raw scores q.k
    float l_part = 0.f;       // this lane's share of the running row sum
    const float sl2 = a.scale_log2e;

    int c_cmp = 0, c_ld = 0;
    if (t_lo < t_hi) {
        int64_t r0;
        int nv;
        tile_info(a.ct, t_lo, c_ld, r0, nv);
        load_tile(r0, nv);
        store_tile(smem);
    }
    __syncthreads();

    for (int t = t_lo; t < t_hi; ++t) {
        const int stage = (t - t_lo) & 1;
        int64_t r0_cur;
        int nv_cur;
        tile_info(a.ct, t, c_cmp, r0_cur, nv_cur);
        const bool has_next = t + 1 < t_hi;
        if (has_next) {
            int64_t r0n;
            int nvn;
            tile_info(a.ct, t + 1, c_ld, r0n, nvn);
            load_tile(r0n, nvn);
        }
        const unsigned char *Ks = smem + stage * STAGE;
        const unsigned char *Vs = Ks + K_BYTES;

        // S^T = K Q^T: two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            s[jb] = f32x16{};
            const int jr = 32 * jb + key_of_row(col);
            const unsigned char *krow = Ks + jr * (D * 2);
            const int sw = k_swizzle<D>(jr);
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 kop = *(const bf16x8 *)(krow + (((2 * st + half) ^ sw) << 4));
                s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[st], s[jb], 0, 0, 0);
            }
        }

        // ragged chunk tail: keys past the chunk's true length get -inf
        if (nv_cur < kBlockN) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * jb + 16 * half + v >= nv_cur) s[jb][v] = -INFINITY;
        }

        // online softmax
        float mx = s[0][0];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[jb][v]);
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
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = fast_exp2(fmaf(s[jb][8 * tt + e], sl2, -mc));
                    l_part += p;
                    pb[2 * jb + tt][e] = (__bf16)p;
                }
            }
        }

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int d = 32 * db + col;
            const unsigned char *vrow = Vs + d * (kBlockN * 2);
            const int sw = v_swizzle(d);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int piece = 4 * (st >> 1) + 2 * half + (st & 1);
                const bf16x8 vop = *(const bf16x8 *)(vrow + ((piece ^ sw) << 4));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[st], o[db], 0, 0, 0);
            }
        }

        if (has_next) store_tile(smem + (stage ^ 1) * STAGE);
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------------
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (qrow >= a.q_len) return;
    const bool any_keys = t_hi > t_lo;
    if (MODE == kModeAccum && !any_keys) return;

    float *orow = a.out + ((int64_t)b * a.q_len + qrow) * HD + (int64_t)h * D + 4 * half;
    float *lptr = a.lse + ((int64_t)b * a.heads + h) * a.q_len + qrow;
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
