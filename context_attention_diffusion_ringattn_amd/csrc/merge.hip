// merge.hip -- float32 log-sum-exp merge kernels (HBM-bound, no MFMA).
//
// The merge of attention partials over disjoint key sets by their LSE is the
// float32 step that ContextParallelConfig.convert_to_fp32 protects
// (Parallelism API page, "Paralelisme").  Each thread owns 4 consecutive
// head_dim elements of one (batch, row, head), so a wavefront reads and
// writes 1 KiB of contiguous output per instruction.
#include "kernels.h"

#include <math.h>

namespace ringattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;

// out/lse <- merge over n_splits partial slots (accum = 0), or
// out/lse <- merge(out/lse, merge over the slots) in place (accum = 1: the
// split ring step's float32 accumulator; where its lse is -inf it is
// replaced, never multiplied).  A workgroup owns kMergeSlice consecutive
// 16-byte pieces of the output (a contiguous range of every partial slot and
// of out, covering kMergeSlice / (D/4) whole (b, i, h) rows).  One thread per
// row first reads the row's split LSEs, writes the merged LSE and leaves the
// weights in LDS -- exp(l_s - lse) per split (0 for an empty split, whose
// slot is then never read) and the accumulator's own weight; then every
// thread merges its pieces.
constexpr int kMergePer = 2;
constexpr int kMergeSlice = kMergeThreads * kMergePer;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_slice_kernel(const MergeSplitsArgs a) {
    constexpr int G = D / 4;
    constexpr int NP = kMergeSlice / G;  // rows per workgroup
    constexpr int WS = kMaxSplits + 1;  // per row: the splits, then the accumulator
    __shared__ float w[NP * WS];
    const int NS = a.n_splits;
    const int64_t n4 = (int64_t)a.batch * a.q_len * a.heads * G;
    const int64_t e0 = (int64_t)blockIdx.x * kMergeSlice;
    const int64_t p0 = e0 / G;  // first (b, i, h) row of this workgroup
    const int np = (int)min((int64_t)NP, n4 / G - p0);
    if ((int)threadIdx.x < np) {
        const int64_t bih = p0 + threadIdx.x;
        const int64_t bi = bih / a.heads;
        const int h = (int)(bih - bi * a.heads);
        const int64_t b = bi / a.q_len, i = bi - b * a.q_len;
        const int64_t lse_idx = (b * a.heads + h) * a.q_len + i;
        const float *lp = a.part_lse + lse_idx;
        float mx = -INFINITY;
        for (int sp = 0; sp < NS; ++sp) mx = fmaxf(mx, lp[sp * a.split_lse_stride]);
        float lse = -INFINITY;
        if (mx != -INFINITY) {
            float sum = 0.f;
            for (int sp = 0; sp < NS; ++sp) {
                const float l = lp[sp * a.split_lse_stride];
                if (l != -INFINITY) sum += expf(l - mx);
            }
            lse = mx + logf(sum);
        }
        float wb = 1.f, wa = 0.f, lse_out = lse;
        if (a.accum) {
            const float la = a.lse[lse_idx];
            if (lse == -INFINITY) {  // no keys in any split: the accumulator is unchanged
                wa = 1.f;
                lse_out = la;
            } else if (la != -INFINITY) {
                lse_out = fmaxf(la, lse) + log1pf(expf(-fabsf(la - lse)));
                wa = expf(la - lse_out);
                wb = expf(lse - lse_out);
            }
        }
        for (int sp = 0; sp < NS; ++sp) {
            const float l = lp[sp * a.split_lse_stride];
            w[threadIdx.x * WS + sp] = (lse == -INFINITY || l == -INFINITY) ? 0.f : wb * expf(l - lse);
        }
        w[threadIdx.x * WS + kMaxSplits] = wa;
        a.lse[lse_idx] = lse_out;
    }
    __syncthreads();
    const f32x4 *part = (const f32x4 *)a.part_out;
    const int64_t stride4 = a.split_out_stride / 4;
#pragma unroll
    for (int k = 0; k < kMergePer; ++k) {
        const int le = k * kMergeThreads + threadIdx.x;
        const int64_t e = e0 + le;
        if (e >= n4) break;
        const float *we = w + (le / G) * WS;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < NS; ++sp) {
            const float ws = we[sp];
            if (ws != 0.f) acc += ws * part[sp * stride4 + e];
        }
        const float wa = we[kMaxSplits];
        if (wa != 0.f) acc += wa * ((const f32x4 *)a.out)[e];
        ((f32x4 *)a.out)[e] = acc;
    }
}

// acc <- merge(acc, part) in place.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge2_kernel(float *out_acc, float *lse_acc, const float *out_part,
                                                              const float *lse_part, int64_t q_len, int32_t batch,
                                                              int32_t heads) {
    constexpr int G = D / 4;
    const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    const int64_t n_rows = (int64_t)batch * q_len * heads;
    if (gid >= n_rows * G) return;
    const int g = (int)(gid % G);
    const int64_t bih = gid / G;
    const int h = (int)(bih % heads);
    const int64_t bi = bih / heads;
    const int64_t i = bi % q_len;
    const int64_t b = bi / q_len;
    const int64_t lse_idx = (b * heads + h) * q_len + i;
    const int64_t out_idx = bih * D + 4 * g;

    const float la = lse_acc[lse_idx];
    const float lb = lse_part[lse_idx];
    f32x4 *pa = (f32x4 *)(out_acc + out_idx);
    const f32x4 *pb = (const f32x4 *)(out_part + out_idx);
    f32x4 res;
    float lse;
    if (la == -INFINITY && lb == -INFINITY) {
        res = f32x4{0.f, 0.f, 0.f, 0.f};
        lse = -INFINITY;
    } else if (la == -INFINITY) {
        res = *pb;
        lse = lb;
    } else if (lb == -INFINITY) {
        res = *pa;
        lse = la;
    } else {
        lse = fmaxf(la, lb) + log1pf(expf(-fabsf(la - lb)));
        res = expf(la - lse) * (*pa) + expf(lb - lse) * (*pb);
    }
    *pa = res;
    // The D/4 threads of a row are consecutive lanes of one wavefront, so all
    // of them have read lse_acc (above) before lane g == 0 overwrites it.
    if (g == 0) lse_acc[lse_idx] = lse;
}

__global__ __launch_bounds__(kMergeThreads) void acc_init_kernel(float *out, float *lse, int64_t n_out4,
                                                                int64_t n_lse) {
    const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (gid < n_out4) ((f32x4 *)out)[gid] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (gid < n_lse) lse[gid] = -INFINITY;
}

__global__ __launch_bounds__(kMergeThreads) void acc_init_bf16_kernel(uint16_t *out, uint16_t *lse, int64_t n_out4,
                                                                     int64_t n_lse) {
    const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
    if (gid < n_out4) ((uint2 *)out)[gid] = uint2{0u, 0u};
    if (gid < n_lse) lse[gid] = 0xff80u;  // bf16 -inf
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kMergeThreads - 1) / kMergeThreads); }

}  // namespace

hipError_t launch_merge_splits(const MergeSplitsArgs &a, int head_dim, hipStream_t stream) {
    const int64_t n = (int64_t)a.batch * a.q_len * a.heads * (head_dim / 4);
    const int64_t grid = (n + kMergeSlice - 1) / kMergeSlice;
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_slice_kernel<128>, dim3((unsigned)grid), dim3(kMergeThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(merge_slice_kernel<64>, dim3((unsigned)grid), dim3(kMergeThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_merge2(float *out_acc, float *lse_acc, const float *out_part, const float *lse_part,
                         int64_t q_len, int32_t batch, int32_t heads, int32_t head_dim, hipStream_t stream) {
    const int64_t n = (int64_t)batch * q_len * heads * (head_dim / 4);
    if (head_dim == 128)
        hipLaunchKernelGGL(merge2_kernel<128>, dim3(blocks_for(n)), dim3(kMergeThreads), 0, stream, out_acc, lse_acc,
                           out_part, lse_part, q_len, batch, heads);
    else
        hipLaunchKernelGGL(merge2_kernel<64>, dim3(blocks_for(n)), dim3(kMergeThreads), 0, stream, out_acc, lse_acc,
                           out_part, lse_part, q_len, batch, heads);
    return hipGetLastError();
}

hipError_t launch_acc_init(float *out, float *lse, int64_t n_out, int64_t n_lse, hipStream_t stream) {
    const int64_t n4 = n_out / 4;
    const int64_t n = n4 > n_lse ? n4 : n_lse;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(acc_init_kernel, dim3(blocks_for(n)), dim3(kMergeThreads), 0, stream, out, lse, n4, n_lse);
    return hipGetLastError();
}

hipError_t launch_acc_init_bf16(uint16_t *out, uint16_t *lse, int64_t n_out, int64_t n_lse, hipStream_t stream) {
    const int64_t n4 = n_out / 4;
    const int64_t n = n4 > n_lse ? n4 : n_lse;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(acc_init_bf16_kernel, dim3(blocks_for(n)), dim3(kMergeThreads), 0, stream, out, lse, n4, n_lse);
    return hipGetLastError();
}

}  // namespace ringattn
