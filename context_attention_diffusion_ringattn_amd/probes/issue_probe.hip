// issue_probe.hip -- how a gfx950 SIMD shares its issue between
// v_mfma_f32_32x32x16_bf16 and the softmax's vector work.
//
// One workgroup per compute unit (96 KB of LDS each forces that); every wave
// runs ITERS x 64 MFMAs on register operands (NCH independent accumulator
// chains, 8 unless stated) and, between consecutive MFMAs, NV fma-class VALU
// ops, NE exp2 (each on an independent register, followed by an add), and one
// 16-byte LDS read every LDSPER MFMAs (LDSPER = 0: none) whose result feeds a
// later MFMA as its A operand.  About half a second of MFMA work runs first,
// so that every row is timed at the loaded engine clock.  Measured per wave with s_memtime: cycles per MFMA slot; from the
// wall clock: the engine clock and the matrix rate.  A second mode runs two
// waves per SIMD with one doing only the MFMAs and the other only the vector
// ops, the arrangement of a ping-pong schedule (the role is chosen outside
// the loops: neither stream carries a per-slot branch).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr size_t kLds = 96 * 1024;

// ROLE 0: every wave runs the mixed stream.  ROLE 1: waves 0-3 run only the
// MFMAs, waves 4-7 (same SIMDs) only the vector ops.
template <int NV, int NE, int LDSPER, int ROLE, int NCH>
__global__ __launch_bounds__(512) void issue_kernel(float *sink, int iters, long long *cycles) {
    extern __shared__ char dyn[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < (int)(kLds / 4); i += blockDim.x) ((float *)dyn)[i] = 1e-3f * (i & 255);
    __syncthreads();
    const bool do_mfma = ROLE == 0 || wave < 4;
    const bool do_valu = ROLE == 0 || wave >= 4;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (lane + i));
        b[i] = (__bf16)(0.002f * (lane - i));
    }
    bf16x8 aop[4] = {a, a, a, a};
    f32x16 acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    float x[16], y[8], z[8];
    for (int i = 0; i < 16; ++i) x[i] = 0.5f + 0.01f * (lane + i);
    for (int i = 0; i < 8; ++i) {
        y[i] = -0.25f - 0.001f * (lane + i);
        z[i] = 0.f;
    }
    const float c1 = sink[0] + 0.999f, c2 = sink[1] + 1e-4f;
    const unsigned lbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)dyn + lane * 16 + wave * 1024;
    const long long t0 = __builtin_readcyclecounter();
    // One slot: an MFMA and/or the vector work.  The role test sits outside
    // the loops, so that neither stream carries a branch per slot.
    auto slot = [&](int it, int m, bool mf, bool va) __attribute__((always_inline)) {
        if (mf) {
            acc[m % NCH] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(LDSPER ? aop[m & 3] : a, b, acc[m % NCH], 0, 0, 0);
            if (LDSPER && (m % LDSPER) == 0)
                aop[m & 3] = *(lds_bf16x8 *)(uintptr_t)(lbase + ((unsigned)(m * 4096 + it * 64) & 32767u));
        }
        if (va) {
#pragma unroll
            for (int v = 0; v < NV; ++v) x[(m * NV + v) & 15] = fmaf(x[(m * NV + v) & 15], c1, c2);
#pragma unroll
            for (int e = 0; e < NE; ++e) z[(m * NE + e) & 7] += __builtin_amdgcn_exp2f(y[(m * NE + e) & 7]);
        }
        if (mf && va) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (NV + 2 * NE) __builtin_amdgcn_sched_group_barrier(0x002, NV + 2 * NE, 0);
            if (LDSPER && (m % LDSPER) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    if (ROLE == 0) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < 64; ++m) slot(it, m, true, true);
        }
    } else if (do_mfma) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < 64; ++m) slot(it, m, true, false);
        }
    } else if (do_valu) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < 64; ++m) slot(it, m, false, true);
        }
    }
    const long long t1 = __builtin_readcyclecounter();
    float s = 0.f;
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 16; ++j) s += acc[i][j];
    for (int i = 0; i < 16; ++i) s += x[i];
    for (int i = 0; i < 8; ++i) s += z[i];
    sink[2 + blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) cycles[blockIdx.x * 8 + wave] = t1 - t0;
}

static int g_cus = 256;
static float *g_sink;
static long long *g_cyc;

template <int NV, int NE, int LDSPER, int ROLE, int NCH = 8>
void run(int threads, int iters) {
    auto k = issue_kernel<NV, NE, LDSPER, ROLE, NCH>;
    if (hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds) != hipSuccess) {
        std::printf("attribute failed\n");
        std::exit(1);
    }
    hipLaunchKernelGGL(k, dim3(g_cus), dim3(threads), kLds, 0, g_sink, 10, g_cyc);  // warm-up
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL(k, dim3(g_cus), dim3(threads), kLds, 0, g_sink, iters, g_cyc);
    (void)hipEventRecord(e1, 0);
    (void)hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    const int nw = threads / 64;
    long long *h = (long long *)std::malloc(sizeof(long long) * g_cus * 8);
    (void)hipMemcpy(h, g_cyc, sizeof(long long) * g_cus * 8, hipMemcpyDeviceToHost);
    double cm = 0, cv = 0;
    int nm = 0, nv = 0;
    for (int c = 0; c < g_cus; ++c)
        for (int w = 0; w < nw; ++w) {
            const bool mf = ROLE == 0 || w < 4;
            (mf ? cm : cv) += (double)h[c * 8 + w];
            (mf ? nm : nv) += 1;
        }
    std::free(h);
    cm /= nm;
    const double slots = (double)iters * 64;
    const double mfma_per_simd = slots * (ROLE == 0 ? nw / 4 : 1);
    const double flops = 32768.0 * mfma_per_simd * 4 * g_cus;
    std::printf("%-5s chains %d NV=%2d NE=%d LDS every %d MFMA | waves/SIMD %d | MFMA-wave cycles per MFMA %6.2f", ROLE ? "split" : "mixed", NCH,
                NV, NE, LDSPER, nw / 4, cm / slots);
    if (ROLE) std::printf(" | vector-wave cycles per slot %6.2f", cv / nv / slots);
    std::printf(" | %.0f TFLOP/s in %.2f ms\n", flops / (ms * 1e-3) / 1e12, ms);
}

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 4000;
    (void)hipDeviceGetAttribute(&g_cus, hipDeviceAttributeMultiprocessorCount, 0);
    if (hipMalloc(&g_sink, sizeof(float) * (2 + (size_t)g_cus * 512)) != hipSuccess ||
        hipMalloc(&g_cyc, sizeof(long long) * g_cus * 8) != hipSuccess) {
        std::printf("allocation failed\n");
        return 1;
    }
    (void)hipMemset(g_sink, 0, sizeof(float) * 2);
    // The engine clock ramps up over the first tens of milliseconds of load:
    // about half a second of MFMA work first, so that every row is timed at
    // the loaded clock.
    {
        auto k = issue_kernel<0, 0, 0, 0, 8>;
        if (hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds) != hipSuccess) {
            std::printf("attribute failed\n");
            return 1;
        }
        for (int i = 0; i < 50; ++i) hipLaunchKernelGGL(k, dim3(g_cus), dim3(256), kLds, 0, g_sink, 4000, g_cyc);
        (void)hipDeviceSynchronize();
    }
    std::printf("compute units %d, %d iterations x 64 MFMA slots per wave\n", g_cus, iters);
    run<0, 0, 0, 0>(256, iters);
    run<0, 0, 0, 0, 2>(256, iters);
    run<0, 0, 0, 0, 1>(256, iters);
    run<0, 0, 0, 0>(512, iters / 2);
    run<2, 0, 0, 0>(256, iters);
    run<4, 0, 0, 0>(256, iters);
    run<6, 0, 0, 0>(256, iters);
    run<8, 0, 0, 0>(256, iters);
    run<0, 1, 0, 0>(256, iters);
    run<2, 1, 0, 0>(256, iters);
    run<3, 1, 0, 0>(256, iters);
    run<4, 1, 0, 0>(256, iters);
    run<6, 1, 0, 0>(256, iters);
    run<0, 2, 0, 0>(256, iters);
    run<2, 2, 0, 0>(256, iters);
    run<4, 2, 0, 0>(256, iters);
    run<0, 3, 0, 0>(256, iters);
    run<0, 4, 0, 0>(256, iters);
    run<0, 0, 1, 0>(256, iters);
    run<0, 0, 2, 0>(256, iters);
    run<3, 1, 2, 0>(256, iters);
    run<3, 1, 1, 0>(256, iters);
    run<4, 1, 0, 0>(512, iters / 2);
    run<3, 1, 2, 0>(512, iters / 2);
    run<3, 1, 1, 0>(512, iters / 2);
    run<4, 2, 1, 0>(512, iters / 2);
    run<4, 1, 0, 1>(512, iters);
    run<4, 2, 0, 1>(512, iters);
    const hipError_t e = hipDeviceSynchronize();
    std::printf("status %s\n", hipGetErrorString(e));
    return e == hipSuccess ? 0 : 1;
}
