// lds_probe.hip -- LDS read bandwidth of one gfx950 compute unit for the two
// read forms the attention kernels use: ds_read_b128 (K operand) and
// ds_read_b64_tr_b16 (transposing V^T operand).  One workgroup per compute
// unit (96 KB of LDS each), 4 or 8 waves; every wave issues 16 independent
// conflict-free reads per iteration (addresses move with the iteration, sums
// kept live); bytes per clock from s_memtime per wave.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr size_t kLds = 96 * 1024;

template <int TR>
__global__ __launch_bounds__(512) void lds_kernel(unsigned *sink, int iters, long long *cycles) {
    extern __shared__ char dyn[];
    for (int i = threadIdx.x; i < 32 * 1024 / 4; i += blockDim.x) ((unsigned *)dyn)[i] = i * 2654435761u;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char *)dyn;
    u32x4 acc = {0, 0, 0, 0};
    s16x4 acc2 = {0, 0, 0, 0};
    const long long t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const unsigned off = (unsigned)(r * 4096 + wave * 1024 + (it & 7) * 1024) & 32767u;
            if (TR)
                acc2 += __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)(base + off + lane * 8));
            else
                acc += *(lds_u32x4 *)(uintptr_t)(base + off + lane * 16);
        }
    }
    const long long t1 = __builtin_readcyclecounter();
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ (unsigned)acc2[0] ^ (unsigned)acc2[3];
    if (lane == 0) cycles[blockIdx.x * 8 + wave] = t1 - t0;
}

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
    int cus = 256;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0);
    unsigned *sink;
    long long *cyc;
    if (hipMalloc(&sink, sizeof(unsigned) * cus * 512) != hipSuccess || hipMalloc(&cyc, sizeof(long long) * cus * 8) != hipSuccess) {
        std::printf("allocation failed\n");
        return 1;
    }
    long long *h = (long long *)std::malloc(sizeof(long long) * cus * 8);
    for (int tr = 0; tr < 2; ++tr)
        for (int th : {256, 512}) {
            auto k = tr ? lds_kernel<1> : lds_kernel<0>;
            (void)hipFuncSetAttribute((const void *)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
            hipLaunchKernelGGL(k, dim3(cus), dim3(th), kLds, 0, sink, 100, cyc);
            hipEvent_t e0, e1;
            (void)hipEventCreate(&e0);
            (void)hipEventCreate(&e1);
            (void)hipEventRecord(e0, 0);
            hipLaunchKernelGGL(k, dim3(cus), dim3(th), kLds, 0, sink, iters, cyc);
            (void)hipEventRecord(e1, 0);
            (void)hipEventSynchronize(e1);
            float ms = 0.f;
            (void)hipEventElapsedTime(&ms, e0, e1);
            (void)hipMemcpy(h, cyc, sizeof(long long) * cus * 8, hipMemcpyDeviceToHost);
            const int nw = th / 64;
            double c = 0;
            for (int i = 0; i < cus; ++i)
                for (int w = 0; w < nw; ++w) c += (double)h[i * 8 + w];
            c /= cus * nw;
            const double per_instr = tr ? 512.0 : 1024.0;
            const double bytes_cu = per_instr * 16.0 * iters * nw;
            std::printf("%-18s waves/CU %d: %6.1f bytes/clk/CU, %.2f clocks per wave-instruction per CU, %.1f GB/s per CU\n",
                        tr ? "ds_read_b64_tr_b16" : "ds_read_b128", nw, bytes_cu / c, c / (16.0 * iters * nw),
                        bytes_cu / (ms * 1e-3) / 1e9);
        }
    const hipError_t e = hipDeviceSynchronize();
    std::printf("status %s\n", hipGetErrorString(e));
    return e == hipSuccess ? 0 : 1;
}
