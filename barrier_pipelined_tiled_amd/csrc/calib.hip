// calib.hip -- measurement companion of the GEMM library (not part of it).
//
//   calib copy <MiB> <reps>     plain 16-byte-per-lane copy of <MiB> MiB; its
//                               FETCH_SIZE / WRITE_SIZE counter readings per
//                               dispatch calibrate the GEMM's traffic figures
//   calib mfma <const|random>   v_mfma_f32_32x32x16_f16 on all CUs with no
//                               memory traffic in the loop: the sustained MFMA
//                               throughput and shader clock, with operands that
//                               stay constant or change randomly every MFMA
//
// The clock is measured inside the kernel as s_memtime cycles over
// s_memrealtime ticks (a 100 MHz constant clock).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                      \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            std::exit(1);                                                             \
        }                                                                             \
    } while (0)

__global__ void copy_kernel(const int4_t* __restrict__ src, int4_t* __restrict__ dst, long long n16) {
    long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (; i < n16; i += stride) dst[i] = src[i];
}

// Each wave keeps 16 independent 32x32 accumulators busy; operand sets are
// rotated through 8 register pairs so that with RANDOM they change on every
// MFMA.  Loop trip count is a multiple of 8 so every index is static.
template <bool RANDOM>
__global__ __launch_bounds__(256, 1) void mfma_kernel(const _Float16* src, float* out, long long* clk, int iters) {
    half8_t a[8], b[8];
    for (int u = 0; u < 8; ++u)
        for (int i = 0; i < 8; ++i) {
            int idx = ((blockIdx.x * 256 + threadIdx.x) * 128 + u * 16 + i) & ((1 << 20) - 1);
            a[u][i] = RANDOM ? src[idx] : (_Float16)0.25f;
            b[u][i] = RANDOM ? src[(idx * 7 + 13) & ((1 << 20) - 1)] : (_Float16)0.5f;
        }
    float16_t acc[16];
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(j + u) & 7], b[(j * 3 + u) & 7], acc[j], 0, 0, 0);
    }
    const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[blockIdx.x * 2] = t1 - t0;
        clk[blockIdx.x * 2 + 1] = r1 - r0;
    }
}

static int run_copy(long long mib, int reps) {
    const long long bytes = mib << 20;
    int4_t *src, *dst;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMalloc(&dst, bytes));
    CHECK(hipMemset(src, 1, bytes));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const long long n16 = bytes / 16;
    for (int r = 0; r < reps; ++r) {
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, 0, src, dst, n16);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::printf("copy %lld MiB: %.1f us  %.1f GB/s (read+write)\n", mib, ms * 1e3, 2.0 * bytes / (ms * 1e-3) / 1e9);
    }
    return 0;
}

template <bool RANDOM>
static int run_mfma() {
    const int iters = 8192, grid = 256;
    _Float16* src;
    float* out;
    long long* clk;
    CHECK(hipMalloc(&src, (1 << 20) * 2));
    CHECK(hipMalloc(&out, grid * 256 * 4));
    CHECK(hipMalloc(&clk, grid * 2 * 8));
    std::vector<_Float16> h(1 << 20);
    unsigned x = 12345u;
    for (auto& v : h) {
        x = x * 1664525u + 1013904223u;                           // LCG, seeded
        v = (_Float16)(((x >> 8) & 0xffff) / 32768.0f - 1.0f);    // uniform in [-1, 1)
    }
    CHECK(hipMemcpy(src, h.data(), h.size() * 2, hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int rep = 0; rep < 4; ++rep) {
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(mfma_kernel<RANDOM>, dim3(grid), dim3(256), 0, 0, src, out, clk, iters);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        std::vector<long long> c(grid * 2);
        CHECK(hipMemcpy(c.data(), clk, c.size() * 8, hipMemcpyDeviceToHost));
        double cyc = 0, rt = 0;
        for (int i = 0; i < grid; ++i) {
            cyc += c[2 * i];
            rt += c[2 * i + 1];
        }
        cyc /= grid;
        rt /= grid;
        const double flops = 2.0 * 32 * 32 * 16 * 16.0 * iters * 4 * grid;
        std::printf("mfma %s: %.1f us  %.1f TFLOPS  clock %.3f GHz  %.2f cycles per MFMA\n", RANDOM ? "random" : "const",
                    ms * 1e3, flops / (ms * 1e-3) / 1e12, cyc / (rt / 100e6) / 1e9, cyc / (16.0 * iters));
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 2 && !std::strcmp(argv[1], "copy"))
        return run_copy(argc > 2 ? std::atoll(argv[2]) : 256, argc > 3 ? std::atoi(argv[3]) : 5);
    if (argc >= 3 && !std::strcmp(argv[1], "mfma"))
        return std::strcmp(argv[2], "random") ? run_mfma<false>() : run_mfma<true>();
    std::fprintf(stderr, "usage: calib copy <MiB> <reps> | calib mfma <const|random>\n");
    return 2;
}
