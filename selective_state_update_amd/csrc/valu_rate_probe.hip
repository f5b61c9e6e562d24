// valu_rate_probe.hip -- the issue rate of plain (non-packed) fp32 fma and of
// the hardware exp2 on this GPU, the two operations the selective scan's
// arithmetic roofline is built from.
//
// Each thread runs 16 independent chains (no dependency stalls), 1024-thread
// workgroups, two per compute unit (8 waves per SIMD); the code is compiled
// like libssu (packed fp32 instructions disabled, no contraction), so every
// fma is one v_fmac_f32 and every exp2 one v_exp_f32 plus the v_mul_f32 that
// forms its argument. Each thread writes one float to out[global id]; the
// grid covers out exactly. Prints lane operations per second and wave
// instructions per SIMD per clock (clock: the device attribute).
//
//   selective_state_update_amd/valu_rate_probe
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

constexpr int kChains = 16;

__global__ void __launch_bounds__(1024) fma_chains(float *out, float x, float y, int iters)
{
    float acc[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        acc[i] = static_cast<float>(threadIdx.x) * 1e-3f + static_cast<float>(i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i)
            acc[i] = fmaf(acc[i], x, y);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        s += acc[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(1024) exp2_chains(float *out, float x, int iters)
{
    float acc[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        acc[i] = static_cast<float>(threadIdx.x) * 1e-6f + static_cast<float>(i) * 1e-3f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i)
            acc[i] = __builtin_amdgcn_exp2f(acc[i] * x);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        s += acc[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

#define CHECK(expr)                                                                   \
    do {                                                                              \
        const hipError_t e_ = (expr);                                                 \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "%s failed: %s\n", #expr, hipGetErrorString(e_)); \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

}  // namespace

int main()
{
    int dev = 0, cus = 0, clk_khz = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, dev));
    const int blocks = cus * 2, threads = 1024, iters = 20000;
    float *out = nullptr;
    CHECK(hipMalloc(&out, sizeof(float) * blocks * threads));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    const double simds = 4.0 * cus, clock_hz = clk_khz * 1e3;
    std::printf("# %d compute units, clock attribute %.0f MHz, %d-thread groups x %d, %d chains per thread\n", cus,
                clock_hz / 1e6, threads, blocks, kChains);
    for (int kind = 0; kind < 2; ++kind) {
        const int n = kind == 0 ? iters : iters / 4;
        for (int rep = 0; rep < 3; ++rep) {
            CHECK(hipEventRecord(a));
            if (kind == 0)
                hipLaunchKernelGGL(fma_chains, dim3(blocks), dim3(threads), 0, 0, out, 0.999f, 1e-3f, n);
            else
                hipLaunchKernelGGL(exp2_chains, dim3(blocks), dim3(threads), 0, 0, out, 0.5f, n);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(b));
            CHECK(hipEventSynchronize(b));
            float ms = 0.0f;
            CHECK(hipEventElapsedTime(&ms, a, b));
            const double lane_ops = double(blocks) * threads * n * kChains;
            const double per_s = lane_ops / (ms * 1e-3);
            std::printf("%s: %.3f ms, %.2f T lane-ops/s, %.3f wave instructions per SIMD per clock\n",
                        kind == 0 ? "fma (v_fmac_f32)" : "exp2 (v_exp_f32 + its v_mul_f32)", ms, per_s / 1e12,
                        per_s / 64.0 / simds / clock_hz);
        }
    }
    CHECK(hipFree(out));
    return 0;
}
