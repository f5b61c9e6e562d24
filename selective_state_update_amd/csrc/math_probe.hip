// math_probe.hip -- the fp32 helpers the kernels share, checked exhaustively
// on the GPU against plain references computed there:
//   * bf16_round (the decode's output rounding, gfx950's v_cvt_pk_bf16_f32)
//     against a round-to-nearest-even written out in integer arithmetic, on
//     every one of the 2^32 fp32 bit patterns;
//   * exp_f32 (the decode's decay, internal.h) against the correctly rounded
//     (float)exp((double)x) on every fp32 x in [-110, 90]: the largest ulp
//     distance over normal results, and how many results below 2^-126 came
//     out other than the reference;
//   * exp_f32 and softplus_f32 at 0, -0, +inf, -inf, NaN.
// Prints one line per check, "key value ..." (read by the GPU test). Every
// thread's index is checked against its range before it reads or writes;
// counters are 64-bit device atomics.
//
//   selective_state_update_amd/math_probe
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "internal.h"

namespace {

__device__ __forceinline__ uint16_t rne_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint16_t hw_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// 16 patterns per thread: thread i of launch base covers base * 16 + [16 i, 16 i + 16)
__global__ void bf16_check(uint32_t base, unsigned long long *count)
{
    const uint32_t i = base + blockIdx.x * 256u + threadIdx.x;
    unsigned n = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float f = __uint_as_float(i * 16u + k);
        n += hw_bf16(f) != rne_bf16(f);
    }
    if (n)
        atomicAdd(count, static_cast<unsigned long long>(n));
}

__device__ __forceinline__ int64_t ordered(float f)
{
    const int32_t i = __float_as_int(f);
    return i < 0 ? -static_cast<int64_t>(i & 0x7fffffff) : static_cast<int64_t>(i);
}

// x = the fp32 pattern lo + k, k < n; acc[0] = max ulp distance over normal
// references, acc[1] = results below 2^-126 that differ from the reference
__global__ void exp_check(uint32_t lo, uint32_t n, unsigned long long *acc)
{
    const uint32_t k = blockIdx.x * 256u + threadIdx.x;
    if (k >= n)
        return;
    const float x = __uint_as_float(lo + k);
    const float got = ssu::exp_f32(x);
    const float ref = static_cast<float>(exp(static_cast<double>(x)));
    if (ref >= 1.17549435e-38f) {
        int64_t d = ordered(got) - ordered(ref);
        d = d < 0 ? -d : d;
        atomicMax(&acc[0], static_cast<unsigned long long>(d));
    } else if (got != ref) {
        atomicAdd(&acc[1], 1ull);
    }
}

__global__ void specials(float *out)
{
    const float in[5] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN};
    for (int i = 0; i < 5; ++i) {
        out[i] = ssu::exp_f32(in[i]);
        out[5 + i] = ssu::softplus_f32(in[i]);
    }
}

bool ok(hipError_t e) { return e == hipSuccess; }

}  // namespace

int main()
{
    unsigned long long *acc = nullptr;
    float *sp = nullptr;
    if (!ok(hipMalloc(&acc, 4 * sizeof(unsigned long long))) || !ok(hipMalloc(&sp, 10 * sizeof(float))))
        return 1;

    // bf16: 2^32 patterns = 16 launches of 2^20 blocks x 256 threads x 16
    if (!ok(hipMemset(acc, 0, 4 * sizeof(unsigned long long))))
        return 1;
    for (uint32_t L = 0; L < 16; ++L) {
        hipLaunchKernelGGL(bf16_check, dim3(1u << 16), dim3(256), 0, 0, L << 24, acc);
        if (!ok(hipGetLastError()))
            return 2;
    }
    unsigned long long h[4];
    if (!ok(hipDeviceSynchronize()) || !ok(hipMemcpy(h, acc, sizeof h, hipMemcpyDeviceToHost)))
        return 2;
    std::printf("bf16_mismatches %llu of 4294967296\n", h[0]);
    std::fflush(stdout);

    // exp: [0, 90] and [-110, -0] as fp32 patterns
    const uint32_t ranges[2][2] = {{0x00000000u, 0x42b40000u}, {0x80000000u, 0xc2dc0000u}};
    for (const auto &r : ranges) {
        if (!ok(hipMemset(acc, 0, 4 * sizeof(unsigned long long))))
            return 1;
        const uint32_t n = r[1] - r[0] + 1;
        hipLaunchKernelGGL(exp_check, dim3((n + 255) / 256), dim3(256), 0, 0, r[0], n, acc);
        if (!ok(hipGetLastError()) || !ok(hipDeviceSynchronize()) ||
            !ok(hipMemcpy(h, acc, sizeof h, hipMemcpyDeviceToHost)))
            return 3;
        std::printf("exp_range %08x %08x values %u max_ulp_normal %llu subnormal_differ %llu\n", r[0], r[1], n, h[0],
                    h[1]);
        std::fflush(stdout);
    }

    hipLaunchKernelGGL(specials, dim3(1), dim3(1), 0, 0, sp);
    float o[10];
    if (!ok(hipDeviceSynchronize()) || !ok(hipMemcpy(o, sp, sizeof o, hipMemcpyDeviceToHost)))
        return 4;
    std::printf("exp_specials %.9g %.9g %.9g %.9g %.9g\n", o[0], o[1], o[2], o[3], o[4]);
    std::printf("softplus_specials %.9g %.9g %.9g %.9g %.9g\n", o[5], o[6], o[7], o[8], o[9]);
    return 0;
}
