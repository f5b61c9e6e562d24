// internal.h -- pieces shared by libssu's translation units (not installed).
#ifndef SSU_INTERNAL_H
#define SSU_INTERNAL_H

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssu.h"

namespace ssu {

using f32x4 = float __attribute__((ext_vector_type(4)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));

// Record a one-line description for ssu_last_error() and return `s`.
ssu_status fail(ssu_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Per-device limits, queried once per device (host attribute queries only).
struct DeviceLimits {
    int lds_cu, lds_block;
};
DeviceLimits device_limits(int dev);

// Dynamic LDS that caps residency at `cap` workgroups per CU (0: no cap).
size_t lds_for_cap(int cap, int lds_cu, int lds_block);

// Read-only operands are never written while a kernel runs (the ABI forbids
// aliasing them with anything written), so they are read through the constant
// address space: at a uniform address the compiler can then always use the
// scalar cache, and waiting for them never waits on the vector-memory counter.
template <typename T>
__device__ __forceinline__ T load_ro(const T *ptr)
{
    return *(const __attribute__((address_space(4))) T *)(ptr);
}

template <bool NT>
__device__ __forceinline__ f32x4 load4(const float *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    else
        return *reinterpret_cast<const f32x4 *>(p);
}

template <bool NT>
__device__ __forceinline__ void store4(float *p, f32x4 v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
    else
        *reinterpret_cast<f32x4 *>(p) = v;
}

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2Hi = 0.693147182464599609375f;  // (float)ln 2
constexpr float kLn2Lo = -1.904654323148236e-09f;   // ln 2 - kLn2Hi

// softplus(v) = max(v, 0) + log1p(e) with e = exp(-|v|) in (0, 1], and
// log1p(e) = 2 atanh(s) = s q(s^2), s = e / (2 + e) in (0, 1/3]. q is a
// degree-4 polynomial fitted to 2 atanh(sqrt z) / sqrt z on z in [0, 1/9] by
// the Remez exchange (relative error 4e-9, under a tenth of an fp32 ulp;
// fit_softplus.py beside this file recomputes it). e is the hardware exp2 of
// t = -|v| log2(e) in fp32, times exp(r) ~ 1 + r for the residual
// r = -|v| - t ln 2 (ln 2 split in two, each product exact in an fma), so the
// rounding of t costs nothing. -|v| is clamped at -128, where exp2 is already
// 0 in fp32, so that infinite v give e = 0 rather than inf - inf; the
// positive part is a select that lets NaN through (fmaxf would drop it):
// softplus(+inf) = +inf, softplus(-inf) = 0, softplus(NaN) = NaN, and every
// finite v gives the same bits as without the clamp.
__device__ __forceinline__ float softplus_f32(float v)
{
    const float x = __builtin_amdgcn_fmed3f(-fabsf(v), -128.0f, 0.0f);  // NaN: carried by the select below
    const float t = x * kLog2e;
    const float ex = __builtin_amdgcn_exp2f(t);
    const float r = fmaf(-t, kLn2Lo, fmaf(-t, kLn2Hi, x));
    const float e = fmaf(ex, r, ex);
    const float sv = e * __builtin_amdgcn_rcpf(2.0f + e);
    const float z = sv * sv;
    float q = fmaf(2.817833424e-01f, z, 2.796060145e-01f);
    q = fmaf(q, z, 4.002490938e-01f);
    q = fmaf(q, z, 6.666631699e-01f);
    q = fmaf(q, z, 2.0f);
    return fmaf(sv, q, v <= 0.0f ? 0.0f : v);
}

// exp(x) in fp32 by the same method: the hardware exp2 of t = x log2(e), times
// 1 + r for the residual r = x - t ln 2, so that the rounding of t costs
// nothing (about 2 ulp in all). x is clamped to [-128, 128], beyond which the
// result is 0 or +inf anyway; the residual is applied as a product, so that
// an overflowed exp2 stays +inf; NaN is passed through.
__device__ __forceinline__ float exp_f32(float x)
{
    const float xc = __builtin_amdgcn_fmed3f(x, -128.0f, 128.0f);
    const float t = xc * kLog2e;
    const float ex = __builtin_amdgcn_exp2f(t);
    const float r = fmaf(-t, kLn2Lo, fmaf(-t, kLn2Hi, xc));
    return x == x ? ex * (1.0f + r) : x;
}

// Workgroups are dispatched round-robin over the 8 XCDs. Map the first
// floor(total/8)*8 of them so that logical ids [k*q, (k+1)*q) run on XCD k;
// the tail keeps its order. A bijection on [0, total).
__device__ __forceinline__ int xcd_order(int g, int total)
{
    const int q = total >> 3;
    if (g >= (q << 3))
        return g;
    return (g & 7) * q + (g >> 3);
}

}  // namespace ssu

#endif  // SSU_INTERNAL_H
