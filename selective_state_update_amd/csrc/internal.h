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
