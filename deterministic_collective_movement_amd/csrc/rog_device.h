// rog_device.h -- device helpers shared by the HIP kernels of librog.so
// (rog_kernels.hip: gathers; rog_reduce.hip: rank-ordered sums).
#pragma once

#include "rog_internal.h"

namespace rog {

typedef uint32_t vec16 __attribute__((ext_vector_type(4)));
// The same 16 bytes at any byte address.
typedef uint32_t vec16u __attribute__((ext_vector_type(4), aligned(1)));

// 16-byte loads: non-temporal (streamed past the caches) when NT, else cached.
template <bool NT>
__device__ __forceinline__ vec16 ld16(const vec16 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// The 16 bytes at p, any byte alignment.
template <bool NT>
__device__ __forceinline__ vec16 ldu16(const uint8_t *p) {
    const vec16u *q = reinterpret_cast<const vec16u *>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}

__device__ __forceinline__ void st16(vec16 *p, vec16 v) {
    if constexpr (kNtStore) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
    return __builtin_amdgcn_readfirstlane(x);
}

// floor(v / d) by the host-built multiplier (exact for every 32-bit v).
__device__ __forceinline__ uint32_t divide(uint32_t v, const Divider &d) {
    const uint32_t t = __umulhi(v, d.magic);
    return (t + ((v - t) >> d.sh1)) >> d.sh2;
}

// Workgroups go to the 8 XCDs round-robin (b mod 8).  Hand each XCD runs of
// kXcdRun consecutive chunks, so that neighbouring chunks -- which share the
// cache line a misaligned chunk straddles -- meet in the same L2.  A bijection
// on [0, n): whole spans of 8 * kXcdRun are permuted, the rest is left as is.
__device__ __forceinline__ uint32_t xcd_grouped(uint32_t b, uint32_t n) {
    constexpr uint32_t kSpan = kXcds * kXcdRun;
    if (kXcdRun <= 1 || b >= n - n % kSpan) return b;
    const uint32_t x = b % kXcds, k = b / kXcds;
    return (k / kXcdRun) * kSpan + x * kXcdRun + k % kXcdRun;
}

}  // namespace rog
