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


}  // namespace rog
