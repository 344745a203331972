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

// A 16-byte vector in the global address space: loads through such a pointer
// are global_load instructions, where a generic pointer rebuilt from scalar
// registers would give flat_load (which also waits on the LDS counter and
// checks the address's aperture).
typedef const __attribute__((address_space(1))) vec16 gvec16;
template <bool NT>
__device__ __forceinline__ vec16 ld16(gvec16 *p) {
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

// Word 3 of a buffer resource for raw (untyped, unswizzled, unstrided) buffer
// accesses on CDNA: a 32-bit data format and nothing else set.
constexpr int kBufferWord3 = 0x00020000;

// A window [base, base + bytes) of an output, written by 16-byte buffer stores
// at byte offsets from base under the cache policy AUX.  base and bytes are
// wave-uniform (the resource lives in scalar registers), bytes < 2^31 and a
// multiple of 16; the hardware drops any store that would leave the window.
template <int AUX>
class OutWindow {
public:
    __device__ __forceinline__ OutWindow(void *base, uint32_t bytes)
        : r_(__builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), kBufferWord3)) {}
    __device__ __forceinline__ void st16(uint32_t off, vec16 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r_, int(off), 0, AUX);
    }

private:
    __amdgpu_buffer_rsrc_t r_;
};

// Bytes of [lo, hi) that a window starting at lo and at most cap long holds.
__device__ __forceinline__ uint32_t window_bytes(uint64_t lo, uint64_t hi, uint64_t cap) {
    return uint32_t(lo < hi ? (hi - lo < cap ? hi - lo : cap) : 0);
}

// Lane l gets lane l + 1's value, lane 63 gets 0: the whole-wave DPP shift
// of the gfx9 family (wave_shl:1, control 0x130), one v_mov_b32_dpp with no
// LDS traffic, where __shfl_down would take a ds_bpermute_b32.  The callers
// run it with the whole wave active.
__device__ __forceinline__ uint32_t from_next_lane(uint32_t x) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x130, 0xf, 0xf, false));
}
__device__ __forceinline__ vec16 from_next_lane(vec16 v) {
    return vec16{from_next_lane(v.x), from_next_lane(v.y), from_next_lane(v.z), from_next_lane(v.w)};
}

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
    return __builtin_amdgcn_readfirstlane(x);
}

// The low 32 bits of the 64-bit pair hi:lo shifted right by b = 0..3 bytes:
// one v_alignbyte_b32 on the device, the same shift written out on the host
// (where the CPU tests run it).
__host__ __device__ inline uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_alignbyte(hi, lo, b);
#else
    return uint32_t(((uint64_t(hi) << 32) | lo) >> (8 * b));
#endif
}

// Bytes [m, m + 16) of the 32 bytes lo then hi (little-endian), m = 0..15:
// dword k joins dwords q + k and q + k + 1 (q = m / 4) shifted by m % 4 bytes.
// m is wave-uniform in the kernels, so the switch is a scalar branch.
__host__ __device__ inline vec16 cut16(vec16 lo, vec16 hi, uint32_t m) {
    const uint32_t b = m & 3;
    switch (m >> 2) {
    case 0:
        return vec16{align_bytes(lo.y, lo.x, b), align_bytes(lo.z, lo.y, b), align_bytes(lo.w, lo.z, b),
                     align_bytes(hi.x, lo.w, b)};
    case 1:
        return vec16{align_bytes(lo.z, lo.y, b), align_bytes(lo.w, lo.z, b), align_bytes(hi.x, lo.w, b),
                     align_bytes(hi.y, hi.x, b)};
    case 2:
        return vec16{align_bytes(lo.w, lo.z, b), align_bytes(hi.x, lo.w, b), align_bytes(hi.y, hi.x, b),
                     align_bytes(hi.z, hi.y, b)};
    default:
        return vec16{align_bytes(hi.x, lo.w, b), align_bytes(hi.y, hi.x, b), align_bytes(hi.z, hi.y, b),
                     align_bytes(hi.w, hi.z, b)};
    }
}

// A launch's arguments read through the kernel-argument segment pointer.  The
// kernels take one argument struct by value, which the AMDGPU ABI places at
// offset 0 of that segment; reading it through the segment pointer keeps every
// read a scalar load from the segment, where mixing constant- and
// variable-index reads of the by-value parameter makes the compiler copy it
// to scratch first.
template <typename Args>
__device__ __forceinline__ const Args &launch_args() {
    // A C cast: it converts the constant address space of the segment pointer.
    return *(const Args *)__builtin_amdgcn_kernarg_segment_ptr();
}

// The payload pointers of a launch as the multi-WG FLAT kernel looks them up:
// the first eight are read into scalar registers together with the other
// kernel arguments, so that a wave's payload lookup (r < 8) is a few scalar
// selects rather than one more scalar load that the chunk's first data load
// would wait for; later payloads are read from the kernel arguments.
struct SrcTable {
    const void *const *all;       // every payload pointer (kernel arguments)
    const void *p0, *p1, *p2, *p3, *p4, *p5, *p6, *p7;
    __device__ __forceinline__ explicit SrcTable(const void *const *a)
        : all(a), p0(a[0]), p1(a[1]), p2(a[2]), p3(a[3]), p4(a[4]), p5(a[5]), p6(a[6]), p7(a[7]) {}
};
// Payload r's pointer, r wave-uniform.  Each half of every candidate goes
// through a cross-lane read (free on a value already in scalar registers), so
// that the selects stay scalar selects between registers and are not turned
// back into a load from a selected address.
__device__ __forceinline__ const void *src_of(const SrcTable &t, uint32_t r) {
    if (r >= 8) return t.all[r];
    const void *const c[8] = {t.p0, t.p1, t.p2, t.p3, t.p4, t.p5, t.p6, t.p7};
    uint32_t los[8], his[8];
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
        const uint64_t v = reinterpret_cast<uint64_t>(c[i]);
        los[i] = __builtin_amdgcn_readfirstlane(uint32_t(v));
        his[i] = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
    }
    uint32_t lo = los[0], hi = his[0];
#pragma unroll
    for (uint32_t i = 1; i < 8; ++i) {
        lo = r == i ? los[i] : lo;
        hi = r == i ? his[i] : hi;
    }
    return reinterpret_cast<const void *>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ const void *src_of(const void *const *src, uint32_t r) { return src[r]; }
// Payload rk's pointer for a per-lane rk (a chunk that crosses payloads).
__device__ __forceinline__ const void *lane_src(const void *const *src, uint32_t rk) { return src[rk]; }
__device__ __forceinline__ const void *lane_src(const SrcTable &t, uint32_t rk) { return t.all[rk]; }

// Makes the compiler hold the given values in scalar registers at this point,
// so that the kernel-argument reads behind them go out as one batch of scalar
// loads with one wait, before the first branch, rather than in dependent
// rounds: each round trip lengthens the life of every one-wave workgroup, and
// at full occupancy that costs copy throughput.  Emits no instruction.  One
// overload per argument set a kernel holds (FLAT; PEER and the batches; the
// sum).
__device__ __forceinline__ void hold_scalars(const SrcTable &t, uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t e, const Divider &div, const void *out) {
    asm volatile("" ::"s"(t.p0), "s"(t.p1), "s"(t.p2), "s"(t.p3), "s"(t.p4), "s"(t.p5), "s"(t.p6), "s"(t.p7),
                 "s"(a), "s"(b), "s"(c), "s"(d), "s"(e), "s"(div.magic), "s"(div.sh1), "s"(div.sh2), "s"(out));
}

__device__ __forceinline__ void hold_scalars(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t e) {
    asm volatile("" ::"s"(a), "s"(b), "s"(c), "s"(d), "s"(e));
}
__device__ __forceinline__ void hold_scalars(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t e,
                                             const Divider &div, const void *out) {
    asm volatile("" ::"s"(a), "s"(b), "s"(c), "s"(d), "s"(e), "s"(div.magic), "s"(div.sh1), "s"(div.sh2), "s"(out));
}
__device__ __forceinline__ void hold_scalars(const SrcTable &t, uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t e, const void *out) {
    asm volatile("" ::"s"(t.p0), "s"(t.p1), "s"(t.p2), "s"(t.p3), "s"(t.p4), "s"(t.p5), "s"(t.p6), "s"(t.p7),
                 "s"(a), "s"(b), "s"(c), "s"(d), "s"(e), "s"(out));
}

// floor(v / d) by the host-built multiplier (exact for every 32-bit v).
__device__ __forceinline__ uint32_t divide(uint32_t v, const Divider &d) {
    const uint32_t t = __umulhi(v, d.magic);
    return (t + ((v - t) >> d.sh1)) >> d.sh2;
}


}  // namespace rog
