// rog_reduce.hip -- HIP kernels of the rank-ordered sum for gfx950 (CDNA4) and
// the C entry points that launch them.
//
// out[i] = round(((x_0[i] + x_1[i]) + x_2[i]) + ... + x_{W-1}[i]): the
// reduction of a deterministic all-reduce or reduce-scatter (RL-Align/RL-Kernel
// PR #491 names these collectives in "Not in this PR"; their single-block
// paths have the same size cliff as the gather had).  Every element is summed
// by exactly one lane, in rank order, in binary32 (v_add_f32, round to
// nearest-even, subnormals kept), and rounded once to the element type
// (v_cvt_pk_bf16_f32 for bf16, v_cvt_pk_f16_f32 for binary16), so the bits
// never depend on the launch.
//
// The output is cut like a PEER payload: an element head, a body of 16-byte
// vectors, an element tail.  The body starts at out's first 256-byte boundary
// (split_payload), or, in the granule form, where source 0 is read in whole
// 128-byte lines (split_anchored).  A body lane loads the 16 bytes at the same
// offset of every source, accumulates them in rank order and stores one
// aligned 16-byte vector.  Where the loads stay cached, each source takes one
// global_load_dwordx4 per lane at its own alignment, up to 8 sources' loads in
// flight; where they stream past the caches (ROG_PLAN_NT_LOADS, then
// ROG_PLAN_SHIFTED_LOADS), the launch takes the granule form, which reads every
// source as aligned granules, each lane rebuilding its bytes from its own
// granule and the next lane's, as the PEER gather does (measured faster there
// at every alignment, and mostly slower with cached loads), with 2, 4 or 8
// sources' granules in flight by W (sum_granule_group); the last lane of each
// wave reads one granule per source with a cached load, which for an aligned
// source of a sum of three or more (it needs none) is aimed so that those
// lines alternate between two 128-byte places of a 1 KiB block by rank.
// Multi-WG: one wave per 1 KiB chunk of the body, chunks handed to the XCDs in runs
// (xcd_grouped); single-WG: one workgroup strides over the whole output;
// batch (rog_reduce_many): every tensor's chunks in one launch.  Bandwidth
// bound: (W + 1) * count * esize bytes per sum.
#include <hip/hip_runtime.h>

#include "rog_device.h"

namespace rog {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Element type DT (a rog_dtype value).
template <int DT>
struct Elem {
    static constexpr bool kHalf = DT != ROG_DTYPE_F32;  // 2-byte elements
    static constexpr int kPerVec = kHalf ? 8 : 4;       // elements per 16-byte vector
    static constexpr uint32_t kSize = kHalf ? 2 : 4;
};

__device__ __forceinline__ float from_bits(uint32_t u) { return __builtin_bit_cast(float, u); }

// Two binary32 values -> two 2-byte elements (element 0 in the low half),
// nearest-even: v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32.
template <int DT>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    if constexpr (DT == ROG_DTYPE_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Two 2-byte elements (element 0 in the low half) -> binary32, exactly.
template <int DT>
__device__ __forceinline__ void widen2(uint32_t w, float &lo, float &hi) {
    if constexpr (DT == ROG_DTYPE_BF16) {
        lo = from_bits(w << 16);
        hi = from_bits(w & 0xFFFF0000u);
    } else {
        const f32x2 f = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
        lo = f.x;
        hi = f.y;
    }
}

// The elements of one 16-byte vector, widened to binary32.
template <int DT>
__device__ __forceinline__ void widen(const vec16 &v, float (&x)[Elem<DT>::kPerVec]) {
    if constexpr (Elem<DT>::kHalf) {
#pragma unroll
        for (int k = 0; k < 4; ++k) widen2<DT>(v[k], x[2 * k], x[2 * k + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = from_bits(v[k]);
    }
}

template <int DT>
__device__ __forceinline__ vec16 narrow(const float (&a)[Elem<DT>::kPerVec]) {
    vec16 v;
    if constexpr (Elem<DT>::kHalf) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = narrow2<DT>(a[2 * k], a[2 * k + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(uint32_t, a[k]);
    }
    return v;
}

// Lane 63's cached load of an aligned source in the granule form (see
// sum_vec_wave) goes to the next chunk's line whose 128-byte place alternates
// by rank from this many sources on (0: never), else to the next chunk's
// first granule.  Measured over W = 2 to 16, sources on one line place and
// buffers no cache holds: W = 5 to 16 gained 4-9 %, W = 4 3-4 % (0 to -3 %
// back to back over two boxes), W = 3 4 % (1-2 % lost where the three
// sources already sat on distinct places); W = 2 lost 1-2 %.  Other
// placements stayed within about 1 % from W = 4 on.  W = 2 takes the
// two-source granule group, which leaves it out.
#ifndef ROG_SUM_TOUCH_SPREAD_MIN_W
#define ROG_SUM_TOUCH_SPREAD_MIN_W 3
#endif
constexpr uint32_t kSumTouchSpreadMinW = ROG_SUM_TOUCH_SPREAD_MIN_W;
// Waves per SIMD the multi-WG sum kernels are compiled for at least: the
// 8-source granule form then keeps 5 (95 VGPRs; 98 and 4 waves otherwise,
// which measured up to 10 % slower at W = 4 and 6).
#ifndef ROG_SUM_WAVES_PER_EU
#define ROG_SUM_WAVES_PER_EU 5
#endif

#ifndef ROG_REDUCE_GROUP
#define ROG_REDUCE_GROUP 8
#endif
#ifndef ROG_REDUCE_XCD
#define ROG_REDUCE_XCD 1
#endif
constexpr uint32_t kGroup = ROG_REDUCE_GROUP;   // source loads in flight per lane

// The rank-ordered sum of the 16-byte vectors at byte offset off of every source.
template <int DT, bool NTL>
__device__ __forceinline__ vec16 sum_vec(const void *const *src, uint32_t W, uint64_t off) {
    constexpr int E = Elem<DT>::kPerVec;
    float acc[E];
    for (uint32_t r0 = 0; r0 < W; r0 += kGroup) {
        const uint32_t g = min(W - r0, kGroup);
        vec16 v[kGroup];
#pragma unroll
        for (uint32_t q = 0; q < kGroup; ++q)
            if (q < g) v[q] = ldu16<NTL>(static_cast<const uint8_t *>(src[r0 + q]) + off);
#pragma unroll
        for (uint32_t q = 0; q < kGroup; ++q) {
            if (q < g) {
                float x[E];
                widen<DT>(v[q], x);
                if (r0 + q == 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = x[e];       // the first term as it is
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] += x[e];
                }
            }
        }
    }
    return narrow<DT>(acc);
}

// sum_vec for a whole wave of a multi-WG chunk, reading every source as
// aligned 16-byte granules shared between neighbouring lanes (the PEER
// gather's scheme): every lane calls it, since the shuffle needs all 64.  G
// sources' granules are in flight at once (sum_granule_group).
// `live` lanes own a body vector at byte offset off; `own_hi` lanes (lane 63
// and the body's last lane) make one cached load per source themselves: the
// granule after their own where the source is misaligned, a granule of the
// next chunk where it is aligned.  body and hi are the body's first and end
// byte offsets: source r's bytes sit m_r = (src_r + body) % 16 bytes past a
// granule in every lane.
template <int DT, bool NTL, uint32_t G>
__device__ __forceinline__ vec16 sum_vec_wave(const void *const *src, uint32_t W, uint64_t off, uint64_t body,
                                              uint64_t hi, bool live, bool own_hi) {
    constexpr int E = Elem<DT>::kPerVec;
    float acc[E];
    for (uint32_t r0 = 0; r0 < W; r0 += G) {
        const uint32_t g = min(W - r0, G);
        vec16 v[G], h[G];
        uint32_t m[G];
        // The few cached loads of lane 63 (and the body's last lane) go out
        // before the group's streamed loads: issued after them, they waited
        // behind them and the sum ran 3-6% slower.  They are the sum's only
        // loads that allocate in the Infinity Cache.  On aligned sources they
        // read no byte of the sum, yet against none at all (W = 2 to 8) they
        // measured 5-14 % faster back to back over the same buffers, where
        // their lines are still there for the next call, 2-5 % faster over
        // buffers no cache holds, and 4-13 % slower after other work has left
        // dirty lines there (each allocation first writes one back).  Over
        // buffers no cache holds, the gain needs the loaded lines on several
        // 128-byte places of a 1 KiB block: when all W landed on one place,
        // as the first granule of the next chunk does for sources on 2 MiB
        // boundaries, the W = 8 sum ran 6.3 TB/s against 6.8-6.9 with the
        // places alternating by rank.  So from W = kSumTouchSpreadMinW on, an
        // aligned source's load goes to the next chunk's line that alternates
        // the place by rank, whatever the sources' own places.
#pragma unroll
        for (uint32_t q = 0; q < G; ++q) {
            v[q] = h[q] = vec16{0, 0, 0, 0};
            m[q] = 0;
            if (q < g) {
                const uint8_t *s = static_cast<const uint8_t *>(src[r0 + q]);
                const uint32_t a = uniform(uint32_t(reinterpret_cast<uintptr_t>(s) + body));
                m[q] = a & 15;
                const vec16 *gp = reinterpret_cast<const vec16 *>(s + off - m[q]);
                // Misaligned: the granule after the lane's own holds payload
                // bytes (line 0, read even past the body's end).  Aligned:
                // line `line` of the next chunk, whose place in a 1 KiB block,
                // (a >> 7) + line, is 4 * (r & 1); read inside the body only.
                // One conditional load with a uniform offset: split into two
                // branches, the loads waited for one another.
                uint32_t line = 0;
                if constexpr (G >= 4 && kSumTouchSpreadMinW != 0)   // the group of 2 serves W <= 2 only
                    if (W >= kSumTouchSpreadMinW && m[q] == 0) line = (4u * ((r0 + q) & 1u) - (a >> 7)) & 7u;
                if (own_hi && (m[q] != 0 || off + 32 + 128 * uint64_t(line) <= hi))
                    h[q] = ld16<false>(gp + 1 + 8 * line);
            }
        }
#pragma unroll
        for (uint32_t q = 0; q < G; ++q) {
            if (q < g && live) {
                const uint8_t *s = static_cast<const uint8_t *>(src[r0 + q]);
                v[q] = ld16<NTL>(reinterpret_cast<const vec16 *>(s + off - m[q]));
            }
        }
#pragma unroll
        for (uint32_t q = 0; q < G; ++q) {
            if (q < g) {
                const vec16 next = from_next_lane(v[q]);
                float x[E];
                widen<DT>(cut16(v[q], own_hi ? h[q] : next, m[q]), x);
                if (r0 + q == 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = x[e];       // the first term as it is
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] += x[e];
                }
            }
        }
    }
    return narrow<DT>(acc);
}

template <int DT>
__device__ __forceinline__ float load_elem(const void *p, uint64_t i) {
    if constexpr (Elem<DT>::kHalf) {
        float lo, hi;
        widen2<DT>(static_cast<const uint16_t *>(p)[i], lo, hi);
        return lo;
    } else {
        return static_cast<const float *>(p)[i];
    }
}

// One element: the rank-ordered sum of element i of every source, stored to out.
template <int DT>
__device__ __forceinline__ void sum_elem(const void *const *src, uint32_t W, uint64_t i, void *out) {
    float acc = load_elem<DT>(src[0], i);
    for (uint32_t r = 1; r < W; ++r) acc += load_elem<DT>(src[r], i);
    if constexpr (Elem<DT>::kHalf) static_cast<uint16_t *>(out)[i] = uint16_t(narrow2<DT>(acc, 0.0f) & 0xFFFFu);
    else static_cast<float *>(out)[i] = acc;
}

// One wave: body chunk j (body vectors [64j, 64j + 64)) of a sum of `count`
// elements into out; chunk 0 also sums the head and tail elements.  SH: the
// granule form (the plan's ROG_PLAN_SHIFTED_LOADS), its body cut so that
// source 0 is read in whole 128-byte lines (split_anchored); else one
// unaligned load per lane and source, the body cut at out's first 256-byte
// boundary (split_payload).
template <int DT, bool NTL, bool SH, uint32_t G>
__device__ __forceinline__ void sum_chunk(const void *const *src, uint32_t W, void *out, uint64_t count,
                                          uint32_t j) {
    const uint32_t lane = __lane_id();
    const uint64_t bytes = count * Elem<DT>::kSize;
    const PeerSplit cut = SH ? split_anchored(reinterpret_cast<uintptr_t>(out), bytes, reinterpret_cast<uintptr_t>(src[0]))
                             : split_payload(reinterpret_cast<uintptr_t>(out), bytes);
    if (j == 0) {
        for (uint64_t i = lane; i < cut.lo / Elem<DT>::kSize; i += 64) sum_elem<DT>(src, W, i, out);
        for (uint64_t i = cut.hi / Elem<DT>::kSize + lane; i < count; i += 64) sum_elem<DT>(src, W, i, out);
    }
    const uint64_t w0 = cut.lo + uint64_t(j) * 1024;  // the wave's first body byte
    const OutWindow<kSumStoreAux> w(static_cast<uint8_t *>(out) + w0, window_bytes(w0, cut.hi, 1024));
    const uint64_t off = w0 + 16 * lane;
    const bool live = off < cut.hi;
    if constexpr (SH) {
        const bool own_hi = live && (lane == 63 || off + 16 >= cut.hi);
        const vec16 v = sum_vec_wave<DT, NTL, G>(src, W, off, cut.lo, cut.hi, live, own_hi);
        if (live) w.st16(16 * lane, v);
    } else if (live) {
        w.st16(16 * lane, sum_vec<DT, NTL>(src, W, off));
    }
}

// Multi-WG: one wave per workgroup and per 1 KiB chunk of the body, chunks
// handed to the XCDs in runs (a chunk's last granule is its neighbour's
// first; without runs the granule form measured 8 % slower), grid-strided
// over a capped grid.
template <int DT, bool NTL, bool SH, uint32_t G>
__global__ __launch_bounds__(kWaveBlock) __attribute__((amdgpu_waves_per_eu(ROG_SUM_WAVES_PER_EU)))
void rog_reduce_kernel(ReduceArgs) {
    // Every argument the first chunk needs, the first eight source pointers
    // included, in one batch of scalar loads with one wait.
    const ReduceArgs &a = launch_args<ReduceArgs>();
    const SrcTable src(a.src);
    const uint32_t n_chunks = a.n_chunks, W = a.W, grid = a.grid;
    const uint64_t count = a.count;
    void *const out = a.out;
    hold_scalars(src, n_chunks, W, uint32_t(count), uint32_t(count >> 32), grid, out);
    for (uint32_t vb = blockIdx.x; vb < n_chunks; vb += grid)
        sum_chunk<DT, NTL, SH, G>(a.src, W, out, count, ROG_REDUCE_XCD ? xcd_grouped(vb, n_chunks) : vb);
}

// Batch: the tensors' chunks laid end to end; a wave finds its tensor by a
// scalar binary search over the tensors' first chunks.
template <int DT, bool NTL, bool SH, uint32_t G>
__global__ __launch_bounds__(kWaveBlock) __attribute__((amdgpu_waves_per_eu(ROG_SUM_WAVES_PER_EU)))
void rog_reduce_batch_kernel(ReduceBatchArgs) {
    const ReduceBatchArgs &a = launch_args<ReduceBatchArgs>();
    const uint32_t n_chunks = a.n_chunks, W = a.W, grid = a.grid;
    hold_scalars(n_chunks, a.n, W, grid, 0u);
    for (uint32_t vb = blockIdx.x; vb < n_chunks; vb += grid) {
        const uint32_t c = ROG_REDUCE_XCD ? xcd_grouped(vb, n_chunks) : vb;
        const uint32_t lo = search_tensor(a.first, a.n, c);
        const ReduceTensor &t = a.t[lo];
        // the output address through a global pointer: global head and tail stores
        void *const out = (void *)(__attribute__((address_space(1))) uint8_t *)t.out;
        sum_chunk<DT, NTL, SH, G>(a.src + lo * W, W, out, t.count, c - a.first[lo]);
    }
}

// Single-WG: one workgroup over the whole output.
template <int DT, bool NTL>
__global__ __launch_bounds__(kSingleBlock) void rog_reduce_single_kernel(ReduceArgs a) {
    const uint32_t tid = threadIdx.x, nt = blockDim.x;
    const uint64_t bytes = a.count * Elem<DT>::kSize;
    const PeerSplit cut = split_payload(reinterpret_cast<uintptr_t>(a.out), bytes);
    uint8_t *o = static_cast<uint8_t *>(a.out);
    for (uint64_t i = tid; i < cut.lo / Elem<DT>::kSize; i += nt) sum_elem<DT>(a.src, a.W, i, a.out);
    for (uint64_t i = cut.hi / Elem<DT>::kSize + tid; i < a.count; i += nt) sum_elem<DT>(a.src, a.W, i, a.out);
    const uint64_t step = 16 * uint64_t(nt);
    for (uint64_t t0 = cut.lo; t0 < cut.hi; t0 += step) {
        const OutWindow<kSumStoreAux> w(o + t0, window_bytes(t0, cut.hi, step));
        const uint64_t off = t0 + 16 * uint64_t(tid);
        if (off < cut.hi) w.st16(16 * tid, sum_vec<DT, NTL>(a.src, a.W, off));
    }
}

template <typename K>
const void *kfn(K *k) { return reinterpret_cast<const void *>(k); }

template <int DT>
const void *reduce_kernel(bool single, bool ntl, bool sh, uint32_t g) {
    if (single) return ntl ? kfn(&rog_reduce_single_kernel<DT, true>) : kfn(&rog_reduce_single_kernel<DT, false>);
    if (sh && ntl)
        return g == 2 ? kfn(&rog_reduce_kernel<DT, true, true, 2>)
             : g == 4 ? kfn(&rog_reduce_kernel<DT, true, true, 4>) : kfn(&rog_reduce_kernel<DT, true, true, 8>);
    if (sh) return kfn(&rog_reduce_kernel<DT, false, true, kGroup>);
    return ntl ? kfn(&rog_reduce_kernel<DT, true, false, kGroup>) : kfn(&rog_reduce_kernel<DT, false, false, kGroup>);
}

rog_status launch_reduce(Plan &p, hipStream_t stream) {
    const rog_plan_info &i = p.info;
    if (i.kernel == ROG_KERNEL_NONE) return ROG_OK;
    const bool single = i.path == ROG_PATH_SINGLE_WG;
    const bool ntl = (i.flags & ROG_PLAN_NT_LOADS) != 0;
    const bool sh = (i.flags & ROG_PLAN_SHIFTED_LOADS) != 0;
    const uint32_t g = sum_granule_group(p.reduce.W);
    const void *k = p.dtype == ROG_DTYPE_BF16  ? reduce_kernel<ROG_DTYPE_BF16>(single, ntl, sh, g)
                    : p.dtype == ROG_DTYPE_F16 ? reduce_kernel<ROG_DTYPE_F16>(single, ntl, sh, g)
                                               : reduce_kernel<ROG_DTYPE_F32>(single, ntl, sh, g);
    void *params[] = {&p.reduce};
    const hipError_t e = hipLaunchKernel(k, dim3(i.grid), dim3(i.block), params, 0, stream);
    if (e != hipSuccess) {
        g_last_hip_error = int(e);
        return ROG_ERR_LAUNCH;
    }
    return ROG_OK;
}

template <int DT>
const void *reduce_batch_kernel(bool ntl, bool sh, uint32_t g) {
    if (sh && ntl)
        return g == 2 ? kfn(&rog_reduce_batch_kernel<DT, true, true, 2>)
             : g == 4 ? kfn(&rog_reduce_batch_kernel<DT, true, true, 4>) : kfn(&rog_reduce_batch_kernel<DT, true, true, 8>);
    if (sh) return kfn(&rog_reduce_batch_kernel<DT, false, true, kGroup>);
    return ntl ? kfn(&rog_reduce_batch_kernel<DT, true, false, kGroup>) : kfn(&rog_reduce_batch_kernel<DT, false, false, kGroup>);
}

}  // namespace
}  // namespace rog

// ---------------------------------------------------------------------------
// C ABI (include/rog.h)
// ---------------------------------------------------------------------------
extern "C" {

ROG_API rog_status rog_reduce_ex(const void *const *srcs, int W, size_t count, rog_dtype dtype, void *out,
                                 hipStream_t stream, rog_path path) {
    rog::Plan p;
    const rog_status st = rog::plan_reduce(srcs, W, count, dtype, out, path, &p);
    if (st != ROG_OK) return st;
    return rog::launch_reduce(p, stream);
}

ROG_API rog_status rog_reduce(const void *const *srcs, int W, size_t count, rog_dtype dtype, void *out,
                              hipStream_t stream) {
    return rog_reduce_ex(srcs, W, count, dtype, out, stream, ROG_PATH_AUTO);
}

ROG_API rog_status rog_reduce_plan(const void *const *srcs, int W, size_t count, rog_dtype dtype,
                                   const void *out, rog_path path, rog_plan_info *info) {
    if (!info) return ROG_ERR_INVALID_ARGUMENT;
    rog::Plan p;
    const rog_status st = rog::plan_reduce(srcs, W, count, dtype, out, path, &p);
    if (st == ROG_OK) *info = p.info;
    return st;
}

ROG_API size_t rog_reduce_single_wg_max_bytes(void) { return rog::kReduceSingleWgMaxBytes; }

ROG_API rog_status rog_reduce_many(const rog_reduce_desc *descs, int n, int W, rog_dtype dtype,
                                   hipStream_t stream) {
    rog::ReduceBatchArgs args;
    uint32_t grid = 0;
    bool ntl = false, sh = false;
    const rog_status st = rog::plan_reduce_batch(descs, n, W, dtype, &args, &grid, &ntl, &sh);
    if (st != ROG_OK || grid == 0) return st;
    const uint32_t g = rog::sum_granule_group(uint32_t(W));
    const void *k = dtype == ROG_DTYPE_BF16  ? rog::reduce_batch_kernel<ROG_DTYPE_BF16>(ntl, sh, g)
                    : dtype == ROG_DTYPE_F16 ? rog::reduce_batch_kernel<ROG_DTYPE_F16>(ntl, sh, g)
                                             : rog::reduce_batch_kernel<ROG_DTYPE_F32>(ntl, sh, g);
    void *params[] = {&args};
    const hipError_t e = hipLaunchKernel(k, dim3(grid), dim3(rog::kWaveBlock), params, 0, stream);
    if (e != hipSuccess) {
        rog::g_last_hip_error = int(e);
        return ROG_ERR_LAUNCH;
    }
    return ROG_OK;
}

}  // extern "C"
