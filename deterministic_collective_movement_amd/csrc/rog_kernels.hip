// rog_kernels.hip -- HIP kernels of the rank-ordered gather for gfx950 (CDNA4)
// and the C entry points that launch them.
//
// The copy is the one RL-Align/RL-Kernel PR #491 ("perf(cuda): vectorize the
// deterministic all-gather copy and right-size its single-block path") builds
// its three all-gather kernels on (section "What", copy_rank_ordered bullet):
// out[r*S + i] = src_r[i].  The pages' fix replaced a loop that moved one byte
// per thread and divided by the payload size for every byte.  Here:
//
//  * FLAT kernel (output, S and every payload 16-byte aligned): one flat loop
//    over all W*S/16 vectors of the output, so every wave stays busy across
//    payload boundaries.  A 64-lane wave owns a chunk of 64*U consecutive
//    vectors; each of its U loads and U stores is one dwordx4 instruction over
//    64 consecutive vectors (1 KiB, fully coalesced).  The payload of a chunk
//    is found once per chunk, in scalar registers, by one 32-bit multiply-high
//    (no division on the device at all); a chunk that crosses a payload
//    boundary walks the few payloads it touches with per-lane range masks.
//  * PEER kernel (anything else): each payload on its own, 16-byte vectors plus
//    a byte tail where its source and destination are both 16-byte aligned,
//    byte by byte otherwise.  Multi-WG, the grid is split into W groups of
//    workgroups, one group per payload, so all payloads are copied at once;
//    single-WG, the one workgroup takes the payloads in turn.
//  * BATCH kernel (rog_gather_many): one launch; each workgroup finds its
//    tensor by a scalar binary search over the tensors' first workgroups and
//    runs the FLAT or PEER work of that tensor.
//
// Everything a launch needs is in its kernel arguments; there are no scratch
// buffers, atomics or inter-workgroup synchronisation, and every output byte
// has exactly one writer.
#include <hip/hip_runtime.h>

#include "rog_internal.h"

namespace rog {

typedef uint32_t vec16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ vec16 ld16(const vec16 *p) {
    if constexpr (kNonTemporal) return __builtin_nontemporal_load(p);
    else return *p;
}

__device__ __forceinline__ void st16(vec16 *p, vec16 v) {
    if constexpr (kNonTemporal) __builtin_nontemporal_store(v, p);
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

// ---------------------------------------------------------------------------
// FLAT: vectors [0, n_vec) of one gather, by workgroups `block` of `nblocks`.
// Vector v comes from payload r = v / vpr at index v - r*vpr.
// ---------------------------------------------------------------------------
template <int BLOCK>
__device__ __forceinline__ void flat_copy(const void *const *src, void *out, uint32_t n_vec,
                                          uint32_t vpr, const Divider &div, uint32_t block,
                                          uint32_t nblocks) {
    constexpr uint32_t kWaves = BLOCK / 64;
    const uint32_t lane = __lane_id();
    const uint32_t wave = uniform(threadIdx.x / 64);
    // n_vec < 2^32; no expression below wraps: b + kChunkVecs - 1 <= 2^32 - 1
    // because b is a multiple of kChunkVecs below n_vec.
    const uint32_t n_chunks = n_vec / kChunkVecs + (n_vec % kChunkVecs != 0);
    const uint32_t stride = nblocks * kWaves;
    vec16 *o = static_cast<vec16 *>(out);

    for (uint32_t c = block * kWaves + wave; c < n_chunks; c += stride) {
        const uint32_t b = c * kChunkVecs;              // first vector of the chunk
        const uint32_t n = min(n_vec - b, kChunkVecs);  // vectors in the chunk
        const uint32_t e = b + n;                       // chunk end
        const uint32_t r = divide(b, div);              // payload of b (scalar)
        const uint32_t seg_lo = r * vpr;
        if (e <= seg_lo + vpr) {
            // The whole chunk lies in payload r: scalar bases, lane offsets.
            const vec16 *s = static_cast<const vec16 *>(src[r]) + (b - seg_lo);
            vec16 *d = o + b;
            if (n == kChunkVecs) {
                vec16 v[kVecUnroll];
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) v[u] = ld16(s + u * 64 + lane);
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) st16(d + u * 64 + lane, v[u]);
            } else {
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) {
                    const uint32_t k = u * 64 + lane;
                    if (k < n) st16(d + k, ld16(s + k));
                }
            }
        } else {
            // The chunk crosses payload boundaries: visit each payload it
            // touches (uniform loop, at most W turns); lanes copy the vectors
            // that fall in the current payload's range.
            for (uint32_t rr = r, lo = seg_lo; lo < e; ++rr, lo += vpr) {
                const vec16 *s = static_cast<const vec16 *>(src[rr]);
                const uint32_t hi = lo + vpr;
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) {
                    const uint32_t k = b + u * 64 + lane;
                    if (k >= lo && k < hi && k < e) st16(o + k, ld16(s + (k - lo)));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// PEER: one payload of S bytes from s to d, tiles part, part+parts, ...
// ---------------------------------------------------------------------------
template <int BLOCK>
__device__ __forceinline__ void peer_copy(const void *sp, void *dp, uint64_t S, bool vec,
                                          uint32_t part, uint32_t parts) {
    const uint32_t tid = threadIdx.x;
    if (vec) {
        // 16-byte vectors, then the S % 16 tail bytes (by tile 0's workgroup).
        const vec16 *s = static_cast<const vec16 *>(sp);
        vec16 *d = static_cast<vec16 *>(dp);
        const uint64_t nv = S >> 4;
        constexpr uint32_t kTile = BLOCK * kVecUnroll;
        for (uint64_t base = uint64_t(part) * kTile; base < nv; base += uint64_t(parts) * kTile) {
            if (base + kTile <= nv) {
                vec16 v[kVecUnroll];
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) v[u] = ld16(s + base + u * BLOCK + tid);
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) st16(d + base + u * BLOCK + tid, v[u]);
            } else {
#pragma unroll
                for (int u = 0; u < kVecUnroll; ++u) {
                    const uint64_t k = base + u * BLOCK + tid;
                    if (k < nv) st16(d + k, ld16(s + k));
                }
            }
        }
        if (part == 0) {
            const uint64_t k = (nv << 4) + tid;
            if (k < S) static_cast<uint8_t *>(dp)[k] = static_cast<const uint8_t *>(sp)[k];
        }
    } else {
        const uint8_t *s = static_cast<const uint8_t *>(sp);
        uint8_t *d = static_cast<uint8_t *>(dp);
        constexpr uint32_t kTile = BLOCK * kByteUnroll;
        for (uint64_t base = uint64_t(part) * kTile; base < S; base += uint64_t(parts) * kTile) {
            if (base + kTile <= S) {
                uint8_t v[kByteUnroll];
#pragma unroll
                for (int u = 0; u < kByteUnroll; ++u) v[u] = s[base + u * BLOCK + tid];
#pragma unroll
                for (int u = 0; u < kByteUnroll; ++u) d[base + u * BLOCK + tid] = v[u];
            } else {
#pragma unroll
                for (int u = 0; u < kByteUnroll; ++u) {
                    const uint64_t k = base + u * BLOCK + tid;
                    if (k < S) d[k] = s[k];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void rog_flat_kernel(FlatArgs a) {
    flat_copy<BLOCK>(a.src, a.out, a.n_vec, a.vpr, a.div, blockIdx.x, gridDim.x);
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void rog_peer_kernel(PeerArgs a) {
    uint8_t *out = static_cast<uint8_t *>(a.out);
    if (a.blocks_per_peer == 0) {
        for (uint32_t r = 0; r < a.W; ++r)
            peer_copy<BLOCK>(a.src[r], out + uint64_t(r) * a.S, a.S, (a.vec_ok >> r) & 1, 0, 1);
    } else {
        const uint32_t r = blockIdx.x / a.blocks_per_peer;
        const uint32_t part = blockIdx.x - r * a.blocks_per_peer;
        peer_copy<BLOCK>(a.src[r], out + uint64_t(r) * a.S, a.S, (a.vec_ok >> r) & 1, part,
                         a.blocks_per_peer);
    }
}

__global__ __launch_bounds__(kMultiBlock) void rog_batch_kernel(BatchArgs a) {
    const uint32_t b = blockIdx.x;
    // Last tensor whose first workgroup is <= b (first_block strictly increases).
    uint32_t lo = 0, hi = a.n;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (a.t[mid].first_block <= b) lo = mid;
        else hi = mid;
    }
    const BatchTensor &t = a.t[lo];
    const uint32_t lb = b - t.first_block;
    const void *const *src = a.src + lo * a.W;
    if (t.flat) {
        flat_copy<kMultiBlock>(src, reinterpret_cast<void *>(t.out), t.n_vec, t.vpr, t.div, lb,
                               t.n_blocks);
    } else {
        const uint32_t r = lb / t.blocks_per_peer;
        const uint32_t part = lb - r * t.blocks_per_peer;
        peer_copy<kMultiBlock>(src[r], reinterpret_cast<uint8_t *>(t.out) + uint64_t(r) * t.S, t.S,
                               (t.vec_ok >> r) & 1, part, t.blocks_per_peer);
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
namespace {

thread_local int g_last_hip_error = 0;

template <typename Args>
rog_status launch(const void *kernel, uint32_t grid, uint32_t block, Args &args,
                  hipStream_t stream) {
    void *params[] = {&args};
    const hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(block), params, 0, stream);
    if (e != hipSuccess) {
        g_last_hip_error = int(e);
        return ROG_ERR_LAUNCH;
    }
    return ROG_OK;
}

rog_status launch_plan(Plan &p, hipStream_t stream) {
    const rog_plan_info &i = p.info;
    const bool single = i.path == ROG_PATH_SINGLE_WG;
    switch (i.kernel) {
    case ROG_KERNEL_NONE:
        return ROG_OK;
    case ROG_KERNEL_FLAT:
        return single
            ? launch(reinterpret_cast<const void *>(&rog_flat_kernel<kSingleBlock>), i.grid, i.block, p.flat, stream)
            : launch(reinterpret_cast<const void *>(&rog_flat_kernel<kMultiBlock>), i.grid, i.block, p.flat, stream);
    case ROG_KERNEL_PEER:
        return single
            ? launch(reinterpret_cast<const void *>(&rog_peer_kernel<kSingleBlock>), i.grid, i.block, p.peer, stream)
            : launch(reinterpret_cast<const void *>(&rog_peer_kernel<kMultiBlock>), i.grid, i.block, p.peer, stream);
    default:
        return ROG_ERR_INVALID_ARGUMENT;
    }
}

}  // namespace
}  // namespace rog

// ---------------------------------------------------------------------------
// C ABI (include/rog.h)
// ---------------------------------------------------------------------------
extern "C" {

ROG_API rog_status rog_gather_ex(const void *const *srcs, int W, size_t bytes_per_rank,
                                 void *out, hipStream_t stream, rog_path path) {
    rog::Plan p;
    const rog_status st = rog::plan_gather(srcs, W, bytes_per_rank, out, path, &p);
    if (st != ROG_OK) return st;
    return rog::launch_plan(p, stream);
}

ROG_API rog_status rog_gather(const void *const *srcs, int W, size_t bytes_per_rank, void *out,
                              hipStream_t stream) {
    return rog_gather_ex(srcs, W, bytes_per_rank, out, stream, ROG_PATH_AUTO);
}

ROG_API rog_status rog_gather_many(const rog_gather_desc *descs, int n, int W,
                                   hipStream_t stream) {
    rog::BatchArgs args;
    uint32_t grid = 0;
    const rog_status st = rog::plan_batch(descs, n, W, &args, &grid);
    if (st != ROG_OK || grid == 0) return st;
    return rog::launch(reinterpret_cast<const void *>(&rog::rog_batch_kernel), grid,
                       rog::kMultiBlock, args, stream);
}

ROG_API rog_status rog_plan(const void *const *srcs, int W, size_t bytes_per_rank,
                            const void *out, rog_path path, rog_plan_info *info) {
    if (!info) return ROG_ERR_INVALID_ARGUMENT;
    rog::Plan p;
    const rog_status st = rog::plan_gather(srcs, W, bytes_per_rank, out, path, &p);
    if (st == ROG_OK) *info = p.info;
    return st;
}

ROG_API size_t rog_single_wg_max_bytes(void) { return rog::kSingleWgMaxBytes; }
ROG_API int rog_max_peers(void) { return rog::kMaxPeers; }
ROG_API int rog_max_batch(void) { return rog::kMaxBatch; }
ROG_API int rog_max_batch_pointers(void) { return rog::kMaxBatchPtrs; }
ROG_API int rog_last_hip_error(void) { return rog::g_last_hip_error; }

ROG_API const char *rog_status_string(rog_status s) {
    switch (s) {
    case ROG_OK: return "ROG_OK";
    case ROG_ERR_INVALID_ARGUMENT: return "ROG_ERR_INVALID_ARGUMENT";
    case ROG_ERR_OVERLAP: return "ROG_ERR_OVERLAP";
    case ROG_ERR_TOO_LARGE: return "ROG_ERR_TOO_LARGE";
    case ROG_ERR_LAUNCH: return "ROG_ERR_LAUNCH";
    }
    return "ROG_ERR_UNKNOWN";
}

}  // extern "C"
