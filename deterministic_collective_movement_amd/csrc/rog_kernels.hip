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
//  * PEER kernel (anything else): each payload on its own -- a byte head, a
//    body of aligned 16-byte stores and a byte tail; the body loads aligned
//    source vectors, funnel-shifted when source and destination are misaligned
//    differently (the pages' fallback copies such payloads byte by byte; the
//    bytes written are the same).  Multi-WG, the grid is split into W groups of
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

// 16-byte loads: non-temporal (streamed past the caches) when NT, else cached.
template <bool NT>
__device__ __forceinline__ vec16 ld16(const vec16 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
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

// ---------------------------------------------------------------------------
// FLAT: vectors [0, n_vec) of one gather, by workgroups `block` of `nblocks`,
// each of `waves` waves.  Vector v comes from payload r = v / vpr at index
// v - r*vpr.  A wave owns chunks of 64*U consecutive vectors, grid-strided.
// ---------------------------------------------------------------------------
template <int U, bool NTL>
__device__ __forceinline__ void flat_copy(const void *const *src, void *out, uint32_t n_vec,
                                          uint32_t vpr, const Divider &div, uint32_t block,
                                          uint32_t nblocks, uint32_t waves) {
    constexpr uint32_t kChunk = 64 * U;
    const uint32_t lane = __lane_id();
    const uint32_t wave = uniform(threadIdx.x / 64);
    // n_vec < 2^32 and b is a multiple of kChunk below n_vec, so no expression
    // below wraps (b + kChunk - 1 <= 2^32 - 1; seg_lo + vpr <= n_vec).
    const uint32_t n_chunks = n_vec / kChunk + (n_vec % kChunk != 0);
    const uint32_t stride = nblocks * waves;
    vec16 *o = static_cast<vec16 *>(out);

    for (uint32_t c = block * waves + wave; c < n_chunks; c += stride) {
        const uint32_t b = c * kChunk;                  // first vector of the chunk
        const uint32_t n = min(n_vec - b, kChunk);      // vectors in the chunk
        const uint32_t e = b + n;                       // chunk end
        const uint32_t r = divide(b, div);              // payload of b (scalar)
        const uint32_t seg_lo = r * vpr;
        if (e <= seg_lo + vpr) {
            // The whole chunk lies in payload r: scalar bases, lane offsets.
            const vec16 *s = static_cast<const vec16 *>(src[r]) + (b - seg_lo);
            vec16 *d = o + b;
            if (n == kChunk) {
                vec16 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) v[u] = ld16<NTL>(s + u * 64 + lane);
#pragma unroll
                for (int u = 0; u < U; ++u) st16(d + u * 64 + lane, v[u]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t k = u * 64 + lane;
                    if (k < n) st16(d + k, ld16<NTL>(s + k));
                }
            }
        } else {
            // The chunk crosses payload boundaries (rare unless payloads are
            // small): each lane finds its own payload with the same multiply-
            // high and reads that payload's base pointer itself, so all lanes
            // proceed at once whatever the number of payloads in the chunk.
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t k = b + u * 64 + lane;
                if (k < e) {
                    const uint32_t rk = divide(k, div);
                    const vec16 *s = static_cast<const vec16 *>(src[rk]);
                    st16(o + k, ld16<NTL>(s + (k - rk * vpr)));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// PEER: one payload of S bytes from sp to dp by a workgroup of BLOCK threads
// (BLOCK >= 64); this workgroup takes tiles part, part + parts, ...  Tiles are
// BLOCK*U 16-byte output vectors; within a tile thread t handles vectors t,
// t + BLOCK, ... (coalesced).  Tile bases are wave-uniform (scalar registers);
// lanes add 32-bit offsets.
// ---------------------------------------------------------------------------

// Bytes [lo, hi) of a payload, one byte per thread per step (heads and tails).
__device__ __forceinline__ void copy_bytes(const uint8_t *s, uint8_t *d, uint64_t lo, uint64_t hi,
                                           uint32_t BLOCK) {
    for (uint64_t i = lo + threadIdx.x; i < hi; i += BLOCK) d[i] = s[i];
}

// count aligned 16-byte vectors from s to d.
template <int U, bool NTL>
__device__ __forceinline__ void vec_body(const vec16 *s0, vec16 *d0, uint64_t count, uint32_t part,
                                         uint32_t parts, uint32_t BLOCK) {
    const uint32_t tid = threadIdx.x;
    const uint32_t kTile = BLOCK * U;
    for (uint64_t base = uint64_t(part) * kTile; base < count; base += uint64_t(parts) * kTile) {
        const vec16 *s = s0 + base;
        vec16 *d = d0 + base;
        if (base + kTile <= count) {
            vec16 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = ld16<NTL>(s + (u * BLOCK + tid));
#pragma unroll
            for (int u = 0; u < U; ++u) st16(d + (u * BLOCK + tid), v[u]);
        } else {
            const uint32_t n = uint32_t(count - base);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t k = u * BLOCK + tid;
                if (k < n) st16(d + k, ld16<NTL>(s + k));
            }
        }
    }
}

// The 16 bytes that start 4*Q + sh bytes into the 32 bytes a:b (little-endian
// byte order, a first): each output dword joins two neighbouring input dwords
// with one v_alignbyte_b32.
template <int Q>
__device__ __forceinline__ vec16 funnel(const vec16 &a, const vec16 &b, uint32_t sh) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    vec16 r;
    r.x = __builtin_amdgcn_alignbyte(w[Q + 1], w[Q + 0], sh);
    r.y = __builtin_amdgcn_alignbyte(w[Q + 2], w[Q + 1], sh);
    r.z = __builtin_amdgcn_alignbyte(w[Q + 3], w[Q + 2], sh);
    r.w = __builtin_amdgcn_alignbyte(w[Q + 4], w[Q + 3], sh);
    return r;
}

// count aligned 16-byte output vectors d[k], each the 16 bytes that start
// delta = 4*Q + sh bytes into the aligned source vectors p[k], p[k+1].  Both
// loads are cached: lane t's p[k+1] is lane t+1's p[k], fetched by the same
// wave an instruction earlier, so the second load is served by the cache.
// (Measured faster than streaming loads, and than passing the neighbour's
// block across lanes with a DPP wavefront shift.)
template <int U, int Q>
__device__ __forceinline__ void shift_body(const vec16 *p0, vec16 *d0, uint64_t count, uint32_t sh,
                                           uint32_t part, uint32_t parts, uint32_t BLOCK) {
    const uint32_t tid = threadIdx.x;
    const uint32_t kTile = BLOCK * U;
    for (uint64_t base = uint64_t(part) * kTile; base < count; base += uint64_t(parts) * kTile) {
        const vec16 *p = p0 + base;
        vec16 *d = d0 + base;
        if (base + kTile <= count) {
            vec16 a[U], b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                a[u] = ld16<false>(p + (u * BLOCK + tid));
                b[u] = ld16<false>(p + (u * BLOCK + tid + 1));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) st16(d + (u * BLOCK + tid), funnel<Q>(a[u], b[u], sh));
        } else {
            const uint32_t n = uint32_t(count - base);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t k = u * BLOCK + tid;
                if (k < n) st16(d + k, funnel<Q>(ld16<false>(p + k), ld16<false>(p + k + 1), sh));
            }
        }
    }
}

// One payload.  The destination is cut at 256-byte boundaries (split_payload):
// a byte head, a body of aligned 16-byte stores, a byte tail.  The body's data
// comes from aligned source vectors -- one per output vector when source and
// destination are equally misaligned (in particular both 16-byte aligned),
// else two neighbours funnel-shifted.  Body vectors whose aligned source
// vectors would reach outside the payload go to the head or tail, so every
// read stays inside [sp, sp + S).  Every output byte is written exactly once.
template <int U, bool NTL>
__device__ __forceinline__ void peer_copy(const void *sp, void *dp, uint64_t S, uint32_t part,
                                          uint32_t parts, uint32_t BLOCK) {
    const uint8_t *s = static_cast<const uint8_t *>(sp);
    uint8_t *d = static_cast<uint8_t *>(dp);
    const PeerSplit cut = split_payload(reinterpret_cast<uintptr_t>(s), reinterpret_cast<uintptr_t>(d), S);
    const uint64_t lo = cut.lo, hi = cut.hi;
    const uint32_t delta = cut.delta;
    if (part == 0) {
        copy_bytes(s, d, 0, lo, BLOCK);
        copy_bytes(s, d, hi, S, BLOCK);
    }
    if (hi == lo) return;
    vec16 *D = reinterpret_cast<vec16 *>(d + lo);
    const uint64_t count = (hi - lo) >> 4;
    if (delta == 0) {
        vec_body<U, NTL>(reinterpret_cast<const vec16 *>(s + lo), D, count, part, parts, BLOCK);
        return;
    }
    const vec16 *P = reinterpret_cast<const vec16 *>(s + lo - delta);
    const uint32_t sh = delta & 3;
    switch (delta >> 2) {
    case 0: shift_body<U, 0>(P, D, count, sh, part, parts, BLOCK); break;
    case 1: shift_body<U, 1>(P, D, count, sh, part, parts, BLOCK); break;
    case 2: shift_body<U, 2>(P, D, count, sh, part, parts, BLOCK); break;
    default: shift_body<U, 3>(P, D, count, sh, part, parts, BLOCK); break;
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
// Multi-WG FLAT: workgroups of BLOCK threads over the whole output.
template <int BLOCK, bool NTL>
__global__ __launch_bounds__(BLOCK) void rog_flat_kernel(FlatArgs a) {
    flat_copy<kFlatUnroll, NTL>(a.src, a.out, a.n_vec, a.vpr, a.div, blockIdx.x, gridDim.x, BLOCK / 64);
}

// Single-WG FLAT: one workgroup of as many waves as there are chunks (<= 16).
template <bool NTL>
__global__ __launch_bounds__(kSingleBlock) void rog_flat_single_kernel(FlatArgs a) {
    flat_copy<kSingleUnroll, NTL>(a.src, a.out, a.n_vec, a.vpr, a.div, 0, 1, blockDim.x / 64);
}

// Multi-WG PEER: W groups of blocks_per_peer workgroups, one group per payload.
template <int BLOCK, bool NTL>
__global__ __launch_bounds__(BLOCK) void rog_peer_kernel(PeerArgs a) {
    const uint32_t r = blockIdx.x / a.blocks_per_peer;
    const uint32_t part = blockIdx.x - r * a.blocks_per_peer;
    peer_copy<kPeerUnroll, NTL>(a.src[r], static_cast<uint8_t *>(a.out) + uint64_t(r) * a.S, a.S, part,
                                a.blocks_per_peer, BLOCK);
}

// Single-WG PEER: one workgroup takes the payloads in turn.  Its block size is
// known only at run time, so its unroll is smaller (register budget of a
// 1024-thread workgroup: 128 VGPRs per lane).
template <bool NTL>
__global__ __launch_bounds__(kSingleBlock) void rog_peer_single_kernel(PeerArgs a) {
    for (uint32_t r = 0; r < a.W; ++r)
        peer_copy<kSinglePeerUnroll, NTL>(a.src[r], static_cast<uint8_t *>(a.out) + uint64_t(r) * a.S, a.S,
                                          0, 1, blockDim.x);
}

template <bool NTL>
__global__ __launch_bounds__(kBatchBlock) void rog_batch_kernel(BatchArgs a) {
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
        flat_copy<kFlatUnroll, NTL>(src, reinterpret_cast<void *>(t.out), t.n_vec, t.vpr, t.div, lb,
                                    t.n_blocks, kBatchBlock / 64);
    } else {
        const uint32_t r = lb / t.blocks_per_peer;
        const uint32_t part = lb - r * t.blocks_per_peer;
        peer_copy<kBatchPeerUnroll, NTL>(src[r], reinterpret_cast<uint8_t *>(t.out) + uint64_t(r) * t.S, t.S,
                                         part, t.blocks_per_peer, kBatchBlock);
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

template <typename K>
const void *kfn(K *k) { return reinterpret_cast<const void *>(k); }

rog_status launch_plan(Plan &p, hipStream_t stream) {
    const rog_plan_info &i = p.info;
    const bool single = i.path == ROG_PATH_SINGLE_WG;
    const bool ntl = (i.flags & ROG_PLAN_NT_LOADS) != 0;
    const void *k = nullptr;
    switch (i.kernel) {
    case ROG_KERNEL_NONE:
        return ROG_OK;
    case ROG_KERNEL_FLAT:
        if (single) k = ntl ? kfn(&rog_flat_single_kernel<true>) : kfn(&rog_flat_single_kernel<false>);
        else        k = ntl ? kfn(&rog_flat_kernel<kFlatBlock, true>) : kfn(&rog_flat_kernel<kFlatBlock, false>);
        return launch(k, i.grid, i.block, p.flat, stream);
    case ROG_KERNEL_PEER:
        if (single) k = ntl ? kfn(&rog_peer_single_kernel<true>) : kfn(&rog_peer_single_kernel<false>);
        else        k = ntl ? kfn(&rog_peer_kernel<kPeerBlock, true>) : kfn(&rog_peer_kernel<kPeerBlock, false>);
        return launch(k, i.grid, i.block, p.peer, stream);
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
    bool ntl = false;
    const rog_status st = rog::plan_batch(descs, n, W, &args, &grid, &ntl);
    if (st != ROG_OK || grid == 0) return st;
    const void *k = ntl ? rog::kfn(&rog::rog_batch_kernel<true>) : rog::kfn(&rog::rog_batch_kernel<false>);
    return rog::launch(k, grid, rog::kBatchBlock, args, stream);
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
