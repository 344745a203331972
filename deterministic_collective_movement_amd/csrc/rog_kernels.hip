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
//    (no division on the device at all); in a chunk that crosses a payload
//    boundary each lane finds its own payload with the same multiply-high.
//  * PEER kernel (anything else): each payload on its own -- a byte head up to
//    a 256-byte boundary of its destination, a body of aligned 16-byte stores,
//    a byte tail.  Every body store takes the 16 source bytes at the same
//    payload offset, whatever byte alignment the source has.  At a multiple of
//    4 bytes that is one unaligned global_load_dwordx4 (gfx950 global loads
//    run in unaligned-access mode under the HSA runtime), and so it is with
//    cached loads at any alignment.  Where the loads stream past the caches
//    and the source sits an odd or 2-mod-4 number of bytes past a 16-byte
//    granule, the multi-WG lanes load aligned granules instead and rebuild
//    their bytes from their own granule and the next lane's (a lane shuffle
//    and v_alignbyte), which streams faster than split unaligned loads.  The pages' fallback copies
//    such payloads byte by byte ("vectors where aligned, byte-wise tail"); the
//    bytes written are the same.  Multi-WG, the body is cut into 1 KiB chunks,
//    one wave per chunk, all payloads at once; single-WG, the one workgroup
//    takes the payloads in turn.
//  * BATCH kernel (rog_gather_many): one launch; every wave finds its tensor by
//    a scalar binary search over the tensors' first chunks and does one FLAT
//    or PEER chunk of that tensor.
//
// Everything a launch needs is in its kernel arguments; there are no scratch
// buffers, atomics or inter-workgroup synchronisation, and every output byte
// has exactly one writer.
#include <hip/hip_runtime.h>

#include "rog_device.h"

namespace rog {

// ---------------------------------------------------------------------------
// FLAT: vectors [0, n_vec) of one gather.  Vector v comes from payload
// r = v / vpr at index v - r*vpr.  Chunk c is vectors [64*U*c, 64*U*(c + 1)).
// ---------------------------------------------------------------------------
template <int U, bool NTL>
__device__ __forceinline__ void flat_chunk(const void *const *src, vec16 *o, uint32_t n_vec,
                                           uint32_t vpr, const Divider &div, uint32_t c) {
    constexpr uint32_t kChunk = 64 * U;
    const uint32_t lane = __lane_id();
    // n_vec < 2^32 and b is a multiple of kChunk below n_vec, so no expression
    // below wraps (b + kChunk - 1 <= 2^32 - 1; seg_lo + vpr <= n_vec).
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
        // small): each lane finds its own payload with the same multiply-high
        // and reads that payload's base pointer itself, so all lanes proceed at
        // once whatever the number of payloads in the chunk.
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

// FLAT by workgroups `block` of `nblocks`, each of `waves` waves: a wave owns
// chunks wave_id, wave_id + stride, ... (grid-stride over a capped grid).
template <int U, bool NTL>
__device__ __forceinline__ void flat_copy(const void *const *src, void *out, uint32_t n_vec,
                                          uint32_t vpr, const Divider &div, uint32_t block,
                                          uint32_t nblocks, uint32_t waves) {
    constexpr uint32_t kChunk = 64 * U;
    const uint32_t wave = uniform(threadIdx.x / 64);
    const uint32_t n_chunks = n_vec / kChunk + (n_vec % kChunk != 0);
    const uint32_t stride = nblocks * waves;
    vec16 *o = static_cast<vec16 *>(out);
    for (uint32_t c = block * waves + wave; c < n_chunks; c += stride)
        flat_chunk<U, NTL>(src, o, n_vec, vpr, div, c);
}

// ---------------------------------------------------------------------------
// PEER: one payload of S bytes from s to d, cut by split_payload into a byte
// head [0, lo), a body [lo, hi) of aligned 16-byte stores -- each fed by the
// 16 source bytes at the same payload offset, read inside [s, s + S) or, in
// the shuffled form, inside the 16-byte granules that hold those bytes -- and
// a byte tail [hi, S).  Every output byte is written exactly once.
// ---------------------------------------------------------------------------

// One wave: body chunk j (body vectors [64j, 64j + 64)); chunk 0 also moves the
// head and tail bytes (at most kBodyAlign - 1 and 15 of them).
//
// Body source bytes sit m = (s + lo) % 16 bytes past a 16-byte granule, the
// same m for every lane.  Unless the loads stream past the caches (NTL) and
// kPeerShift takes this m, each lane reads its 16 bytes with one unaligned
// load.  Otherwise (the shuffled form) each lane loads the aligned granule g
// holding its first byte; the granule after g is the next lane's g, passed
// across by a lane shuffle, and only the last lane of the wave or of the body
// loads it itself (a cached load: that granule is the next chunk's first).
// Every granule read holds at least one byte of the payload, so it lies in
// the payload's pages.
template <bool NTL>
__device__ __forceinline__ void peer_chunk(const uint8_t *s, uint8_t *d, uint64_t S, uint32_t j) {
    const uint32_t lane = __lane_id();
    const PeerSplit cut = split_payload(reinterpret_cast<uintptr_t>(d), S);
    if (j == 0) {
        for (uint64_t i = lane; i < cut.lo; i += 64) d[i] = s[i];
        for (uint64_t i = cut.hi + lane; i < S; i += 64) d[i] = s[i];
    }
    const uint64_t off = cut.lo + 16 * (uint64_t(j) * 64 + lane);
    const bool live = off < cut.hi;
    const uint32_t m = uniform(uint32_t(reinterpret_cast<uintptr_t>(s + cut.lo)) & 15);
    if (!NTL || !shift_granules(m, kPeerShift)) {
        if (live) st16(reinterpret_cast<vec16 *>(d + off), ldu16<NTL>(s + off));
        return;
    }
    const vec16 *g = reinterpret_cast<const vec16 *>(s + off - m);
    // The granule after the body's end is read only if it holds payload bytes
    // (m != 0); the last lane of a wave inside the body always may.
    const bool own_hi = live && (lane == 63 || off + 16 >= cut.hi) && (m != 0 || off + 16 < cut.hi);
    vec16 lo = vec16{0, 0, 0, 0}, hi = lo;
    if (live) lo = ld16<NTL>(g);
    if (own_hi) hi = ld16<false>(g + 1);  // cached; in flight beside lo
    // Lane l + 1's granule; all 64 lanes take part in the shuffle.
    const vec16 next = vec16{__shfl_down(lo.x, 1u), __shfl_down(lo.y, 1u), __shfl_down(lo.z, 1u),
                             __shfl_down(lo.w, 1u)};
    if (live) st16(reinterpret_cast<vec16 *>(d + off), cut16(lo, own_hi ? hi : next, m));
}

// One workgroup of nt threads, the whole payload: head and tail bytes, then the
// body in tiles of nt * U vectors (U loads in flight per thread).
template <int U, bool NTL>
__device__ __forceinline__ void peer_whole(const uint8_t *s, uint8_t *d, uint64_t S, uint32_t nt) {
    const uint32_t tid = threadIdx.x;
    const PeerSplit cut = split_payload(reinterpret_cast<uintptr_t>(d), S);
    for (uint64_t i = tid; i < cut.lo; i += nt) d[i] = s[i];
    for (uint64_t i = cut.hi + tid; i < S; i += nt) d[i] = s[i];
    const uint8_t *sb = s + cut.lo;
    vec16 *db = reinterpret_cast<vec16 *>(d + cut.lo);
    const uint64_t count = (cut.hi - cut.lo) >> 4;
    const uint64_t tile = uint64_t(nt) * U;
    for (uint64_t base = 0; base < count; base += tile) {
        if (base + tile <= count) {
            vec16 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = ldu16<NTL>(sb + 16 * (base + u * nt + tid));
#pragma unroll
            for (int u = 0; u < U; ++u) st16(db + base + u * nt + tid, v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t k = base + u * nt + tid;
                if (k < count) st16(db + k, ldu16<NTL>(sb + 16 * k));
            }
        }
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

// Single-WG FLAT: one workgroup of as many waves as there are chunks (<= 16),
// U = single_flat_unroll(n_vec) vectors per lane.
template <int U, bool NTL>
__global__ __launch_bounds__(kSingleBlock) void rog_flat_single_kernel(FlatArgs a) {
    flat_copy<U, NTL>(a.src, a.out, a.n_vec, a.vpr, a.div, 0, 1, blockDim.x / 64);
}

// Multi-WG PEER: one wave per workgroup and per body chunk, chunks grouped by
// XCD, grid-strided over the n_chunks = W * chunks_per_peer chunks.
template <bool NTL>
__global__ __launch_bounds__(kWaveBlock) void rog_peer_kernel(PeerArgs a) {
    for (uint32_t vb = blockIdx.x; vb < a.n_chunks; vb += gridDim.x) {
        const uint32_t b = xcd_grouped(vb, a.n_chunks);
        const uint32_t r = divide(b, a.cdiv);
        peer_chunk<NTL>(static_cast<const uint8_t *>(a.src[r]), static_cast<uint8_t *>(a.out) + uint64_t(r) * a.S,
                        a.S, b - r * a.chunks_per_peer);
    }
}

// Single-WG PEER: one workgroup takes the payloads in turn.  Its block size is
// known only at run time, so its unroll is smaller (register budget of a
// 1024-thread workgroup: 128 VGPRs per lane).
template <bool NTL>
__global__ __launch_bounds__(kSingleBlock) void rog_peer_single_kernel(PeerArgs a) {
    for (uint32_t r = 0; r < a.W; ++r)
        peer_whole<kSinglePeerUnroll, NTL>(static_cast<const uint8_t *>(a.src[r]),
                                           static_cast<uint8_t *>(a.out) + uint64_t(r) * a.S, a.S, blockDim.x);
}

// BATCH: one wave per workgroup and per chunk of some tensor.  The FLAT
// tensors' chunks come first and go to the XCDs round-robin, as in the FLAT
// kernel; the PEER tensors' chunks follow, handed out in XCD runs as in the
// PEER kernel.  (Runs over the FLAT chunks too measured 5 % slower on an
// aligned batch; no runs at all, 9 % slower on 8 x 64 MiB PEER payloads.)
template <bool NTL>
__global__ __launch_bounds__(kWaveBlock) void rog_batch_kernel(BatchArgs a) {
    for (uint32_t vb = blockIdx.x; vb < a.n_chunks; vb += gridDim.x) {
        const uint32_t c = vb < a.flat_chunks
                               ? vb
                               : a.flat_chunks + xcd_grouped(vb - a.flat_chunks, a.n_chunks - a.flat_chunks);
        const uint32_t lo = batch_tensor(a.first, a.n, c);
        const BatchTensor &t = a.t[lo];
        const uint32_t lc = c - a.first[lo];
        const void *const *src = a.src + lo * a.W;
        if (t.flat) {
            flat_chunk<kFlatUnroll, NTL>(src, reinterpret_cast<vec16 *>(t.out), t.n_vec, t.vpr, t.div, lc);
        } else {
            const uint32_t r = divide(lc, t.div);
            peer_chunk<NTL>(static_cast<const uint8_t *>(src[r]), reinterpret_cast<uint8_t *>(t.out) + uint64_t(r) * t.S,
                            t.S, lc - r * t.chunks_per_peer);
        }
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
thread_local int g_last_hip_error = 0;

namespace {

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
        if (single && single_flat_unroll(p.flat.n_vec) == 1)
            k = ntl ? kfn(&rog_flat_single_kernel<1, true>) : kfn(&rog_flat_single_kernel<1, false>);
        else if (single)
            k = ntl ? kfn(&rog_flat_single_kernel<kSingleUnroll, true>) : kfn(&rog_flat_single_kernel<kSingleUnroll, false>);
        else        k = ntl ? kfn(&rog_flat_kernel<kFlatBlock, true>) : kfn(&rog_flat_kernel<kFlatBlock, false>);
        return launch(k, i.grid, i.block, p.flat, stream);
    case ROG_KERNEL_PEER:
        if (single) k = ntl ? kfn(&rog_peer_single_kernel<true>) : kfn(&rog_peer_single_kernel<false>);
        else        k = ntl ? kfn(&rog_peer_kernel<true>) : kfn(&rog_peer_kernel<false>);
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
    return rog::launch(k, grid, rog::kWaveBlock, args, stream);
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
