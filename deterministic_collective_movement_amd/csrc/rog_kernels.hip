// rog_kernels.hip -- HIP kernels of the rank-ordered gather for gfx950 (CDNA4)
// and the C entry points that launch them.
//
// The copy is the one RL-Align/RL-Kernel PR #491 ("perf(cuda): vectorize the
// deterministic all-gather copy and right-size its single-block path") builds
// its three all-gather kernels on (section "What", copy_rank_ordered bullet):
// out[r*S + i] = src_r[i].  The pages' fix replaced a loop that moved one byte
// per thread and divided by the payload size for every byte.  Here:
//
//  * FLAT kernel (output, S and every payload 16-byte aligned): a single loop
//    over all W*S/16 vectors of the output, so every wave stays busy across
//    payload boundaries.  A 64-lane wave owns a chunk of 64*U consecutive
//    vectors; each of its U loads and U stores is one dwordx4 instruction over
//    64 consecutive vectors (1 KiB, fully coalesced).  The first chunk is cut
//    short so that the others start on the output's 128-byte lines, and off
//    the line grid chunks go to the XCDs in runs.  The payload of a chunk
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
//    and v_alignbyte), which streams faster than split unaligned loads.  The
//    pages' fallback copies such payloads byte by byte (vectors only where
//    both sides are aligned); the bytes written are the same.  Multi-WG, the
//    body is cut into 1 KiB chunks, one wave per chunk, all payloads at once;
//    single-WG, the one workgroup takes the payloads in turn.
//  * BATCH kernel (rog_gather_many): one launch; every wave finds its tensor
//    through a bucket table of the chunk index (a scalar load of two bucket
//    entries, then a search only between the tensors those name) and does one
//    FLAT or PEER chunk of that tensor.
//
// Everything a launch needs is in its kernel arguments; there are no scratch
// buffers, atomics or inter-workgroup synchronisation, and every output byte
// has exactly one writer.  16-byte stores go through OutWindow: buffer stores
// that stream and write through the XCD's L2 (nt sc1).
#include <hip/hip_runtime.h>

#include "rog_device.h"

namespace rog {

// ---------------------------------------------------------------------------
// FLAT: vectors [0, n_vec) of one gather.  Vector v comes from payload
// r = v / vpr at index v - r*vpr.  Chunk c is flat_span(c, 64*U, shift, n_vec):
// 64*U vectors, the first chunk shorter by shift so that the others start on
// the output's 128-byte lines.
// ---------------------------------------------------------------------------
template <int U, bool NTL, typename Src>
__device__ __forceinline__ void flat_chunk(const Src &src, vec16 *o, uint32_t n_vec,
                                           uint32_t vpr, const Divider &div, uint32_t shift, uint32_t c) {
    constexpr uint32_t kChunk = 64 * U;
    const uint32_t lane = __lane_id();
    // b < e = b + n <= n_vec < 2^32, and b + kChunk - 1 <= 2^32 - 1 (shift is
    // 0 unless n_vec < 2^31, else b is a multiple of kChunk), so no
    // expression below wraps (seg_lo + vpr <= n_vec).
    const ChunkSpan span = flat_span(c, kChunk, shift, n_vec);
    const uint32_t b = span.b;                      // first vector of the chunk
    const uint32_t n = span.n;                      // vectors in the chunk
    const uint32_t e = b + n;                       // chunk end
    const uint32_t r = divide(b, div);              // payload of b (scalar)
    const uint32_t seg_lo = r * vpr;
    const OutWindow<kStoreAux> w(o + b, n * 16);    // the chunk's output
    if (e <= seg_lo + vpr) {
        // The whole chunk lies in payload r: scalar bases, lane offsets.
        gvec16 *s = (gvec16 *)src_of(src, r) + (b - seg_lo);
        if (n == kChunk) {
            vec16 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = ld16<NTL>(s + u * 64 + lane);
#pragma unroll
            for (int u = 0; u < U; ++u) w.st16(16 * (u * 64 + lane), v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t k = u * 64 + lane;
                if (k < n) w.st16(16 * k, ld16<NTL>(s + k));
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
                gvec16 *s = (gvec16 *)lane_src(src, rk);
                w.st16(16 * (k - b), ld16<NTL>(s + (k - rk * vpr)));
            }
        }
    }
}

// FLAT by one workgroup of `waves` waves: wave w owns chunks w, w + waves, ...
template <int U, bool NTL>
__device__ __forceinline__ void flat_copy(const FlatArgs &a, uint32_t waves) {
    constexpr uint32_t kChunk = 64 * U;
    const uint32_t wave = uniform(threadIdx.x / 64);
    const uint32_t n_chunks = flat_chunk_count(a.n_vec, kChunk, a.shift);
    for (uint32_t c = wave; c < n_chunks; c += waves)
        flat_chunk<U, NTL>(a.src, static_cast<vec16 *>(a.out), a.n_vec, a.vpr, a.div, a.shift, c);
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
    const uint64_t w0 = cut.lo + uint64_t(j) * 1024;  // the wave's first body byte
    const OutWindow<kStoreAux> w(d + w0, window_bytes(w0, cut.hi, 1024));
    const uint64_t off = w0 + 16 * lane;
    const bool live = off < cut.hi;
    const uint32_t m = uniform(uint32_t(reinterpret_cast<uintptr_t>(s + cut.lo)) & 15);
    if (!NTL || !shift_granules(m, kPeerShift)) {
        if (live) w.st16(16 * lane, ldu16<NTL>(s + off));
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
    const vec16 next = from_next_lane(lo);
    if (live) w.st16(16 * lane, cut16(lo, own_hi ? hi : next, m));
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
    uint8_t *db = d + cut.lo;
    const uint64_t count = (cut.hi - cut.lo) >> 4;
    const uint64_t tile = uint64_t(nt) * U;
    for (uint64_t base = 0; base < count; base += tile) {
        const OutWindow<kStoreAux> w(db + 16 * base, window_bytes(16 * base, 16 * count, 16 * tile));
        if (base + tile <= count) {
            vec16 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = ldu16<NTL>(sb + 16 * (base + u * nt + tid));
#pragma unroll
            for (int u = 0; u < U; ++u) w.st16(16 * (u * nt + tid), v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t k = base + u * nt + tid;
                if (k < count) w.st16(uint32_t(16 * (k - base)), ldu16<NTL>(sb + 16 * k));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
// Multi-WG FLAT: one wave per workgroup and per chunk, grid-strided over a
// capped grid.  Where the output, the payload size and every source sit on
// 128-byte lines, chunks go to the XCDs round-robin.  Otherwise neighbouring
// chunks read parts of the same source lines, and they go to the XCDs in runs
// (xcd_grouped) that keep those lines in one L2: 17-26 % faster there, 1-1.5 %
// slower on aligned gathers.  The arguments, the first eight payload pointers
// included, are read in one batch of scalar loads and a wave picks its
// payload's pointer with scalar selects, so it waits for one scalar round trip
// before its first data load (three before: small multi-WG gathers 0.1-0.2 us
// faster, cold 64 MiB outputs half a point to a point).
template <bool NTL>
__global__ __launch_bounds__(kWaveBlock) void rog_flat_kernel(FlatArgs) {
    constexpr uint32_t kChunk = 64 * kFlatUnroll;
    const FlatArgs &a = launch_args<FlatArgs>();
    const SrcTable src(a.src);
    const uint32_t n_vec = a.n_vec, vpr = a.vpr, shift = a.shift, runs = a.runs, grid = a.grid;
    const Divider div = a.div;
    vec16 *const out = static_cast<vec16 *>(a.out);
    hold_scalars(src, n_vec, vpr, shift, runs, grid, div, out);
    const uint32_t n_chunks = flat_chunk_count(n_vec, kChunk, shift);
    for (uint32_t vb = blockIdx.x; vb < n_chunks; vb += grid)
        flat_chunk<kFlatUnroll, NTL>(src, out, n_vec, vpr, div, shift, runs ? xcd_grouped(vb, n_chunks) : vb);
}

// Single-WG FLAT: one workgroup of as many waves as there are chunks (<= 16),
// U = single_flat_unroll(n_vec) vectors per lane.
template <int U, bool NTL>
__global__ __launch_bounds__(kSingleBlock) void rog_flat_single_kernel(FlatArgs a) {
    flat_copy<U, NTL>(a, blockDim.x / 64);
}

// Multi-WG PEER: one wave per workgroup and per body chunk, chunks grouped by
// XCD, grid-strided over the n_chunks = W * chunks_per_peer chunks.
// The arguments are read in one batch of scalar loads, as in the FLAT kernel,
// but the payload's pointer with one more dependent load: picking it from
// preloaded registers by scalar selects, as FLAT does, measured 1-3 % slower
// here (streamed loads at odd offsets), the dependent load 0-1 % faster than
// leaving the reads as the compiler orders them.
template <bool NTL>
__global__ __launch_bounds__(kWaveBlock) void rog_peer_kernel(PeerArgs) {
    const PeerArgs &a = launch_args<PeerArgs>();
    const uint32_t n_chunks = a.n_chunks, cpp = a.chunks_per_peer, grid = a.grid;
    const uint64_t S = a.S;
    const Divider cdiv = a.cdiv;
    uint8_t *const out = static_cast<uint8_t *>(a.out);
    hold_scalars(n_chunks, cpp, uint32_t(S), uint32_t(S >> 32), grid, cdiv, out);
    for (uint32_t vb = blockIdx.x; vb < n_chunks; vb += grid) {
        const uint32_t b = xcd_grouped(vb, n_chunks);
        const uint32_t r = divide(b, cdiv);
        peer_chunk<NTL>(static_cast<const uint8_t *>(a.src[r]), out + uint64_t(r) * S, S, b - r * cpp);
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

// BATCH: one wave per workgroup and per chunk of some tensor.  The chunks of
// the FLAT tensors whose output, size and sources all sit on 128-byte lines
// come first and go to the XCDs round-robin; the other tensors' chunks (FLAT
// or PEER) follow, handed out in XCD runs as in the FLAT and PEER kernels.
// (Runs over the aligned FLAT chunks too measured 5 % slower on an aligned
// batch; no runs at all, 9 % slower on 8 x 64 MiB PEER payloads.)
template <bool NTL>
__global__ __launch_bounds__(kWaveBlock) void rog_batch_kernel(BatchArgs) {
    const BatchArgs &a = launch_args<BatchArgs>();
    const uint32_t n_chunks = a.n_chunks, aligned = a.aligned_chunks, W = a.W, grid = a.grid;
    hold_scalars(n_chunks, aligned, a.lookup.shift, W, grid);
    for (uint32_t vb = blockIdx.x; vb < n_chunks; vb += grid) {
        const uint32_t c = vb < aligned ? vb : aligned + xcd_grouped(vb - aligned, n_chunks - aligned);
        const uint32_t lo = batch_tensor(a.first, a.lookup, c);
        const BatchTensor &t = a.t[lo];
        const uint32_t lc = c - a.first[lo];
        // the tensor's fields either form needs, in one batch of scalar loads
        hold_scalars(lc, t.flat, t.vpr, t.n_vec, t.shift, t.div, reinterpret_cast<const void *>(t.out));
        hold_scalars(t.chunks_per_peer, uint32_t(t.S), uint32_t(t.S >> 32), 0u, 0u);
        const void *const *src = a.src + lo * W;
        if (t.flat) {
            flat_chunk<kFlatUnroll, NTL>(src, reinterpret_cast<vec16 *>(t.out), t.n_vec, t.vpr, t.div, t.shift, lc);
        } else {
            const uint32_t r = divide(lc, t.div);
            // the output address through a global pointer, so that the head
            // and tail byte stores are global stores rather than flat ones
            uint8_t *const d = (uint8_t *)(__attribute__((address_space(1))) uint8_t *)t.out;
            peer_chunk<NTL>(static_cast<const uint8_t *>(src[r]), d + uint64_t(r) * t.S,
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
        else        k = ntl ? kfn(&rog_flat_kernel<true>) : kfn(&rog_flat_kernel<false>);
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
