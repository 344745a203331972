// rog_plan.cpp -- argument validation, alignment classification, path dispatch
// and grid sizing for the rank-ordered gather and the rank-ordered sum.  Pure
// host code: no HIP calls, so every decision here can be checked on a machine
// without a GPU.
//
// Decisions follow RL-Align/RL-Kernel PR #491 ("perf(cuda): vectorize the
// deterministic all-gather copy and right-size its single-block path"):
//  * "What", copy_rank_ordered bullet: if the output address, the payload
//    size and every source address are multiples of 16, a single loop walks
//    the 16-byte vectors of all payloads as one range; if not, payloads are
//    copied one by one, in vectors only where source and destination allow
//    it, byte by byte for the rest.
//  * "What", kAllGatherSingleBlockMaxBytes bullet: the single-block path is
//    chosen by output size, inclusive; the bound here is measured on MI355X.
//  * review thread on grid sizing: the multi-block grid follows the number of
//    16-byte vectors on the aligned path and each payload's own work on the
//    other.
//  * author's reply on the benchmark sizes: the all-reduce's single-block
//    bound is tested on input bytes; rog_reduce's bound likewise counts source
//    bytes (W * count * element size).
#include <limits.h>
#include <string.h>

#include <algorithm>

#include "rog_internal.h"

namespace rog {

Divider make_divider(uint32_t d) {
    // d >= 1.  l = ceil(log2 d); magic = floor(2^32 * (2^l - d) / d) + 1.
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    const uint64_t magic = ((((uint64_t(1) << l) - d) << 32) / d) + 1;
    Divider r;
    r.magic = uint32_t(magic);
    r.sh1 = l < 1 ? l : 1;
    r.sh2 = l > 0 ? l - 1 : 0;
    return r;
}

namespace {

constexpr uint64_t kMaxOutputBytes = uint64_t(1) << 36;   // 2^32 vectors of 16 bytes

inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

inline uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// [a, a+na) and [b, b+nb) share a byte.
inline bool ranges_overlap(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb) {
    return na && nb && a < b + nb && b < a + na;
}

// Shared checks of one gather: pointers, limits, address wrap, overlap.
rog_status validate(const void *const *srcs, int W, size_t S, const void *out,
                    uint64_t *total_out) {
    if (!srcs || W < 1 || W > kMaxPeers) return ROG_ERR_INVALID_ARGUMENT;
    if (S == 0) { *total_out = 0; return ROG_OK; }
    if (!out) return ROG_ERR_INVALID_ARGUMENT;
    for (int r = 0; r < W; ++r)
        if (!srcs[r]) return ROG_ERR_INVALID_ARGUMENT;
    if (S > SIZE_MAX / size_t(W)) return ROG_ERR_TOO_LARGE;
    const uint64_t total = uint64_t(S) * uint64_t(W);
    if (total >= kMaxOutputBytes) return ROG_ERR_TOO_LARGE;
    const uintptr_t o = addr(out);
    if (o > UINTPTR_MAX - total) return ROG_ERR_INVALID_ARGUMENT;
    for (int r = 0; r < W; ++r) {
        const uintptr_t s = addr(srcs[r]);
        if (s > UINTPTR_MAX - S) return ROG_ERR_INVALID_ARGUMENT;
        // The one overlap allowed: payload r already sits in its own segment.
        if (ranges_overlap(s, S, o, total) && s != o + uint64_t(r) * S)
            return ROG_ERR_OVERLAP;
    }
    *total_out = total;
    return ROG_OK;
}

bool is_flat(const void *const *srcs, int W, size_t S, const void *out) {
    uintptr_t bits = addr(out) | uintptr_t(S);
    for (int r = 0; r < W; ++r) bits |= addr(srcs[r]);
    return (bits & 15) == 0;
}

uint64_t vec_ok_mask(const void *const *srcs, int W, size_t S, const void *out) {
    uint64_t m = 0;
    for (int r = 0; r < W; ++r) {
        const uintptr_t d = addr(out) + uintptr_t(r) * S;
        if (((addr(srcs[r]) | d) & 15) == 0) m |= uint64_t(1) << r;
    }
    return m;
}

// Largest grid for a workgroup size: an AMD dispatch counts work-items in 32
// bits, so grid * block must stay below 2^32.  Kernels grid-stride, so a capped
// grid still covers all work.
uint32_t max_grid(int block) {
    return std::min<uint32_t>(kGridCap, 0xFFFFFFFFu / uint32_t(block));
}

// Multi-WG FLAT grid: one one-wave workgroup per chunk (flat_span).
uint32_t flat_blocks(uint32_t n_vec, uint32_t shift) {
    const uint32_t chunks = flat_chunk_count(n_vec, 64 * uint32_t(kFlatUnroll), shift);
    return std::max<uint32_t>(1, std::min<uint32_t>(chunks, max_grid(kWaveBlock)));
}

// Whether the output, the payload size and every source sit on 128-byte lines.
bool line_aligned(const void *const *srcs, int W, size_t S, const void *out) {
    uint64_t bits = addr(out) | uint64_t(S);
    for (int r = 0; r < W; ++r) bits |= addr(srcs[r]);
    return (bits & 127) == 0;
}

// Multi-WG PEER: 1 KiB body chunks per payload, enough for the largest body
// (every payload has at most S/16 body vectors, whatever its alignment).
// S/16 < 2^32 / W, so W * chunks_per_peer stays below 2^26 + W.
uint32_t peer_chunks_per_peer(size_t S) {
    return uint32_t(std::max<uint64_t>(1, ceil_div(S / 16, 64)));
}

uint32_t round_up_64(uint64_t threads) {
    return uint32_t(std::min<uint64_t>(kSingleBlock, std::max<uint64_t>(64, (threads + 63) / 64 * 64)));
}

// Single-WG FLAT workgroup: one wave per chunk of 64 * single_flat_unroll
// vectors, at most 16 waves (idle waves only cost launch time).
uint32_t flat_single_block(uint64_t n_vec) {
    return round_up_64(ceil_div(n_vec, 64 * uint64_t(single_flat_unroll(n_vec))) * 64);
}

// Whether the multi-WG body of a payload of S bytes from src to the output
// address d is read as shared aligned granules (mode as kPeerShift).
bool shifted_body(const void *src, uint64_t d, uint64_t S, int mode) {
    const PeerSplit cut = split_payload(d, S);
    if (cut.hi == cut.lo) return false;
    return shift_granules(uint32_t(addr(src) + cut.lo) & 15, mode);
}

// Single-WG PEER workgroup: enough threads for one tile of the largest payload.
uint32_t peer_single_block(size_t S) {
    return round_up_64(ceil_div(S / 16, kSinglePeerUnroll));
}

}  // namespace

rog_status plan_gather(const void *const *srcs, int W, size_t S, const void *out,
                       rog_path path, Plan *plan) {
    if (path != ROG_PATH_AUTO && path != ROG_PATH_SINGLE_WG && path != ROG_PATH_MULTI_WG)
        return ROG_ERR_INVALID_ARGUMENT;
    uint64_t total = 0;
    const rog_status st = validate(srcs, W, S, out, &total);
    if (st != ROG_OK) return st;

    rog_plan_info &info = plan->info;
    memset(&info, 0, sizeof(info));
    if (path == ROG_PATH_AUTO)
        path = total <= kSingleWgMaxBytes ? ROG_PATH_SINGLE_WG : ROG_PATH_MULTI_WG;
    info.path = path;
    if (total == 0) {
        info.kernel = ROG_KERNEL_NONE;
        return ROG_OK;
    }
    const bool single = path == ROG_PATH_SINGLE_WG;
    const bool flat = is_flat(srcs, W, S, out);
    if (total >= kGatherNtLoadMinBytes) info.flags |= ROG_PLAN_NT_LOADS;

    if (flat) {
        FlatArgs &a = plan->flat;
        memset(&a, 0, sizeof(a));
        for (int r = 0; r < W; ++r) a.src[r] = srcs[r];
        a.out = const_cast<void *>(out);
        a.n_vec = uint32_t(total / 16);
        a.vpr = uint32_t(S / 16);
        a.div = make_divider(a.vpr);
        a.shift = single ? 0 : flat_shift(addr(out), a.n_vec);
        a.runs = !single && !line_aligned(srcs, W, S, out);
        info.kernel = ROG_KERNEL_FLAT;
        info.units = a.n_vec;
        info.block = single ? flat_single_block(a.n_vec) : kWaveBlock;
        info.grid = single ? 1 : flat_blocks(a.n_vec, a.shift);
        a.grid = info.grid;
        info.peer_magic = a.div.magic;
        info.peer_sh1 = a.div.sh1;
        info.peer_sh2 = a.div.sh2;
    } else {
        PeerArgs &a = plan->peer;
        memset(&a, 0, sizeof(a));
        for (int r = 0; r < W; ++r) a.src[r] = srcs[r];
        a.out = const_cast<void *>(out);
        a.S = S;
        a.W = uint32_t(W);
        info.kernel = ROG_KERNEL_PEER;
        info.vec_ok_mask = vec_ok_mask(srcs, W, S, out);
        info.units = total;
        if (single) {
            info.block = peer_single_block(S);
            info.grid = 1;
        } else {
            a.chunks_per_peer = peer_chunks_per_peer(S);
            a.n_chunks = a.chunks_per_peer * uint32_t(W);
            a.cdiv = make_divider(a.chunks_per_peer);
            info.block = kWaveBlock;
            info.grid = std::min(a.n_chunks, max_grid(kWaveBlock));
            a.grid = info.grid;
            if (info.flags & ROG_PLAN_NT_LOADS)
                for (int r = 0; r < W; ++r)
                    if (shifted_body(srcs[r], addr(out) + uint64_t(r) * S, S, kPeerShift))
                        info.flags |= ROG_PLAN_SHIFTED_LOADS;
        }
    }
    return ROG_OK;
}

namespace {

// Shared checks of one rank-ordered sum: pointers, element alignment, limits,
// address wrap, overlap (out may be exactly a source).  *bytes_out = count * esize.
rog_status validate_reduce(const void *const *srcs, int W, size_t count, size_t esize, const void *out,
                           uint64_t *bytes_out) {
    if (!srcs || W < 1 || W > kMaxPeers) return ROG_ERR_INVALID_ARGUMENT;
    *bytes_out = 0;
    if (count == 0) return ROG_OK;
    if (!out) return ROG_ERR_INVALID_ARGUMENT;
    for (int r = 0; r < W; ++r)
        if (!srcs[r]) return ROG_ERR_INVALID_ARGUMENT;
    if (count > SIZE_MAX / esize) return ROG_ERR_TOO_LARGE;
    const uint64_t bytes = uint64_t(count) * esize;
    if (bytes >= kMaxOutputBytes) return ROG_ERR_TOO_LARGE;
    const uintptr_t o = addr(out);
    if (o % esize) return ROG_ERR_INVALID_ARGUMENT;
    if (o > UINTPTR_MAX - bytes) return ROG_ERR_INVALID_ARGUMENT;
    for (int r = 0; r < W; ++r) {
        const uintptr_t s = addr(srcs[r]);
        if (s % esize) return ROG_ERR_INVALID_ARGUMENT;
        if (s > UINTPTR_MAX - bytes) return ROG_ERR_INVALID_ARGUMENT;
        // In place (out is exactly this source) is allowed: every element is
        // read from every source before the one thread that owns it writes it.
        if (ranges_overlap(s, bytes, o, bytes) && s != o) return ROG_ERR_OVERLAP;
    }
    *bytes_out = bytes;
    return ROG_OK;
}

inline size_t dtype_size(rog_dtype dtype) { return dtype == ROG_DTYPE_F32 ? 4 : 2; }

inline bool dtype_ok(rog_dtype dtype) {
    return dtype == ROG_DTYPE_F32 || dtype == ROG_DTYPE_BF16 || dtype == ROG_DTYPE_F16;
}

// Multi-WG REDUCE: one wave per 1 KiB chunk of the body (at most bytes / 16
// vectors).  bytes < 2^36, so the count fits 26 bits.
uint32_t reduce_chunks(uint64_t bytes) {
    return uint32_t(std::max<uint64_t>(1, ceil_div(bytes / 16, 64)));
}

}  // namespace

rog_status plan_reduce(const void *const *srcs, int W, size_t count, rog_dtype dtype,
                       const void *out, rog_path path, Plan *plan) {
    if (path != ROG_PATH_AUTO && path != ROG_PATH_SINGLE_WG && path != ROG_PATH_MULTI_WG)
        return ROG_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(dtype)) return ROG_ERR_INVALID_ARGUMENT;
    uint64_t bytes = 0;
    const rog_status st = validate_reduce(srcs, W, count, dtype_size(dtype), out, &bytes);
    if (st != ROG_OK) return st;
    rog_plan_info &info = plan->info;
    memset(&info, 0, sizeof(info));
    plan->dtype = dtype;
    if (count == 0) {
        info.path = path == ROG_PATH_AUTO ? ROG_PATH_SINGLE_WG : path;
        info.kernel = ROG_KERNEL_NONE;
        return ROG_OK;
    }
    if (path == ROG_PATH_AUTO)
        path = uint64_t(W) * bytes <= kReduceSingleWgMaxBytes ? ROG_PATH_SINGLE_WG : ROG_PATH_MULTI_WG;
    info.path = path;
    info.kernel = ROG_KERNEL_REDUCE;
    info.units = count;
    if (uint64_t(W) * bytes >= kSumNtLoadMinBytes) info.flags |= ROG_PLAN_NT_LOADS;

    ReduceArgs &a = plan->reduce;
    memset(&a, 0, sizeof(a));
    for (int r = 0; r < W; ++r) a.src[r] = srcs[r];
    a.out = const_cast<void *>(out);
    a.count = count;
    a.W = uint32_t(W);
    if (path == ROG_PATH_SINGLE_WG) {
        // One thread per 16-byte output vector, at most 1024.
        info.block = round_up_64(ceil_div(bytes, 16));
        info.grid = 1;
    } else {
        a.n_chunks = reduce_chunks(bytes);
        info.block = kWaveBlock;
        info.grid = std::min(a.n_chunks, max_grid(kWaveBlock));
        a.grid = info.grid;
        // The granule form where loads stream past the caches (kReduceShift).
        if (kReduceShift == 2 || (kReduceShift == 1 && (info.flags & ROG_PLAN_NT_LOADS)))
            info.flags |= ROG_PLAN_SHIFTED_LOADS;
    }
    return ROG_OK;
}

rog_status plan_reduce_batch(const rog_reduce_desc *descs, int n, int W, rog_dtype dtype,
                             ReduceBatchArgs *args, uint32_t *grid, bool *nt_loads, bool *shifted) {
    *grid = 0;
    *nt_loads = false;
    *shifted = false;
    if (n < 0 || W < 1 || W > kMaxPeers || !dtype_ok(dtype)) return ROG_ERR_INVALID_ARGUMENT;
    if (n > 0 && !descs) return ROG_ERR_INVALID_ARGUMENT;
    if (n > kMaxBatch || n * W > kMaxBatchPtrs) return ROG_ERR_TOO_LARGE;
    const size_t esize = dtype_size(dtype);
    uint64_t bytes[kMaxBatch];
    for (int t = 0; t < n; ++t) {
        const rog_status st = validate_reduce(descs[t].srcs, W, descs[t].count, esize, descs[t].out, &bytes[t]);
        if (st != ROG_OK) return st;
    }
    // Tensors are summed concurrently: no output may overlap another tensor's
    // output or another tensor's sources.
    for (int t = 0; t < n; ++t) {
        if (!bytes[t]) continue;
        const uintptr_t o = addr(descs[t].out);
        for (int u = 0; u < n; ++u) {
            if (u == t || !bytes[u]) continue;
            if (ranges_overlap(o, bytes[t], addr(descs[u].out), bytes[u])) return ROG_ERR_OVERLAP;
            for (int r = 0; r < W; ++r)
                if (ranges_overlap(o, bytes[t], addr(descs[u].srcs[r]), bytes[u])) return ROG_ERR_OVERLAP;
        }
    }
    memset(args, 0, sizeof(*args));
    args->W = uint32_t(W);
    uint64_t next = 0, source_bytes = 0;
    uint32_t k = 0;
    for (int t = 0; t < n; ++t) {
        if (!bytes[t]) continue;            // empty tensors get no chunks
        ReduceTensor &rt = args->t[k];
        for (int r = 0; r < W; ++r) args->src[k * uint32_t(W) + uint32_t(r)] = descs[t].srcs[r];
        rt.out = addr(descs[t].out);
        rt.count = descs[t].count;
        args->first[k] = uint32_t(next);
        rt.n_chunks = reduce_chunks(bytes[t]);
        next += rt.n_chunks;
        source_bytes += uint64_t(W) * bytes[t];
        ++k;
    }
    args->n = k;
    args->n_chunks = uint32_t(next);   // 32 tensors of < 2^26 chunks each
    *grid = uint32_t(std::min<uint64_t>(next, max_grid(kWaveBlock)));
    args->grid = *grid;
    *nt_loads = source_bytes >= kSumNtLoadMinBytes;
    *shifted = kReduceShift == 2 || (kReduceShift == 1 && *nt_loads);
    return ROG_OK;
}

rog_status plan_batch(const rog_gather_desc *descs, int n, int W, BatchArgs *args,
                      uint32_t *grid, bool *nt_loads) {
    *grid = 0;
    *nt_loads = false;
    if (n < 0 || W < 1 || W > kMaxPeers) return ROG_ERR_INVALID_ARGUMENT;
    if (n > 0 && !descs) return ROG_ERR_INVALID_ARGUMENT;
    if (n > kMaxBatch || n * W > kMaxBatchPtrs) return ROG_ERR_TOO_LARGE;

    uint64_t totals[kMaxBatch];
    for (int t = 0; t < n; ++t) {
        const rog_status st = validate(descs[t].srcs, W, descs[t].bytes_per_rank,
                                       descs[t].out, &totals[t]);
        if (st != ROG_OK) return st;
    }
    // Work of different tensors runs concurrently: no output may overlap another
    // tensor's output or another tensor's sources.
    for (int t = 0; t < n; ++t) {
        if (!totals[t]) continue;
        const uintptr_t o = addr(descs[t].out);
        for (int u = 0; u < n; ++u) {
            if (u == t || !totals[u]) continue;
            if (ranges_overlap(o, totals[t], addr(descs[u].out), totals[u])) return ROG_ERR_OVERLAP;
            for (int r = 0; r < W; ++r)
                if (ranges_overlap(o, totals[t], addr(descs[u].srcs[r]), descs[u].bytes_per_rank))
                    return ROG_ERR_OVERLAP;
        }
    }

    memset(args, 0, sizeof(*args));
    args->W = uint32_t(W);
    // One chunk per wave: 64 * kFlatUnroll output vectors of a FLAT tensor
    // (flat_span), 64 body vectors of one payload of a PEER tensor.  Each
    // tensor has fewer than 2^26 + W chunks, so the batch's chunk count fits
    // 32 bits.  The line-aligned FLAT tensors come first: their chunks go to
    // the XCDs round-robin, the other tensors' chunks that follow in XCD runs.
    bool flat[kMaxBatch], aligned[kMaxBatch];
    for (int t = 0; t < n; ++t) {
        const rog_gather_desc &d = descs[t];
        flat[t] = totals[t] && is_flat(d.srcs, W, d.bytes_per_rank, d.out);
        aligned[t] = flat[t] && line_aligned(d.srcs, W, d.bytes_per_rank, d.out);
    }
    uint64_t next = 0;
    uint32_t k = 0;
    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) args->aligned_chunks = uint32_t(next);
        for (int t = 0; t < n; ++t) {
            if (!totals[t] || aligned[t] != (pass == 0)) continue;   // empty tensors get no chunks
            const rog_gather_desc &d = descs[t];
            const size_t S = d.bytes_per_rank;
            BatchTensor &bt = args->t[k];
            for (int r = 0; r < W; ++r) args->src[k * uint32_t(W) + uint32_t(r)] = d.srcs[r];
            bt.out = addr(d.out);
            bt.S = S;
            args->first[k] = uint32_t(next);
            if (flat[t]) {
                bt.flat = 1;
                bt.n_vec = uint32_t(totals[t] / 16);
                bt.vpr = uint32_t(S / 16);
                bt.div = make_divider(bt.vpr);
                bt.shift = flat_shift(bt.out, bt.n_vec);
                bt.n_chunks = flat_chunk_count(bt.n_vec, 64 * uint32_t(kFlatUnroll), bt.shift);
            } else {
                bt.flat = 0;
                bt.chunks_per_peer = peer_chunks_per_peer(S);
                bt.div = make_divider(bt.chunks_per_peer);
                bt.n_chunks = bt.chunks_per_peer * uint32_t(W);
            }
            next += bt.n_chunks;
            ++k;
        }
    }
    if (next > UINT32_MAX) return ROG_ERR_TOO_LARGE;
    args->n = k;
    args->n_chunks = uint32_t(next);
    *grid = uint32_t(std::min<uint64_t>(next, max_grid(kWaveBlock)));
    args->grid = *grid;
    if (k > 0) plan_lookup(args->first, k, args->n_chunks, &args->lookup);
    uint64_t source_bytes = 0;
    for (int t = 0; t < n; ++t) source_bytes += totals[t];
    *nt_loads = source_bytes >= kGatherNtLoadMinBytes;
    return ROG_OK;
}

}  // namespace rog
