// rog_internal.h -- launch plans and kernel-argument layouts shared by the host
// planner (rog_plan.cpp) and the HIP kernels (rog_kernels.hip, rog_reduce.hip).
// Internal to librog.so; the public interface is include/rog.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rog.h"

namespace rog {

// Kernel-argument capacities.  Everything a launch needs travels in the kernel
// arguments, so the library never allocates device memory.  The largest
// argument block (BatchArgs) stays below 4 KiB.
constexpr int kMaxPeers = 64;
constexpr int kMaxBatch = 32;
constexpr int kMaxBatchPtrs = 192;

// Tunables.  Each default was measured on MI355X (bench sweeps over forced
// paths, workgroup sizes, unroll depths, cache policies and workgroup-to-XCD
// placement); a variant build may override one with -D for a sweep.
#ifndef ROG_SINGLE_WG_MAX_BYTES
#define ROG_SINGLE_WG_MAX_BYTES (32 * 1024)
#endif
#ifndef ROG_REDUCE_SINGLE_WG_MAX_BYTES
#define ROG_REDUCE_SINGLE_WG_MAX_BYTES (64 * 1024)
#endif
#ifndef ROG_FLAT_UNROLL
#define ROG_FLAT_UNROLL 1
#endif
#ifndef ROG_SINGLE_UNROLL
#define ROG_SINGLE_UNROLL 4
#endif
#ifndef ROG_STORE_AUX
#define ROG_STORE_AUX 18
#endif
#ifndef ROG_SUM_STORE_AUX
#define ROG_SUM_STORE_AUX 2
#endif
#ifndef ROG_GATHER_NT_LOAD_MIN_BYTES
#define ROG_GATHER_NT_LOAD_MIN_BYTES (128ull << 20)
#endif
#ifndef ROG_SUM_NT_LOAD_MIN_BYTES
#define ROG_SUM_NT_LOAD_MIN_BYTES (128ull << 20)
#endif
#ifndef ROG_BODY_ALIGN
#define ROG_BODY_ALIGN 256
#endif
#ifndef ROG_XCD_RUN
#define ROG_XCD_RUN 128
#endif
#ifndef ROG_PEER_SHIFT
#define ROG_PEER_SHIFT 1
#endif
#ifndef ROG_REDUCE_SHIFT
#define ROG_REDUCE_SHIFT 1
#endif
#ifndef ROG_GRID_CAP
#define ROG_GRID_CAP (1u << 30)
#endif

// Output bytes up to which ROG_PATH_AUTO uses the single-workgroup path
// (inclusive), measured by sweeping both forced paths.
constexpr size_t kSingleWgMaxBytes = ROG_SINGLE_WG_MAX_BYTES;
// The bound for rog_reduce, on its source bytes W * count * esize: the measured
// crossover sits at the same source bytes for W = 2 (32 KiB out) and W = 8
// (8 KiB out), as the pages' all-reduce bound is tested on input bytes.
constexpr size_t kReduceSingleWgMaxBytes = ROG_REDUCE_SINGLE_WG_MAX_BYTES;

// Launch shapes.  A multi-WG wave works on a chunk of 64 * unroll consecutive
// 16-byte output vectors; each of its loads and stores is one dwordx4
// instruction over 64 consecutive vectors (1 KiB).  Small workgroups of one
// wave, one 1 KiB chunk each, measured fastest for the HBM-bound launches
// (FLAT, PEER, BATCH and REDUCE alike).
constexpr int kFlatUnroll = ROG_FLAT_UNROLL;      // vectors per lane per chunk
constexpr int kWaveBlock = 64;                    // multi-WG workgroup (FLAT, PEER, BATCH, REDUCE)
constexpr int kSingleBlock = 1024;                // the single workgroup (16 waves)
constexpr int kSingleUnroll = ROG_SINGLE_UNROLL;  // single-WG FLAT vectors per lane
constexpr int kSinglePeerUnroll = 4;              // single-WG PEER vectors per thread
// Cache-policy bits of the gathers' 16-byte output stores (the buffer
// instructions' aux operand: 1 = sc0, 2 = nt, 16 = sc1).  18 = nt sc1:
// streamed, and written through each XCD's L2 at device scope, so the end of
// a launch finds no dirty output lines there to write back.  Against nt alone
// it measured 3 % faster on 8 x 64 MiB gathers (FLAT and PEER alike).  It
// loses where neighbouring chunks split output lines between them, since two
// partial writes then go out instead of one merged line.
constexpr int kStoreAux = ROG_STORE_AUX;
// The rank-ordered sum's stores: nt alone.  Its granule form starts the body
// where source 0's lines start, so output lines may be split between chunks;
// there nt sc1 measured 3-7 % slower, and it gained nothing where aligned.
constexpr int kSumStoreAux = ROG_SUM_STORE_AUX;
// Vectors per lane of the single-WG FLAT kernel for an output of n_vec vectors:
// 1 while one pass of 16 waves covers the output (1 KiB wave chunks then line
// up with payloads of 1 KiB or more, so no chunk takes the per-lane payload
// lookup), kSingleUnroll beyond.
inline int single_flat_unroll(uint64_t n_vec) { return n_vec <= uint64_t(kSingleBlock) ? 1 : kSingleUnroll; }
// Source bytes from which 16-byte loads are non-temporal: below it the payloads
// may still sit in the 256 MB Infinity Cache, and cached loads then win.
// Gathers, single (FLAT or PEER) or batched, switch at 128 MiB: there, over
// buffers that miss the Infinity Cache, streamed loads measured 81-82 % of
// peak against 78 % cached for FLAT (128 MiB of output) and 83-84 % against
// 80 % (256 MiB), 79-83 % against 77-80 % for PEER and batches (128-312 MiB),
// while over buffers it still holds they measured 80-83 % against 89-91 %
// cached; at 64 MiB of output cached loads keep 85 % warm (77 % streamed) and
// lose 2 points cold (75 % against 77 %).  Sums (single or batched) switch at
// 128 MiB of sources too, where they then read shared granules
// (sum_granule_group): over W = 2 to 16 and 128 to 512 MiB of sources,
// streamed loads lifted the slower of warm and cold against cached loads or
// tied it.
constexpr uint64_t kGatherNtLoadMinBytes = ROG_GATHER_NT_LOAD_MIN_BYTES;
constexpr uint64_t kSumNtLoadMinBytes = ROG_SUM_NT_LOAD_MIN_BYTES;

// Sources whose granules a lane of the sum's granule form holds in flight at
// once, by W.  The registers scale with it: 8 sources take 95 VGPRs (5 waves
// per SIMD), 4 take 54 and 2 take 37 (8 waves each).  Measured over W = 2 to
// 16 and 256 to 512 MiB of sources: 2 for W <= 2 (24-30 % faster than 8),
// 4 for W = 3 (9-13 % faster than 8), 8 from W = 4 on (the best group, or
// within 2.5 % of it).
inline uint32_t sum_granule_group(uint32_t W) { return W <= 2 ? 2 : W == 3 ? 4 : 8; }
constexpr uint32_t kGridCap = ROG_GRID_CAP;       // workgroups of one launch, at most
// Destination alignment at which a PEER payload's 16-byte body starts (a power
// of two >= 16): each wave's 1 KiB of stores then covers whole cache lines.
// 256 measured best (vs 16: +4.7 % on 8 x 64 MiB at offsets 1/3).
constexpr uint64_t kBodyAlign = ROG_BODY_ALIGN;
static_assert(kBodyAlign >= 16 && (kBodyAlign & (kBodyAlign - 1)) == 0, "body alignment");
// Workgroups are dispatched to the 8 XCDs round-robin.  PEER, BATCH and REDUCE
// launches hand each XCD runs of kXcdRun consecutive 1 KiB chunks (128 measured
// best of 1..1024 for PEER: a misaligned chunk straddles one cache line with
// its neighbour, which then sits in the same L2).
constexpr uint32_t kXcds = 8;
constexpr uint32_t kXcdRun = ROG_XCD_RUN;
// Multi-WG PEER body loads, where the loads stream past the caches, at a
// source misaligned by m = 1..15 bytes from its 16-byte granule: 0 = one
// unaligned 16-byte load per lane; 1 = for m not a multiple of 4, one aligned
// load per lane, the next granule taken from the next lane and the 16 bytes
// cut out of the pair; 2 = the same for every m.  1 measured best on
// 8 x 64 MiB: +2-4 % over 0 at odd and 2-mod-4 offsets, equal at multiples of
// 4 (where 2 loses 1-2 %).  With cached loads (2 or 4 x 64 MiB) unaligned
// loads win at every offset (+7 %), so the kernel keeps them there.
constexpr int kPeerShift = ROG_PEER_SHIFT;
// When the multi-WG rank-ordered sum reads every source as shared granules
// (its granule form) instead of one unaligned 16-byte load per lane and
// source: 0 never; 1 whenever the launch streams its loads past the caches
// (ROG_PLAN_NT_LOADS), whatever the alignment; 2 always.  Measured on MI355X: with
// streamed loads (W = 8 x 64 MiB) the granule form runs 6.55-6.6 TB/s aligned
// or misaligned, against 6.2-6.3 aligned and 5.4-6.0 misaligned for unaligned
// loads; with cached loads (W = 2-4 x 64 MiB, 8 x 8 MiB) the unaligned loads
// are as fast or faster at every offset (up to +20 %).
constexpr int kReduceShift = ROG_REDUCE_SHIFT;

// Whether a body whose source bytes sit m = 0..15 bytes past a 16-byte
// granule is read as aligned granules shared between neighbouring lanes,
// under mode 0, 1 or 2 above.
__host__ __device__ inline bool shift_granules(uint32_t m, int mode) {
    return mode == 2 ? m != 0 : (mode == 1 && (m & 3) != 0);
}

// Exact floor(v / d) for every 32-bit v by one 32x32 high multiply:
// t = mulhi(v, magic); q = (t + ((v - t) >> sh1)) >> sh2.
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, unsigned case with the 33-bit multiplier.)
struct Divider {
    uint32_t magic;
    uint32_t sh1;
    uint32_t sh2;
};

Divider make_divider(uint32_t d);

// How the PEER path cuts a payload, and the REDUCE path its output
// (destination address da, S bytes): bytes [0, lo) and [hi, S) move one by one
// (one element at a time for REDUCE), bytes [lo, hi) as aligned 16-byte
// stores, each fed by 16-byte loads of the source bytes at the same offset
// (aligned or not).  The body starts at the first kBodyAlign-aligned
// destination byte; every read lies inside the source's S bytes and every
// store is aligned.
struct PeerSplit {
    uint64_t lo;      // first byte of the body (da + lo is kBodyAlign-aligned)
    uint64_t hi;      // end of the body; (hi - lo) % 16 == 0; lo == hi: no body
};

__host__ __device__ inline PeerSplit split_payload(uint64_t da, uint64_t S) {
    const uint64_t to_line = (kBodyAlign - (da & (kBodyAlign - 1))) & (kBodyAlign - 1);
    if (S < to_line + 16) return PeerSplit{S, S};          // too small for a body
    return PeerSplit{to_line, to_line + ((S - to_line) & ~uint64_t(15))};
}

// The cut of the rank-ordered sum's granule form: the body starts at the
// first offset l (< 128) where out + l is 16-byte aligned and the anchor
// source's granule run starts a 128-byte line ((anchor + l) % 128 < 16), so
// that each 1 KiB chunk reads that source as whole lines.  Output stores stay
// aligned 16-byte vectors; the head [0, lo) and tail [hi, S) are elements.
// Streamed sums whose sources sat elsewhere in a line measured 4 % slower
// with split_payload's cut.
__host__ __device__ inline PeerSplit split_anchored(uint64_t da, uint64_t S, uint64_t anchor) {
    uint64_t l = (16 - (da & 15)) & 15;
    while (((anchor + l) & 127) >= 16) l += 16;   // at most 7 steps: l + 16k covers every residue
    if (S < l + 16) return PeerSplit{S, S};
    return PeerSplit{l, l + ((S - l) & ~uint64_t(15))};
}

// Workgroups go to the 8 XCDs round-robin (b mod 8).  Hand each XCD runs of
// kXcdRun consecutive chunks, so that neighbouring chunks -- which share the
// cache line a misaligned chunk straddles -- meet in the same L2.  A bijection
// on [0, n): whole spans of 8 * kXcdRun are permuted, the rest is left as is.
__host__ __device__ inline uint32_t xcd_grouped(uint32_t b, uint32_t n) {
    constexpr uint32_t kSpan = kXcds * kXcdRun;
    if (kXcdRun <= 1 || b >= n - n % kSpan) return b;
    const uint32_t x = b % kXcds, k = b / kXcds;
    return (k / kXcdRun) * kSpan + x * kXcdRun + k % kXcdRun;
}

// FLAT chunks of `chunk` output vectors, shifted back by `shift` vectors:
// chunk c covers vectors [c * chunk - shift, (c + 1) * chunk - shift) clipped
// to [0, n_vec).  With shift = (out % 128) / 16 every chunk after the first
// starts on one of the output's 128-byte lines, so no two chunks write parts
// of one line.  The host keeps shift = 0 unless n_vec < 2^31, so c * chunk
// never wraps (c * chunk < n_vec + shift, and 2^32 is a multiple of chunk).
struct ChunkSpan {
    uint32_t b;   // first vector
    uint32_t n;   // vectors, >= 1 for c < flat_chunk_count(...)
};
__host__ __device__ inline ChunkSpan flat_span(uint32_t c, uint32_t chunk, uint32_t shift, uint32_t n_vec) {
    const uint32_t b = c == 0 ? 0 : c * chunk - shift;
    const uint32_t cap = c == 0 ? chunk - shift : chunk;
    const uint32_t left = n_vec - b;
    return ChunkSpan{b, left < cap ? left : cap};
}
__host__ __device__ inline uint32_t flat_chunk_count(uint32_t n_vec, uint32_t chunk, uint32_t shift) {
    return uint32_t((uint64_t(n_vec) + shift + chunk - 1) / chunk);
}
// The shift for an output at address out of n_vec vectors (out 16-byte aligned).
inline uint32_t flat_shift(uint64_t out, uint64_t n_vec) {
    return n_vec < (uint64_t(1) << 31) ? uint32_t((out & 127) >> 4) : 0;
}

// A batch launch's chunks are its tensors' chunks laid end to end; tensor t
// owns chunks [first[t], first[t + 1]).  For the batched gather to find the
// tensor of chunk c without a full binary search of dependent loads (1-1.5 %
// faster on batches with misaligned tensors), the chunk space is cut into
// kBatchBuckets buckets of 2^shift chunks, and bucket_lo[b] names the tensor
// that owns the first chunk of bucket b (bucket_lo[kBatchBuckets] the last
// tensor).  Chunk c's tensor lies in [bucket_lo[b], bucket_lo[b + 1]] for
// b = c >> shift, so the search runs only over the tensors that meet the
// bucket: none at all for a chunk of a tensor larger than a bucket.
constexpr uint32_t kBatchBuckets = 256;
struct BatchLookup {
    uint32_t shift;                          // log2 of the chunks per bucket
    uint32_t bucket_lo[kBatchBuckets / 4 + 1];   // entry b in byte b % 4 of word b / 4; b <= kBatchBuckets
};
static_assert(kMaxBatch <= 256, "bucket entries are bytes");

// Entry b of a bucket table, read as whole 32-bit words (scalar loads; the
// device has no scalar byte load, and a byte read from memory would become a
// vector load).
__host__ __device__ inline uint32_t bucket_entry(const BatchLookup &lk, uint32_t b) {
    return (lk.bucket_lo[b >> 2] >> (8 * (b & 3))) & 0xFFu;
}

// The tensor that owns chunk c (c below the launch's chunk count, first[0] == 0
// and first[] strictly increasing over the tensors).
__host__ __device__ inline uint32_t batch_tensor(const uint32_t *first, const BatchLookup &lk, uint32_t c) {
    const uint32_t b = c >> lk.shift;
    uint32_t lo = bucket_entry(lk, b), hi = bucket_entry(lk, b + 1) + 1;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (first[mid] <= c) lo = mid;
        else hi = mid;
    }
    return lo;
}

// The tensor that owns chunk c by a binary search over all n first chunks
// (n >= 1, the same conditions on first[]).  The batched sums use it: there
// the bucket table measured 0.5-1 % slower than this search.
__host__ __device__ inline uint32_t search_tensor(const uint32_t *first, uint32_t n, uint32_t c) {
    uint32_t lo = 0, hi = n;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (first[mid] <= c) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Fill lk for n tensors (n >= 1) with first chunks first[0 .. n) and
// n_chunks chunks in all (n_chunks >= 1).
inline void plan_lookup(const uint32_t *first, uint32_t n, uint32_t n_chunks, BatchLookup *lk) {
    uint32_t shift = 0;
    while (((n_chunks - 1) >> shift) >= kBatchBuckets) ++shift;
    lk->shift = shift;
    for (uint32_t w = 0; w < kBatchBuckets / 4 + 1; ++w) lk->bucket_lo[w] = 0;
    uint32_t t = 0;
    for (uint32_t b = 0; b <= kBatchBuckets; ++b) {
        const uint64_t c0 = uint64_t(b) << shift;
        const uint32_t c = c0 < n_chunks ? uint32_t(c0) : n_chunks - 1;
        while (t + 1 < n && first[t + 1] <= c) ++t;
        lk->bucket_lo[b >> 2] |= t << (8 * (b & 3));
    }
}

// ---------------------------------------------------------------------------
// Kernel arguments
// ---------------------------------------------------------------------------

// FLAT: the whole output is one space of n_vec 16-byte vectors; vector v comes
// from payload r = v / vpr at index v - r*vpr.  Chunks as flat_span cuts them.
struct FlatArgs {
    const void *src[kMaxPeers];
    void *out;
    uint32_t n_vec;
    uint32_t vpr;
    Divider div;
    uint32_t shift;   // flat_span's shift: 0..7 (multi-WG), 0 (single-WG)
    uint32_t runs;    // multi-WG: 1 = chunks to the XCDs in runs, 0 = round-robin
    uint32_t grid;    // multi-WG: workgroups launched (the grid stride), read
                      // with the other arguments instead of from the dispatch
};

// PEER: each payload is its own copy job, cut by split_payload into a byte
// head, a body of aligned 16-byte stores and a byte tail.
// Multi-WG: chunk b of n_chunks = W * chunks_per_peer is chunk b % chunks_per_peer
// of payload b / chunks_per_peer (cdiv divides by chunks_per_peer); a chunk is
// 64 body vectors, and chunk 0 also moves the head and tail bytes.
// Single-WG (chunk fields unused): the one workgroup takes the payloads in turn.
struct PeerArgs {
    const void *src[kMaxPeers];
    void *out;
    uint64_t S;
    uint32_t W;
    uint32_t chunks_per_peer;
    uint32_t n_chunks;
    Divider cdiv;
    uint32_t grid;    // multi-WG: workgroups launched (the grid stride)
};

// One tensor of a batch.  Chunks [first, first + n_chunks) of the launch
// belong to it.  FLAT tensors: chunk c is flat_span(c, 64, shift, n_vec), the
// payload found by div (divides by vpr).  PEER tensors: chunk c is chunk
// c % chunks_per_peer of payload c / chunks_per_peer (div divides by
// chunks_per_peer).
struct BatchTensor {
    uint64_t out;
    uint64_t S;
    uint32_t n_chunks;
    uint32_t flat;              // 1: FLAT tensor, 0: PEER tensor
    uint32_t vpr;               // FLAT: vectors per rank
    uint32_t n_vec;             // FLAT: W * vpr
    uint32_t shift;             // FLAT: flat_span's shift
    uint32_t chunks_per_peer;   // PEER
    Divider div;
};

struct BatchArgs {
    const void *src[kMaxBatchPtrs];   // tensor t's payloads at [t*W, t*W + W)
    uint32_t first[kMaxBatch];        // tensor t's first chunk (strictly increasing over [0, n))
    BatchTensor t[kMaxBatch];
    uint32_t n;
    uint32_t W;
    uint32_t n_chunks;                // all tensors' chunks
    uint32_t aligned_chunks;          // chunks of the line-aligned FLAT tensors, which come first
    uint32_t grid;                    // workgroups launched (the grid stride)
    BatchLookup lookup;               // chunk -> tensor buckets
};

static_assert(sizeof(BatchArgs) <= 4096, "kernel arguments must stay below 4 KiB");

// REDUCE: out[i] = rank-ordered binary32 sum of src[r][i], rounded to the
// element type.  The output is cut by split_payload into an element head, a
// body of 16-byte vectors (8 bf16 or 4 f32 elements each) and an element tail;
// multi-WG chunk j is body vectors [64j, 64j + 64), and chunk 0 also sums the
// head and tail elements.
struct ReduceArgs {
    const void *src[kMaxPeers];
    void *out;
    uint64_t count;             // elements
    uint32_t W;
    uint32_t n_chunks;          // multi-WG
    uint32_t grid;              // multi-WG: workgroups launched (the grid stride)
};

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

struct Plan {
    rog_plan_info info;
    FlatArgs flat;
    PeerArgs peer;
    ReduceArgs reduce;
    rog_dtype dtype;
};

// hipError_t of this thread's last failed launch (rog_last_hip_error).
extern thread_local int g_last_hip_error;

// Validate and plan one gather (no HIP calls).
rog_status plan_gather(const void *const *srcs, int W, size_t S, const void *out,
                       rog_path path, Plan *plan);

// One tensor of a batched sum: chunks [first, first + n_chunks) of
// the launch, each 64 body vectors of its output (chunk 0 also sums the head
// and tail elements).
struct ReduceTensor {
    uint64_t out;
    uint64_t count;             // elements
    uint32_t n_chunks;
};

struct ReduceBatchArgs {
    const void *src[kMaxBatchPtrs];   // tensor t's payloads at [t*W, t*W + W)
    uint32_t first[kMaxBatch];        // tensor t's first chunk (strictly increasing over [0, n))
    ReduceTensor t[kMaxBatch];
    uint32_t n;
    uint32_t W;
    uint32_t n_chunks;                // all tensors' chunks
    uint32_t grid;                    // workgroups launched (the grid stride)
};

static_assert(sizeof(ReduceBatchArgs) <= 4096, "kernel arguments must stay below 4 KiB");

// Validate and plan one rank-ordered sum (no HIP calls).
rog_status plan_reduce(const void *const *srcs, int W, size_t count, rog_dtype dtype,
                       const void *out, rog_path path, Plan *plan);

// Validate and plan a batch of rank-ordered sums (no HIP calls).  grid == 0
// means nothing to launch.  *shifted: some tensor's body is read as shared
// aligned granules (the launch takes the kernel that can).
rog_status plan_reduce_batch(const rog_reduce_desc *descs, int n, int W, rog_dtype dtype,
                             ReduceBatchArgs *args, uint32_t *grid, bool *nt_loads, bool *shifted);

// Validate and plan a batch (no HIP calls).  grid == 0 means nothing to launch.
// *nt_loads: the launch streams its loads past the caches.
rog_status plan_batch(const rog_gather_desc *descs, int n, int W, BatchArgs *args,
                      uint32_t *grid, bool *nt_loads);

}  // namespace rog
