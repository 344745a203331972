// rog_internal.h -- launch plans and kernel-argument layouts shared by the host
// planner (rog_plan.cpp) and the HIP kernels (rog_kernels.hip).  Internal to
// librog.so; the public interface is include/rog.h.
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
// paths, workgroup sizes, unroll depths and cache policies); a variant build
// may override one with -D for a sweep.
#ifndef ROG_SINGLE_WG_MAX_BYTES
#define ROG_SINGLE_WG_MAX_BYTES (32 * 1024)
#endif
#ifndef ROG_FLAT_BLOCK
#define ROG_FLAT_BLOCK 64
#endif
#ifndef ROG_FLAT_UNROLL
#define ROG_FLAT_UNROLL 1
#endif
#ifndef ROG_SINGLE_UNROLL
#define ROG_SINGLE_UNROLL 4
#endif
#ifndef ROG_PEER_BLOCK
#define ROG_PEER_BLOCK 256
#endif
#ifndef ROG_PEER_UNROLL
#define ROG_PEER_UNROLL 2
#endif
#ifndef ROG_BATCH_BLOCK
#define ROG_BATCH_BLOCK 256
#endif
#ifndef ROG_BATCH_PEER_UNROLL
#define ROG_BATCH_PEER_UNROLL 1
#endif
#ifndef ROG_NT_STORE
#define ROG_NT_STORE 1
#endif
#ifndef ROG_NT_LOAD_MIN_BYTES
#define ROG_NT_LOAD_MIN_BYTES (384ull << 20)
#endif
#ifndef ROG_BODY_ALIGN
#define ROG_BODY_ALIGN 256
#endif
#ifndef ROG_GRID_CAP
#define ROG_GRID_CAP (1u << 30)
#endif

// Output bytes up to which ROG_PATH_AUTO uses the single-workgroup path
// (inclusive), measured by sweeping both forced paths.
constexpr size_t kSingleWgMaxBytes = ROG_SINGLE_WG_MAX_BYTES;

// Launch shapes.  A FLAT wave copies a chunk of 64 * unroll consecutive 16-byte
// vectors; each of its loads and stores is one dwordx4 instruction over 64
// consecutive vectors (1 KiB).  Small workgroups of one wave, one 1 KiB chunk
// each, measured fastest for HBM-bound gathers.
constexpr int kFlatBlock = ROG_FLAT_BLOCK;        // multi-WG FLAT workgroup (threads)
constexpr int kFlatUnroll = ROG_FLAT_UNROLL;      // vectors per lane per chunk
constexpr int kSingleBlock = 1024;                // the single workgroup (16 waves)
constexpr int kSingleUnroll = ROG_SINGLE_UNROLL;  // single-WG FLAT vectors per lane
constexpr int kPeerBlock = ROG_PEER_BLOCK;        // multi-WG PEER workgroup
constexpr int kPeerUnroll = ROG_PEER_UNROLL;      // PEER vectors per thread per tile
constexpr int kSinglePeerUnroll = 4;              // single-WG PEER vectors per thread
constexpr int kBatchBlock = ROG_BATCH_BLOCK;      // rog_gather_many workgroup
constexpr int kBatchPeerUnroll = ROG_BATCH_PEER_UNROLL;  // its PEER vectors per thread
constexpr bool kNtStore = ROG_NT_STORE != 0;      // non-temporal 16-byte stores
// Source bytes from which 16-byte loads are non-temporal: below it the payloads
// may still sit in the 256 MB Infinity Cache, and cached loads then win.
constexpr uint64_t kNtLoadMinBytes = ROG_NT_LOAD_MIN_BYTES;
constexpr uint32_t kGridCap = ROG_GRID_CAP;       // workgroups of one launch, at most
// Destination alignment at which a PEER payload's 16-byte body starts (a power
// of two >= 16): each wave's 1 KiB of stores then covers whole cache lines.
// 256 measured best (vs 16: +4.7 % on 8 x 64 MiB at offsets 1/3).
constexpr uint64_t kBodyAlign = ROG_BODY_ALIGN;
static_assert(kBodyAlign >= 16 && (kBodyAlign & (kBodyAlign - 1)) == 0, "body alignment");

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

// How the PEER kernel cuts a payload that is not 16-byte aligned on both sides
// (source address sa, destination address da, S bytes): bytes [0, lo) and
// [hi, S) move one by one; bytes [lo, hi) as aligned 16-byte stores whose data
// comes from the aligned source vectors that start at sa + lo - delta -- one per
// output vector when delta == 0, else two neighbours funnel-shifted by delta
// bytes.  The cut keeps every one of those aligned source vectors inside
// [sa, sa + S): vectors whose source blocks would reach outside move as bytes.
struct PeerSplit {
    uint64_t lo;      // first byte of the aligned body (da + lo is 16-byte aligned)
    uint64_t hi;      // end of the body; (hi - lo) % 16 == 0; lo == hi: no body
    uint32_t delta;   // (sa + lo) % 16
};

__host__ __device__ inline PeerSplit split_payload(uint64_t sa, uint64_t da, uint64_t S) {
    // The body starts at a kBodyAlign-aligned destination byte, so that the
    // 1 KiB a wave stores covers whole cache lines.
    const uint64_t to_line = (kBodyAlign - (da & (kBodyAlign - 1))) & (kBodyAlign - 1);
    const uint64_t h = to_line < S ? to_line : S;
    const uint64_t nb = (S - h) >> 4;                   // aligned output vectors after h
    const uint32_t delta = uint32_t((sa + h) & 15);
    uint64_t jlo = 0, jhi = nb;
    if (delta != 0) {
        // Output vector j reads source blocks at P0 + 16j and P0 + 16(j+1),
        // P0 = sa + h - delta; both must lie inside [sa, sa + S).
        const uint64_t p0 = sa + h - delta;
        jlo = p0 < sa ? 1 : 0;
        const uint64_t lim = (sa + S - p0) >> 4;
        jhi = lim > 1 ? lim - 1 : 0;
        if (jhi > nb) jhi = nb;
    }
    if (jhi <= jlo) return PeerSplit{S, S, 0};           // too small for a body
    return PeerSplit{h + 16 * jlo, h + 16 * jhi, delta};
}

// ---------------------------------------------------------------------------
// Kernel arguments
// ---------------------------------------------------------------------------

// FLAT: the whole output is one space of n_vec 16-byte vectors; vector v comes
// from payload r = v / vpr at index v - r*vpr.
struct FlatArgs {
    const void *src[kMaxPeers];
    void *out;
    uint32_t n_vec;
    uint32_t vpr;
    Divider div;
};

// PEER: each payload is its own copy job, cut by split_payload into a byte
// head, a body of aligned 16-byte stores (from aligned or funnel-shifted
// aligned source vectors) and a byte tail.
// Multi-WG: workgroup b works on payload b / blocks_per_peer; single-WG
// (blocks_per_peer unused): the one workgroup takes the payloads in turn.
struct PeerArgs {
    const void *src[kMaxPeers];
    void *out;
    uint64_t S;
    uint32_t blocks_per_peer;
    uint32_t W;
};

// One tensor of a batch.  Workgroups [first_block, first_block + n_blocks) of the
// launch belong to it.
struct BatchTensor {
    uint64_t out;
    uint64_t S;
    uint32_t first_block;
    uint32_t n_blocks;
    uint32_t flat;              // 1: FLAT tensor, 0: PEER tensor
    uint32_t vpr;               // FLAT: vectors per rank
    uint32_t n_vec;             // FLAT: W * vpr
    uint32_t blocks_per_peer;   // PEER
    Divider div;                // FLAT
};

struct BatchArgs {
    const void *src[kMaxBatchPtrs];   // tensor t's payloads at [t*W, t*W + W)
    BatchTensor t[kMaxBatch];
    uint32_t n;
    uint32_t W;
};

static_assert(sizeof(BatchArgs) <= 4096, "kernel arguments must stay below 4 KiB");

// ---------------------------------------------------------------------------
// Plans
// ---------------------------------------------------------------------------

struct Plan {
    rog_plan_info info;
    FlatArgs flat;
    PeerArgs peer;
};

// Validate and plan one gather (no HIP calls).
rog_status plan_gather(const void *const *srcs, int W, size_t S, const void *out,
                       rog_path path, Plan *plan);

// Validate and plan a batch (no HIP calls).  grid == 0 means nothing to launch.
// *nt_loads: the launch streams its loads past the caches.
rog_status plan_batch(const rog_gather_desc *descs, int n, int W, BatchArgs *args,
                      uint32_t *grid, bool *nt_loads);

}  // namespace rog
