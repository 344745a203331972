// Host fuzz of the planners (csrc/rog_plan.cpp) and the host/device helpers in
// csrc/rog_internal.h, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host side by tests/test_plan_fuzz.py: random pointers (aligned,
// misaligned, null, near the top of the address space, overlapping), sizes
// (0, small, huge, overflowing), W, element types and paths.  No pointer is
// ever dereferenced; the program checks that every call returns a status and,
// when it plans a launch, that the launch is well formed.  Exit 0 = clean.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rog_internal.h"

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t next() {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
uint64_t pick(uint64_t n) { return n ? next() % n : 0; }

const uint64_t kBase = uint64_t(1) << 40;

uint64_t rand_addr() {
    switch (pick(8)) {
    case 0: return 0;                                   // null
    case 1: return ~uint64_t(0) - pick(1 << 12);        // top of the address space
    case 2: return kBase + pick(64) * 16;               // aligned, near others
    default: return kBase + pick(uint64_t(1) << 24);    // anywhere nearby
    }
}

uint64_t rand_size() {
    switch (pick(8)) {
    case 0: return 0;
    case 1: return pick(64);
    case 2: return uint64_t(1) << pick(40);
    case 3: return ~uint64_t(0) - pick(16);             // overflowing
    case 4: return (uint64_t(1) << 36) / (1 + pick(64));
    default: return pick(uint64_t(1) << 22);
    }
}

int failures = 0;
void fail(const char *what, uint64_t i) {
    if (failures++ < 10) fprintf(stderr, "case %llu: %s\n", (unsigned long long)i, what);
}

bool status_ok(rog_status s) {
    return s == ROG_OK || s == ROG_ERR_INVALID_ARGUMENT || s == ROG_ERR_OVERLAP || s == ROG_ERR_TOO_LARGE;
}

}  // namespace

int main(int argc, char **argv) {
    const uint64_t n = argc > 1 ? strtoull(argv[1], nullptr, 10) : 200000;
    const void *srcs[rog::kMaxBatchPtrs];
    for (uint64_t i = 0; i < n; ++i) {
        const int W = int(pick(rog::kMaxPeers + 2));              // 0 .. kMaxPeers + 1
        const uint64_t S = rand_size();
        const uint64_t out = rand_addr();
        for (int r = 0; r < W && r < rog::kMaxBatchPtrs; ++r)
            srcs[r] = pick(4) == 0 ? reinterpret_cast<const void *>(out + uint64_t(r) * S)
                                   : reinterpret_cast<const void *>(rand_addr());
        const rog_path path = rog_path(pick(4));
        rog::Plan p;
        rog_status st = rog::plan_gather(srcs, W, size_t(S), reinterpret_cast<const void *>(out), path, &p);
        if (!status_ok(st)) fail("plan_gather: unknown status", i);
        if (st == ROG_OK && p.info.kernel != ROG_KERNEL_NONE &&
            (p.info.grid == 0 || p.info.block == 0 || uint64_t(p.info.grid) * p.info.block >= (uint64_t(1) << 32)))
            fail("plan_gather: bad launch", i);
        if (st == ROG_OK && p.info.kernel == ROG_KERNEL_FLAT) {
            // The chunks tile [0, n_vec) and, shifted, start on the output's lines.
            const rog::FlatArgs &a = p.flat;
            const uint32_t chunk = 64 * uint32_t(p.info.path == ROG_PATH_SINGLE_WG ? 1 : rog::kFlatUnroll);
            const uint32_t nc = rog::flat_chunk_count(a.n_vec, chunk, a.shift);
            if (a.shift > 7 || (a.n_vec >= (uint32_t(1) << 31) && a.shift) ||
                (p.info.path == ROG_PATH_SINGLE_WG && (a.shift || a.runs)))
                fail("plan_gather: FLAT shift", i);
            uint64_t bits = out | S;
            for (int r = 0; r < W; ++r) bits |= uint64_t(reinterpret_cast<uintptr_t>(srcs[r]));
            if (p.info.path == ROG_PATH_MULTI_WG && a.runs != ((bits & 127) != 0))
                fail("plan_gather: FLAT runs", i);
            const rog::ChunkSpan c0 = rog::flat_span(0, chunk, a.shift, a.n_vec);
            const rog::ChunkSpan cl = rog::flat_span(nc - 1, chunk, a.shift, a.n_vec);
            if (c0.b != 0 || c0.n == 0 || cl.n == 0 || uint64_t(cl.b) + cl.n != a.n_vec)
                fail("plan_gather: FLAT chunks", i);
            if (nc > 1 && a.n_vec < (uint32_t(1) << 31) && p.info.path == ROG_PATH_MULTI_WG &&
                ((out + 16 * uint64_t(rog::flat_span(1, chunk, a.shift, a.n_vec).b)) & 127) != 0)
                fail("plan_gather: FLAT chunk 1 off the output's lines", i);
        }

        const rog_dtype dt = rog_dtype(pick(4));                  // 3 is not a type
        st = rog::plan_reduce(srcs, W, size_t(S >> pick(4)), dt, reinterpret_cast<const void *>(out), path, &p);
        if (!status_ok(st)) fail("plan_reduce: unknown status", i);
        if (st == ROG_OK && p.info.kernel != ROG_KERNEL_NONE &&
            (p.info.grid == 0 || uint64_t(p.info.grid) * p.info.block >= (uint64_t(1) << 32)))
            fail("plan_reduce: bad launch", i);

        // batches
        const int nb = int(pick(rog::kMaxBatch + 2));
        const int Wb = 1 + int(pick(8));
        static rog_gather_desc gd[rog::kMaxBatch + 2];
        static rog_reduce_desc rd[rog::kMaxBatch + 2];
        static const void *bs[(rog::kMaxBatch + 2) * 8];
        for (int t = 0; t < nb; ++t) {
            for (int r = 0; r < Wb; ++r) bs[t * Wb + r] = reinterpret_cast<const void *>(kBase * (2 + t) + uint64_t(r) * (uint64_t(1) << 30) + pick(32));
            gd[t].srcs = bs + t * Wb;
            gd[t].out = reinterpret_cast<void *>(kBase * (2 + t) + (uint64_t(Wb) << 30) + pick(32));
            gd[t].bytes_per_rank = size_t(pick(3) ? pick(1 << 20) : rand_size());
            rd[t].srcs = bs + t * Wb;
            rd[t].out = gd[t].out;
            rd[t].count = size_t(pick(3) ? pick(1 << 20) : rand_size());
        }
        static rog::BatchArgs ba;
        static rog::ReduceBatchArgs ra;
        uint32_t grid = 0;
        bool nt = false, sh = false;
        st = rog::plan_batch(pick(16) ? gd : nullptr, nb, Wb, &ba, &grid, &nt);
        if (!status_ok(st)) fail("plan_batch: unknown status", i);
        if (st == ROG_OK && grid) {
            if (ba.n == 0 || ba.first[0] != 0) fail("plan_batch: first chunk", i);
            for (uint32_t k = 1; k < ba.n; ++k)
                if (ba.first[k] != ba.first[k - 1] + ba.t[k - 1].n_chunks) fail("plan_batch: chunk layout", i);
            if (ba.aligned_chunks > ba.n_chunks) fail("plan_batch: aligned chunks", i);
            for (uint32_t k = 0; k < ba.n; ++k) {
                const rog::BatchTensor &t = ba.t[k];
                if (t.flat && (t.shift != rog::flat_shift(t.out, t.n_vec) ||
                               t.n_chunks != rog::flat_chunk_count(t.n_vec, 64 * uint32_t(rog::kFlatUnroll), t.shift)))
                    fail("plan_batch: FLAT tensor chunks", i);
                if (ba.first[k] < ba.aligned_chunks) {     // round-robin group: all on 128-byte lines
                    uint64_t bits = t.out | t.S;
                    for (uint32_t r = 0; r < ba.W; ++r)
                        bits |= uint64_t(reinterpret_cast<uintptr_t>(ba.src[k * ba.W + r]));
                    if (!t.flat || (bits & 127) != 0) fail("plan_batch: aligned group", i);
                }
            }
        }
        st = rog::plan_reduce_batch(pick(16) ? rd : nullptr, nb, Wb, rog_dtype(pick(4)), &ra, &grid, &nt, &sh);
        if (!status_ok(st)) fail("plan_reduce_batch: unknown status", i);
        if (st == ROG_OK && grid) {
            for (uint32_t k = 1; k < ra.n; ++k)
                if (ra.first[k] != ra.first[k - 1] + ra.t[k - 1].n_chunks) fail("plan_reduce_batch: chunk layout", i);
        }

        // helpers shared with the kernels
        const rog::PeerSplit c = rog::split_payload(rand_addr(), S);
        if (c.lo > c.hi || c.hi > S) fail("split_payload: range", i);
        const uint32_t nc = uint32_t(next());
        if (nc) {
            const uint32_t b = uint32_t(pick(nc));
            if (rog::xcd_grouped(b, nc) >= nc) fail("xcd_grouped: range", i);
        }
        const uint32_t d = 1 + uint32_t(pick(0xFFFFFFFFu));
        (void)rog::make_divider(d);
    }
    printf("plan_fuzz: %llu cases, %d failures\n", (unsigned long long)n, failures);
    return failures ? 1 : 0;
}
