// Host shim over the batch planners (plan_batch, plan_reduce_batch in
// csrc/rog_plan.cpp), so the CPU tests check the chunk layout the batch
// kernels receive: tensor order, first chunks, chunk counts, kernel choice.
#include <string.h>

#include "rog_internal.h"

// Gather batch: per planned tensor k (k < *n_out): out[k], S[k], flat[k],
// n_chunks[k], first[k], and its W source pointers at srcs[k * W ...].
// meta: n_chunks, aligned_chunks, grid, nt_loads.
extern "C" int rog_test_plan_batch(const rog_gather_desc *descs, int n, int W, uint32_t *n_out,
                                   uint64_t *out, uint64_t *S, uint32_t *flat, uint32_t *n_chunks,
                                   uint32_t *first, uint64_t *srcs, uint32_t *meta) {
    static rog::BatchArgs a;
    uint32_t grid = 0;
    bool nt = false;
    const rog_status st = rog::plan_batch(descs, n, W, &a, &grid, &nt);
    *n_out = 0;
    if (st != ROG_OK) return int(st);
    *n_out = a.n;
    for (uint32_t k = 0; k < a.n; ++k) {
        out[k] = a.t[k].out;
        S[k] = a.t[k].S;
        flat[k] = a.t[k].flat;
        n_chunks[k] = a.t[k].n_chunks;
        first[k] = a.first[k];
        for (int r = 0; r < W; ++r) srcs[k * uint32_t(W) + uint32_t(r)] = uint64_t(uintptr_t(a.src[k * uint32_t(W) + uint32_t(r)]));
    }
    meta[0] = a.n_chunks;
    meta[1] = a.aligned_chunks;
    meta[2] = grid;
    meta[3] = nt ? 1u : 0u;
    return 0;
}

// Sum batch: per planned tensor k: out[k], count[k], n_chunks[k], first[k].
// meta: n_chunks, grid, nt_loads, granule form.
extern "C" int rog_test_plan_reduce_batch(const rog_reduce_desc *descs, int n, int W, int dtype,
                                          uint32_t *n_out, uint64_t *out, uint64_t *count,
                                          uint32_t *n_chunks, uint32_t *first, uint32_t *meta) {
    static rog::ReduceBatchArgs a;
    uint32_t grid = 0;
    bool nt = false, sh = false;
    const rog_status st = rog::plan_reduce_batch(descs, n, W, rog_dtype(dtype), &a, &grid, &nt, &sh);
    *n_out = 0;
    if (st != ROG_OK) return int(st);
    *n_out = a.n;
    for (uint32_t k = 0; k < a.n; ++k) {
        out[k] = a.t[k].out;
        count[k] = a.t[k].count;
        n_chunks[k] = a.t[k].n_chunks;
        first[k] = a.first[k];
    }
    meta[0] = a.n_chunks;
    meta[1] = grid;
    meta[2] = nt ? 1u : 0u;
    meta[3] = sh ? 1u : 0u;
    return 0;
}

// The batched gather's chunk -> tensor lookup (batch_tensor over the planner's
// bucket table) for chunks[0 .. n_query) of a gather batch: the tensor index
// of each, written to tensor[].  Returns the planner's status.
extern "C" int rog_test_batch_lookup(const rog_gather_desc *descs, int n, int W, const uint32_t *chunks,
                                     uint32_t n_query, uint32_t *tensor, uint32_t *shift) {
    static rog::BatchArgs a;
    uint32_t grid = 0;
    bool nt = false;
    const rog_status st = rog::plan_batch(descs, n, W, &a, &grid, &nt);
    if (st != ROG_OK) return int(st);
    *shift = a.lookup.shift;
    for (uint32_t i = 0; i < n_query; ++i) tensor[i] = rog::batch_tensor(a.first, a.lookup, chunks[i]);
    return 0;
}

// The batched sums' lookup (search_tensor over the planner's first chunks),
// likewise.
extern "C" int rog_test_reduce_batch_lookup(const rog_reduce_desc *descs, int n, int W, int dtype,
                                            const uint32_t *chunks, uint32_t n_query, uint32_t *tensor) {
    static rog::ReduceBatchArgs a;
    uint32_t grid = 0;
    bool nt = false, sh = false;
    const rog_status st = rog::plan_reduce_batch(descs, n, W, rog_dtype(dtype), &a, &grid, &nt, &sh);
    if (st != ROG_OK) return int(st);
    for (uint32_t i = 0; i < n_query; ++i) tensor[i] = rog::search_tensor(a.first, a.n, chunks[i]);
    return 0;
}

// The sum's granule group by W (sources whose granules a lane keeps in flight).
extern "C" uint32_t rog_test_sum_granule_group(uint32_t W) { return rog::sum_granule_group(W); }
