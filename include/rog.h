/*
 * rog.h -- rank-ordered gather (rog) and rank-ordered sum for MI355X (gfx950,
 * CDNA4).
 *
 * C ABI of librog.so.  Plain C types, device pointers and sizes; no PyTorch
 * types.  Every entry point below is implemented by hand-written HIP kernels in
 * deterministic_collective_movement_amd/csrc/.
 *
 * The operation is the copy at the heart of a deterministic all-gather
 * (RL-Align/RL-Kernel PR #491, "perf(cuda): vectorize the deterministic
 * all-gather copy and right-size its single-block path", section "What", the
 * copy_rank_ordered bullet): W payloads of S bytes are concatenated in rank
 * order, so that
 *
 *     out[r*S + i] = srcs[r][i]     for 0 <= r < W, 0 <= i < S,
 *
 * byte-identical to a plain concatenation for every alignment and size.  On one
 * GPU the W peers' payloads are W caller-owned device buffers.  Beside it,
 * rog_reduce computes the rank-ordered sum at the heart of the same pages'
 * deterministic all-reduce and reduce-scatter (declared and defined below).
 *
 * Common rules for every entry point:
 *  - Pointers to data (srcs[r], out, the descriptors' buffers) are device
 *    pointers readable/writable by kernels on the current HIP device.  They are
 *    not checked for residency; the Python binding checks tensor devices.
 *  - Host arrays (the srcs array, the descriptor array) are read only during
 *    the call; their contents are copied into the kernel arguments.
 *  - The caller owns every buffer; buffers must stay valid until the work
 *    enqueued on `stream` has completed.
 *  - All argument errors are returned before anything is enqueued: on error no
 *    byte of any output is written and no HIP call has been made.
 *  - Success means the work has been enqueued on `stream` (asynchronous), as
 *    exactly one kernel launch; nothing else is enqueued, so calls can be
 *    captured into a HIP graph.
 *  - The library allocates no device or host memory, keeps no state except a
 *    thread-local copy of the last HIP error, and may be called from any thread.
 *  - Bytes outside the output range (out, W*S bytes for a gather; count
 *    elements for a sum) are never written.  Source bytes are never written,
 *    except by an in-place call where out is itself a source.  Every read lies
 *    inside a source range (S bytes for a gather, count elements for a sum) or,
 *    in the forms flagged ROG_PLAN_SHIFTED_LOADS, inside an aligned 16-byte
 *    granule that holds bytes of one (so within that range's own pages); the
 *    bytes read beyond a range are never used.
 */
#ifndef ROG_H
#define ROG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROG_API __attribute__((visibility("default")))

typedef enum {
    ROG_OK = 0,
    ROG_ERR_INVALID_ARGUMENT = 1, /* null pointer, W out of range, n < 0, bad path  */
    ROG_ERR_OVERLAP = 2,          /* a source range partially overlaps the output   */
    ROG_ERR_TOO_LARGE = 3,        /* size overflow or a limit below exceeded        */
    ROG_ERR_LAUNCH = 4            /* the kernel launch failed; see rog_last_hip_error */
} rog_status;

typedef enum {
    ROG_PATH_AUTO = 0,       /* single-WG iff W*S <= rog_single_wg_max_bytes()  */
    ROG_PATH_SINGLE_WG = 1,  /* one workgroup of up to 1024 threads does it all */
    ROG_PATH_MULTI_WG = 2    /* a grid of small workgroups sized from the work      */
} rog_path;

typedef enum {
    ROG_KERNEL_NONE = 0,     /* nothing to copy (S == 0): nothing is launched       */
    ROG_KERNEL_FLAT = 1,     /* a single loop over every payload's 16-byte vectors  */
    ROG_KERNEL_PEER = 2,     /* per payload: byte head, 16-byte body (aligned
                                stores, loads at any alignment), byte tail          */
    ROG_KERNEL_REDUCE = 3    /* rank-ordered sum: element head, 16-byte body of
                                aligned stores (loads at any element alignment),
                                element tail                                         */
} rog_kernel;

/* Element types of the rank-ordered sum. */
typedef enum {
    ROG_DTYPE_F32 = 0,       /* IEEE binary32, 4 bytes                               */
    ROG_DTYPE_BF16 = 1,      /* bfloat16 (top 16 bits of a binary32), 2 bytes       */
    ROG_DTYPE_F16 = 2        /* IEEE binary16, 2 bytes                               */
} rog_dtype;

/* One tensor of a batch: W source pointers, its output, its per-rank bytes. */
typedef struct {
    const void *const *srcs;   /* W device pointers (host array)                 */
    void *out;                 /* device pointer to W * bytes_per_rank bytes     */
    size_t bytes_per_rank;     /* S of this tensor; 0 is allowed (nothing copied) */
} rog_gather_desc;

/* The launch a call would make (rog_plan), for tests and inspection. */
typedef struct {
    int32_t path;              /* resolved rog_path: SINGLE_WG or MULTI_WG (AUTO never) */
    int32_t kernel;            /* rog_kernel                                            */
    uint32_t grid;             /* workgroups launched (0 when kernel == NONE)           */
    uint32_t block;            /* threads per workgroup                                 */
    uint64_t vec_ok_mask;      /* PEER kernel: bit r set iff srcs[r] and out + r*S are
                                  both 16-byte aligned (where the pages' fallback
                                  copies vectors); informational, every payload
                                  gets a 16-byte body whatever its alignment       */
    uint64_t units;            /* FLAT: 16-byte vectors W*S/16; PEER: bytes W*S;
                                  REDUCE: elements per payload                        */
    uint32_t peer_magic;       /* FLAT: floor(v / (S/16)) = (t + ((v - t) >> peer_sh1))  */
    uint32_t peer_sh1;         /*       >> peer_sh2 with t = mulhi32(v, peer_magic),     */
    uint32_t peer_sh2;         /*       exact for every 32-bit v                         */
    uint32_t flags;            /* ROG_PLAN_* bits                                       */
} rog_plan_info;

/* rog_plan_info.flags: the kernel's 16-byte loads are non-temporal (streamed
 * past the caches); set when the W*S source bytes are too many for the 256 MB
 * Infinity Cache to serve repeated calls well: from 128 MiB, for gathers and
 * sums, single or batched.  16-byte stores are always non-temporal; a
 * gather's are also written through the L2 caches at device scope.  Affects
 * speed only. */
#define ROG_PLAN_NT_LOADS 1u
/* rog_plan_info.flags: the multi-workgroup PEER or REDUCE kernel reads at least
 * one source body as aligned 16-byte granules, each lane taking the granule
 * after its own from the next lane.  Only with ROG_PLAN_NT_LOADS.  PEER: set
 * when a payload's body (from the first 256-byte boundary of its output) is
 * not empty and its source sits an odd or 2-mod-4 number of bytes past a
 * 16-byte granule there.  REDUCE: set with ROG_PLAN_NT_LOADS, for every
 * source.  Affects speed only; the bytes are the same. */
#define ROG_PLAN_SHIFTED_LOADS 2u

/*
 * rog_gather -- out[r*S + i] = srcs[r][i] for r < W, i < S, enqueued on `stream`.
 *
 * srcs            host array of W device pointers (payload r = rank r).
 * W               number of payloads, 1 <= W <= rog_max_peers().
 * bytes_per_rank  S, the byte size of every payload (one S for all, as in an
 *                 all-gather; PR #491 "What": one byte count per rank).
 * out             device pointer to W*S writable bytes.
 * stream          HIP stream (0 = null stream) of the current device.
 *
 * Path: single-workgroup when W*S <= rog_single_wg_max_bytes(), multi-workgroup
 * otherwise (PR #491 "What", kAllGatherSingleBlockMaxBytes bullet: with one
 * block doing all the work the gather is faster only for small outputs; the
 * crossover here is measured on gfx950).  Kernel: FLAT when out, S and every
 * srcs[r] are 16-byte aligned, else PEER (PR #491 "What", copy_rank_ordered).
 * Multi-workgroup FLAT moves 1 KiB chunks, the first one shorter by
 * k = (out mod 128) / 16 vectors so that the rest start on out's 128-byte
 * lines (k = 0 from 2^31 vectors on): grid = ceil((W*S/16 + k) / 64) one-wave
 * workgroups (capped).
 * PEER copies each payload as a byte head up to a 256-byte boundary of its
 * destination, a body of aligned 16-byte stores, each fed by one 16-byte load
 * of the source bytes at the same payload offset (at any source alignment; or,
 * where the loads stream past the caches, by aligned granules shared between
 * neighbouring lanes, see ROG_PLAN_SHIFTED_LOADS), and a byte tail: the pages'
 * fallback (vector copies only where both sides are aligned, bytes otherwise)
 * extended to misaligned payloads, same bytes as a byte-by-byte copy.
 *
 * Errors (nothing enqueued):
 *   ROG_ERR_INVALID_ARGUMENT  srcs NULL; W < 1 or W > rog_max_peers(); S > 0 and
 *                             out or some srcs[r] NULL.
 *   ROG_ERR_OVERLAP           some [srcs[r], srcs[r]+S) overlaps [out, out+W*S)
 *                             other than exactly (srcs[r] == out + r*S, in place).
 *   ROG_ERR_TOO_LARGE         W*S overflows, or W*S >= 2^36 (64 GiB).
 *   ROG_ERR_LAUNCH            hipLaunchKernel failed (rog_last_hip_error()).
 * S == 0: ROG_OK, nothing enqueued.  Sources may alias one another.
 */
ROG_API rog_status rog_gather(const void *const *srcs, int W, size_t bytes_per_rank,
                              void *out, hipStream_t stream);

/*
 * rog_gather_ex -- rog_gather with the path forced.  ROG_PATH_AUTO behaves
 * exactly like rog_gather.  Forcing SINGLE_WG or MULTI_WG changes only the launch
 * shape, never the bytes written; it lets tests reach each path on every case
 * (the pages' review of the size test asks that the otherwise unreachable
 * single-block branch be covered).  path outside rog_path: INVALID_ARGUMENT.
 */
ROG_API rog_status rog_gather_ex(const void *const *srcs, int W, size_t bytes_per_rank,
                                 void *out, hipStream_t stream, rog_path path);

/*
 * rog_gather_many -- n independent gathers sharing W, in one kernel launch.
 * Tensor t: out_t[r*S_t + i] = srcs_t[r][i].  The pages' all_gather_many
 * (PR #491 review threads on the benchmark) gathers a list of tensors with a
 * single synchronisation of the ranks and without copying them into one
 * buffer first; here every tensor keeps its own caller-provided
 * output and its own alignment class (flat or per-peer).
 *
 * descs  host array of n descriptors (each with a host array of W pointers).
 * n      0 <= n <= rog_max_batch(); n == 0 or all S_t == 0: ROG_OK, nothing
 *        enqueued.  n*W must not exceed rog_max_batch_pointers().
 * Errors: as rog_gather for each tensor; outputs of different tensors must not
 * overlap each other (ROG_ERR_OVERLAP), and a tensor's sources must not overlap
 * another tensor's output; limits exceeded: ROG_ERR_TOO_LARGE.
 */
ROG_API rog_status rog_gather_many(const rog_gather_desc *descs, int n, int W,
                                   hipStream_t stream);

/*
 * rog_plan -- validate exactly as rog_gather_ex and describe the launch it would
 * make, without any HIP call.  info must be non-NULL (else INVALID_ARGUMENT).
 * Pointers are only inspected as addresses.
 */
ROG_API rog_status rog_plan(const void *const *srcs, int W, size_t bytes_per_rank,
                            const void *out, rog_path path, rog_plan_info *info);

/* Output bytes W*S up to which ROG_PATH_AUTO takes the single-workgroup path
 * (inclusive), measured on MI355X: 32 KiB.  The pages' counterpart is
 * kAllGatherSingleBlockMaxBytes (RL-Align/RL-Kernel PR #491, section "What",
 * the kAllGatherSingleBlockMaxBytes bullet): one block copying the whole
 * output wins only for small outputs, the bound compares output bytes, and its
 * B200 value (64 KiB) was found by measuring both paths, as this one was on
 * gfx950.  Never fails; a constant of the build. */
ROG_API size_t rog_single_wg_max_bytes(void);

/*
 * rog_reduce -- the rank-ordered sum of W payloads of `count` elements:
 *
 *     out[i] = round( ((x_0[i] + x_1[i]) + x_2[i]) + ... + x_{W-1}[i] ),
 *
 * x_r = srcs[r], the sum taken in rank order with every addition an IEEE
 * binary32 addition rounded to nearest-even, bf16 and binary16 elements
 * widened to binary32 exactly, the first term taken as it is (a lone -0 stays
 * -0), and the result rounded once to `dtype` (nearest-even; binary16 with
 * gradual underflow and overflow to infinity; a NaN stays a NaN, its payload
 * unspecified).  Every element is summed by one thread in that fixed order, so
 * the result is the same bits on every call, whatever the launch shape.
 *
 * This is the reduction at the heart of the pages' deterministic all_reduce
 * and reduce_scatter (RL-Align/RL-Kernel PR #491, "Not in this PR": their
 * single-block paths grow with size as the gather's did; 523 us at 256 KiB
 * per rank on 8 GPUs).  The pages print no arithmetic: they call their backend
 * a fixed tree (the author's replies on the benchmark's recorded backend)
 * without saying which; the left-deep rank-order chain in binary32 above is
 * this library's reading of it.  On one GPU the W ranks are W caller-owned
 * device buffers: an all-reduce is rog_reduce over the W inputs, rank r's share
 * of a reduce-scatter is rog_reduce over the W inputs' r-th shards.
 *
 * srcs    host array of W device pointers, each to `count` elements of dtype,
 *         aligned to the element size (any alignment beyond that).
 * W       1 <= W <= rog_max_peers().
 * count   elements per payload (and in out).
 * dtype   ROG_DTYPE_F32, ROG_DTYPE_BF16 or ROG_DTYPE_F16.
 * out     device pointer to `count` writable elements, element-aligned.  out
 *         may be exactly one (or several) of the srcs (in place); any other
 *         overlap with a source is an error.  Sources may alias each other.
 * stream  HIP stream of the current device.
 *
 * Path: single-workgroup when the source bytes W * count * element size are
 * <= rog_reduce_single_wg_max_bytes() (inclusive, measured on gfx950; the
 * pages test their all-reduce bound on input bytes too), multi-workgroup
 * otherwise.
 * Errors (nothing enqueued):
 *   ROG_ERR_INVALID_ARGUMENT  srcs NULL; W out of range; dtype or path unknown;
 *                             count > 0 and out or some srcs[r] NULL or not
 *                             aligned to the element size.
 *   ROG_ERR_OVERLAP           a source overlaps out other than exactly.
 *   ROG_ERR_TOO_LARGE         count * element size overflows or is >= 2^36.
 *   ROG_ERR_LAUNCH            hipLaunchKernel failed (rog_last_hip_error()).
 * count == 0: ROG_OK, nothing enqueued.
 */
ROG_API rog_status rog_reduce(const void *const *srcs, int W, size_t count, rog_dtype dtype,
                              void *out, hipStream_t stream);

/* rog_reduce with the path forced (changes the launch shape, never the bits). */
ROG_API rog_status rog_reduce_ex(const void *const *srcs, int W, size_t count, rog_dtype dtype,
                                 void *out, hipStream_t stream, rog_path path);

/* Validate exactly as rog_reduce_ex and describe the launch, without any HIP
 * call (kernel ROG_KERNEL_REDUCE, units = count). */
ROG_API rog_status rog_reduce_plan(const void *const *srcs, int W, size_t count, rog_dtype dtype,
                                   const void *out, rog_path path, rog_plan_info *info);

/* Source bytes (W * count * element size) up to which ROG_PATH_AUTO runs
 * rog_reduce on one workgroup (inclusive), measured on MI355X: 64 KiB.  The
 * bound is compared with input bytes because the pages' all-reduce /
 * reduce-scatter fast-path bound is (RL-Align/RL-Kernel PR #491, the author's
 * reply on the benchmark's --size-bytes: the 256 KiB threshold is tested on
 * the per-rank input, world size x the output for reduce_scatter).  Never
 * fails; a constant of the build. */
ROG_API size_t rog_reduce_single_wg_max_bytes(void);

/* One tensor of a batched sum: W source pointers, its output, its count. */
typedef struct {
    const void *const *srcs;   /* W device pointers (host array)                  */
    void *out;                 /* device pointer to `count` elements              */
    size_t count;              /* elements of this tensor; 0 is allowed           */
} rog_reduce_desc;

/*
 * rog_reduce_many -- n independent rank-ordered sums sharing W and dtype, in one
 * kernel launch: tensor t gets out_t[i] = the rank-ordered sum of srcs_t[r][i]
 * (exactly as rog_reduce).  The pages' reduce_scatter_many / all_gather_many
 * (PR #491, "Tests" and the review threads on the benchmark) batch a list of
 * tensors under a single synchronisation of the ranks; here every tensor keeps its own
 * caller-provided output and the whole batch is one launch.
 *
 * descs  host array of n descriptors (each with a host array of W pointers).
 * n      0 <= n <= rog_max_batch(); n == 0 or all counts 0: ROG_OK, nothing
 *        enqueued.  n*W must not exceed rog_max_batch_pointers().
 * Errors: as rog_reduce for each tensor; besides, a tensor's output must not
 * overlap another tensor's output or sources (ROG_ERR_OVERLAP); limits
 * exceeded: ROG_ERR_TOO_LARGE.  Always the multi-workgroup shape.
 */
ROG_API rog_status rog_reduce_many(const rog_reduce_desc *descs, int n, int W, rog_dtype dtype,
                                   hipStream_t stream);

/* Largest W accepted: 64, the capacity of the kernel arguments, which carry
 * every source pointer.  The pages' collectives run over a same-host group of
 * at most eight ranks (RL-Align/RL-Kernel PR #491, "Security Architecture
 * Review", "Security Blast Radius"), so every group size they use fits.
 * Never fails; a constant of the build. */
ROG_API int rog_max_peers(void);

/* Largest n accepted by rog_gather_many, and the largest n*W. */
ROG_API int rog_max_batch(void);
ROG_API int rog_max_batch_pointers(void);

/* hipError_t of the last failed launch on this thread (0 if none). */
ROG_API int rog_last_hip_error(void);

/* Static, human-readable name of a status code ("ROG_OK", ...). */
ROG_API const char *rog_status_string(rog_status s);

#ifdef __cplusplus
}
#endif

#endif /* ROG_H */
