/*
 * abi_c_check.c -- a plain C consumer of librog.so (include/rog.h): no Python,
 * no PyTorch.  It allocates device memory with the HIP runtime, gathers on a
 * stream it created, copies back, and compares every byte -- guards around
 * each output included -- with the CPU oracle (oracle/rog_oracle.c, linked in).
 * Built by the package build step; run by tests/test_abi_c_gpu.py.
 *
 * Cases: aligned (flat) and misaligned (per-payload) gathers on every path,
 * a batch of three tensors in one launch, S = 0, and the argument errors that
 * must be reported before anything is enqueued; rank-ordered sums (bf16 and
 * binary32, every path, element offsets, in place) against the oracle's sum,
 * and a batch of binary16 sums in one launch; both batched calls captured
 * into a HIP graph, which must hold exactly one node, a kernel launch, and
 * whose replays must match the oracle; the plans' cache-policy and
 * shared-granule flags.
 * Exit status 0 = every check passed; the first failure is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rog.h"

void rog_oracle_gather(const unsigned char *const *srcs, int W, size_t S, unsigned char *out);
void rog_oracle_reduce_f32(const float *const *srcs, int W, size_t count, float *out);
void rog_oracle_reduce_bf16(const uint16_t *const *srcs, int W, size_t count, uint16_t *out);
void rog_oracle_reduce_f16(const uint16_t *const *srcs, int W, size_t count, uint16_t *out);

#define GUARD 64
#define FILL 0xA5

static int failures = 0;

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "HIP error %d at %s:%d: %s\n", (int)e_, __FILE__,     \
                    __LINE__, #x);                                                \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

static unsigned char byte_at(unsigned seed, size_t i) {
    unsigned x = seed * 2654435761u + (unsigned)i * 40503u;
    x ^= x >> 13;
    x *= 0x5bd1e995u;
    return (unsigned char)(x >> 24);
}

/* The nodes of a captured graph: how many in all, how many kernel launches. */
static int kernel_nodes(hipGraph_t g, size_t *total) {
    size_t n = 0;
    CHECK_HIP(hipGraphGetNodes(g, NULL, &n));
    hipGraphNode_t *nodes = (hipGraphNode_t *)malloc((n ? n : 1) * sizeof *nodes);
    CHECK_HIP(hipGraphGetNodes(g, nodes, &n));
    int k = 0;
    for (size_t i = 0; i < n; ++i) {
        hipGraphNodeType t;
        CHECK_HIP(hipGraphNodeGetType(nodes[i], &t));
        if (t == hipGraphNodeTypeKernel) ++k;
    }
    free(nodes);
    *total = n;
    return k;
}

/* A batched call captured from `st`: exactly one node, a kernel launch (the
 * pages' all_gather_many synchronises the ranks once for the whole list,
 * RL-Align/RL-Kernel PR #491, review thread on the benchmark's all_gather_many
 * row; here the whole list is one launch).  Returns the instantiated graph,
 * or NULL after counting a failure. */
static hipGraphExec_t capture_one_launch(hipStream_t st, int is_sum, const void *descs, int n, int W,
                                         rog_dtype dtype, const char *what) {
    hipGraph_t g;
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    const rog_status s = is_sum ? rog_reduce_many((const rog_reduce_desc *)descs, n, W, dtype, st)
                                : rog_gather_many((const rog_gather_desc *)descs, n, W, st);
    CHECK_HIP(hipStreamEndCapture(st, &g));
    size_t total = 0;
    const int k = kernel_nodes(g, &total);
    if (s != ROG_OK || k != 1 || total != 1) {
        fprintf(stderr, "FAIL %s: captured status %s, %zu nodes, %d kernel nodes (want 1, 1)\n", what,
                rog_status_string(s), total, k);
        ++failures;
        CHECK_HIP(hipGraphDestroy(g));
        return NULL;
    }
    hipGraphExec_t ex;
    CHECK_HIP(hipGraphInstantiate(&ex, g, NULL, NULL, 0));
    CHECK_HIP(hipGraphDestroy(g));
    return ex;
}

/* One gather of W payloads of S bytes at the given offsets, on `path`. */
static void gather_case(int W, size_t S, size_t in_off, size_t out_off, rog_path path,
                        hipStream_t st) {
    unsigned char *host_src[64];
    unsigned char *dev_buf[64];
    const void *dev_src[64];
    size_t sbytes = GUARD + in_off + S + GUARD;
    for (int r = 0; r < W; ++r) {
        host_src[r] = (unsigned char *)malloc(sbytes);
        memset(host_src[r], FILL, sbytes);
        for (size_t i = 0; i < S; ++i) host_src[r][GUARD + in_off + i] = byte_at(17u * r + 3u, i);
        CHECK_HIP(hipMalloc((void **)&dev_buf[r], sbytes));
        CHECK_HIP(hipMemcpy(dev_buf[r], host_src[r], sbytes, hipMemcpyHostToDevice));
        dev_src[r] = dev_buf[r] + GUARD + in_off;
    }
    size_t obytes = GUARD + out_off + (size_t)W * S + GUARD;
    unsigned char *want = (unsigned char *)malloc(obytes);
    unsigned char *got = (unsigned char *)malloc(obytes);
    memset(want, FILL, obytes);
    const unsigned char *hs[64];
    for (int r = 0; r < W; ++r) hs[r] = host_src[r] + GUARD + in_off;
    rog_oracle_gather(hs, W, S, want + GUARD + out_off);

    unsigned char *dev_out;
    CHECK_HIP(hipMalloc((void **)&dev_out, obytes));
    CHECK_HIP(hipMemset(dev_out, FILL, obytes));
    rog_status s = rog_gather_ex(dev_src, W, S, dev_out + GUARD + out_off, st, path);
    if (s != ROG_OK) {
        fprintf(stderr, "FAIL W=%d S=%zu in=%zu out=%zu path=%d: %s\n", W, S, in_off, out_off,
                (int)path, rog_status_string(s));
        ++failures;
    } else {
        CHECK_HIP(hipStreamSynchronize(st));
        CHECK_HIP(hipMemcpy(got, dev_out, obytes, hipMemcpyDeviceToHost));
        if (memcmp(got, want, obytes) != 0) {
            size_t k = 0;
            while (got[k] == want[k]) ++k;
            fprintf(stderr, "FAIL W=%d S=%zu in=%zu out=%zu path=%d: byte %zu got %d want %d\n", W, S,
                    in_off, out_off, (int)path, k, got[k], want[k]);
            ++failures;
        }
    }
    CHECK_HIP(hipFree(dev_out));
    for (int r = 0; r < W; ++r) {
        CHECK_HIP(hipFree(dev_buf[r]));
        free(host_src[r]);
    }
    free(want);
    free(got);
}

static void batch_case(hipStream_t st) {
    enum { N = 3, W = 4 };
    const size_t sizes[N] = {4096, 1001, 65536 + 7};
    const size_t offs[N] = {0, 3, 1};
    unsigned char *hsrc[N][W], *dsrc[N][W], *dout[N], *want[N], *got[N];
    const void *ptrs[N][W];
    rog_gather_desc desc[N];
    for (int t = 0; t < N; ++t) {
        const size_t S = sizes[t];
        for (int r = 0; r < W; ++r) {
            hsrc[t][r] = (unsigned char *)malloc(S);
            for (size_t i = 0; i < S; ++i) hsrc[t][r][i] = byte_at(101u * t + r, i);
            CHECK_HIP(hipMalloc((void **)&dsrc[t][r], S + offs[t]));
            CHECK_HIP(hipMemcpy(dsrc[t][r] + offs[t], hsrc[t][r], S, hipMemcpyHostToDevice));
            ptrs[t][r] = dsrc[t][r] + offs[t];
        }
        want[t] = (unsigned char *)malloc(W * S);
        got[t] = (unsigned char *)malloc(W * S);
        rog_oracle_gather((const unsigned char *const *)hsrc[t], W, S, want[t]);
        CHECK_HIP(hipMalloc((void **)&dout[t], W * S + 5));
        desc[t].srcs = ptrs[t];
        desc[t].out = dout[t] + 5 * (t % 2);
        desc[t].bytes_per_rank = S;
    }
    rog_status s = rog_gather_many(desc, N, W, st);
    if (s != ROG_OK) {
        fprintf(stderr, "FAIL batch: %s\n", rog_status_string(s));
        ++failures;
    } else {
        CHECK_HIP(hipStreamSynchronize(st));
        for (int t = 0; t < N; ++t) {
            CHECK_HIP(hipMemcpy(got[t], desc[t].out, W * sizes[t], hipMemcpyDeviceToHost));
            if (memcmp(got[t], want[t], W * sizes[t]) != 0) {
                fprintf(stderr, "FAIL batch tensor %d\n", t);
                ++failures;
            }
        }
        /* The same call captured: one kernel node; three replays, each over
         * outputs cleared by eager work in between, each compared in full. */
        hipGraphExec_t ex = capture_one_launch(st, 0, desc, N, W, ROG_DTYPE_F32, "batch graph");
        for (int rep = 0; ex && rep < 3; ++rep) {
            for (int t = 0; t < N; ++t) CHECK_HIP(hipMemset(dout[t], FILL, W * sizes[t] + 5));
            CHECK_HIP(hipGraphLaunch(ex, st));
            CHECK_HIP(hipStreamSynchronize(st));
            for (int t = 0; t < N; ++t) {
                CHECK_HIP(hipMemcpy(got[t], desc[t].out, W * sizes[t], hipMemcpyDeviceToHost));
                if (memcmp(got[t], want[t], W * sizes[t]) != 0) {
                    fprintf(stderr, "FAIL batch graph replay %d tensor %d\n", rep, t);
                    ++failures;
                }
            }
        }
        if (ex) CHECK_HIP(hipGraphExecDestroy(ex));
    }
    for (int t = 0; t < N; ++t) {
        for (int r = 0; r < W; ++r) {
            CHECK_HIP(hipFree(dsrc[t][r]));
            free(hsrc[t][r]);
        }
        CHECK_HIP(hipFree(dout[t]));
        free(want[t]);
        free(got[t]);
    }
}

static void expect_status(rog_status got, rog_status want, const char *what) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: got %s want %s\n", what, rog_status_string(got), rog_status_string(want));
        ++failures;
    }
}

static void error_cases(hipStream_t st) {
    unsigned char *buf;
    CHECK_HIP(hipMalloc((void **)&buf, 4096));
    CHECK_HIP(hipMemset(buf, FILL, 4096));
    const void *two[2] = {buf + 1024, buf + 2048};
    expect_status(rog_gather(NULL, 2, 16, buf, st), ROG_ERR_INVALID_ARGUMENT, "NULL srcs");
    expect_status(rog_gather(two, 0, 16, buf, st), ROG_ERR_INVALID_ARGUMENT, "W = 0");
    expect_status(rog_gather(two, 2, 16, NULL, st), ROG_ERR_INVALID_ARGUMENT, "NULL out");
    expect_status(rog_gather(two, 2, 1024, buf + 512, st), ROG_ERR_OVERLAP, "partial overlap");
    expect_status(rog_gather(two, 2, (size_t)1 << 40, buf, st), ROG_ERR_TOO_LARGE, "too large");
    expect_status(rog_gather_ex(two, 2, 16, buf, st, (rog_path)9), ROG_ERR_INVALID_ARGUMENT, "bad path");
    expect_status(rog_gather(two, 2, 0, buf, st), ROG_OK, "S = 0");
    /* nothing above may have written a byte */
    unsigned char host[4096];
    CHECK_HIP(hipStreamSynchronize(st));
    CHECK_HIP(hipMemcpy(host, buf, 4096, hipMemcpyDeviceToHost));
    for (int i = 0; i < 4096; ++i)
        if (host[i] != FILL) {
            fprintf(stderr, "FAIL an error path wrote byte %d\n", i);
            ++failures;
            break;
        }
    CHECK_HIP(hipFree(buf));
}

/* Element i of payload r for the sums: finite bf16 / binary32 values spread over
 * a few binades, of both signs. */
static uint32_t elem_bits(unsigned seed, size_t i, int bf16) {
    unsigned x = seed * 2246822519u + (unsigned)i * 3266489917u;
    x ^= x >> 15;
    x *= 0x2c1b3c6du;
    x ^= x >> 12;
    const uint32_t sign = (x & 1u) << 31;
    const uint32_t expo = 120u + ((x >> 1) % 12u);          /* 2^-7 .. 2^4 */
    const uint32_t mant = (x >> 5) & 0x7FFFFFu;
    const uint32_t f = sign | (expo << 23) | mant;
    return bf16 ? (f >> 16) : f;
}

/* One sum of W payloads of n elements; payload r at element offset r % 4 of its
 * buffer, out at element offset out_off (or out = payload `in_place`). */
static void reduce_case(int W, size_t n, int bf16, size_t out_off, int in_place, rog_path path, hipStream_t st) {
    const size_t es = bf16 ? 2 : 4;
    unsigned char *host[64], *dev[64];
    const void *dsrc[64];
    const void *hsrc[64];
    for (int r = 0; r < W; ++r) {
        const size_t off = (size_t)(r % 4) * es;
        host[r] = (unsigned char *)malloc(off + n * es + 16);
        for (size_t i = 0; i < n; ++i) {
            const uint32_t b = elem_bits(31u * (unsigned)r + 7u, i, bf16);
            memcpy(host[r] + off + i * es, &b, es);           /* little-endian: low bytes */
        }
        CHECK_HIP(hipMalloc((void **)&dev[r], off + n * es + 16));
        CHECK_HIP(hipMemcpy(dev[r], host[r], off + n * es, hipMemcpyHostToDevice));
        dsrc[r] = dev[r] + off;
        hsrc[r] = host[r] + off;
    }
    unsigned char *want = (unsigned char *)malloc(n * es + 1);
    unsigned char *got = (unsigned char *)malloc(n * es + 1);
    if (bf16) rog_oracle_reduce_bf16((const uint16_t *const *)hsrc, W, n, (uint16_t *)want);
    else rog_oracle_reduce_f32((const float *const *)hsrc, W, n, (float *)want);
    unsigned char *dout = NULL;
    void *out;
    if (in_place >= 0) {
        out = (void *)dsrc[in_place];
    } else {
        CHECK_HIP(hipMalloc((void **)&dout, (out_off + n) * es));
        out = dout + out_off * es;
    }
    const rog_status s = rog_reduce_ex(dsrc, W, n, bf16 ? ROG_DTYPE_BF16 : ROG_DTYPE_F32, out, st, path);
    if (s != ROG_OK) {
        fprintf(stderr, "FAIL reduce W=%d n=%zu bf16=%d path=%d: %s\n", W, n, bf16, (int)path, rog_status_string(s));
        ++failures;
    } else {
        CHECK_HIP(hipStreamSynchronize(st));
        CHECK_HIP(hipMemcpy(got, out, n * es, hipMemcpyDeviceToHost));
        if (memcmp(got, want, n * es) != 0) {
            size_t k = 0;
            while (got[k] == want[k]) ++k;
            fprintf(stderr, "FAIL reduce W=%d n=%zu bf16=%d out_off=%zu in_place=%d path=%d: element %zu\n", W, n,
                    bf16, out_off, in_place, (int)path, k / es);
            ++failures;
        }
    }
    if (dout) CHECK_HIP(hipFree(dout));
    for (int r = 0; r < W; ++r) {
        CHECK_HIP(hipFree(dev[r]));
        free(host[r]);
    }
    free(want);
    free(got);
}

/* A batch of binary16 sums (W = 3) in one launch: counts 0, 1, 1000, 65537. */
static void reduce_batch_case(hipStream_t st) {
    enum { N = 4, W = 3 };
    const size_t counts[N] = {0, 1, 1000, 65537};
    uint16_t *h[N][W], *want[N], *got[N];
    uint16_t *d[N][W], *dout[N];
    const void *ptrs[N][W];
    rog_reduce_desc desc[N];
    for (int t = 0; t < N; ++t) {
        const size_t n = counts[t];
        for (int r = 0; r < W; ++r) {
            h[t][r] = (uint16_t *)malloc(n * 2 + 2);
            for (size_t i = 0; i < n; ++i) {
                /* normal binary16 values of magnitude below 2, from the element hash */
                const uint32_t x = elem_bits(53u * (unsigned)t + (unsigned)r, i, 0);
                h[t][r][i] = (uint16_t)(((x >> 16) & 0x8000u) | ((1u + (x >> 3) % 15u) << 10) | (x & 0x3FFu));
            }
            CHECK_HIP(hipMalloc((void **)&d[t][r], n * 2 + 2));
            CHECK_HIP(hipMemcpy(d[t][r], h[t][r], n * 2, hipMemcpyHostToDevice));
            ptrs[t][r] = d[t][r];
        }
        want[t] = (uint16_t *)malloc(n * 2 + 2);
        got[t] = (uint16_t *)malloc(n * 2 + 2);
        rog_oracle_reduce_f16((const uint16_t *const *)h[t], W, n, want[t]);
        CHECK_HIP(hipMalloc((void **)&dout[t], n * 2 + 2));
        desc[t].srcs = ptrs[t];
        desc[t].out = dout[t];
        desc[t].count = n;
    }
    const rog_status s = rog_reduce_many(desc, N, W, ROG_DTYPE_F16, st);
    if (s != ROG_OK) {
        fprintf(stderr, "FAIL reduce batch: %s\n", rog_status_string(s));
        ++failures;
    } else {
        CHECK_HIP(hipStreamSynchronize(st));
        for (int t = 0; t < N; ++t) {
            CHECK_HIP(hipMemcpy(got[t], dout[t], counts[t] * 2, hipMemcpyDeviceToHost));
            if (memcmp(got[t], want[t], counts[t] * 2) != 0) {
                fprintf(stderr, "FAIL reduce batch tensor %d\n", t);
                ++failures;
            }
        }
        /* Captured: one kernel node; three replays over cleared outputs. */
        hipGraphExec_t ex = capture_one_launch(st, 1, desc, N, W, ROG_DTYPE_F16, "reduce batch graph");
        for (int rep = 0; ex && rep < 3; ++rep) {
            for (int t = 0; t < N; ++t) CHECK_HIP(hipMemset(dout[t], FILL, counts[t] * 2 + 2));
            CHECK_HIP(hipGraphLaunch(ex, st));
            CHECK_HIP(hipStreamSynchronize(st));
            for (int t = 0; t < N; ++t) {
                CHECK_HIP(hipMemcpy(got[t], dout[t], counts[t] * 2, hipMemcpyDeviceToHost));
                if (memcmp(got[t], want[t], counts[t] * 2) != 0) {
                    fprintf(stderr, "FAIL reduce batch graph replay %d tensor %d\n", rep, t);
                    ++failures;
                }
            }
        }
        if (ex) CHECK_HIP(hipGraphExecDestroy(ex));
    }
    for (int t = 0; t < N; ++t) {
        for (int r = 0; r < W; ++r) {
            CHECK_HIP(hipFree(d[t][r]));
            free(h[t][r]);
        }
        CHECK_HIP(hipFree(dout[t]));
        free(want[t]);
        free(got[t]);
    }
}

/* Plan flags from the header's rules (no launch: addresses are never touched). */
static void plan_flag_cases(void) {
    const void *srcs[8];
    const uintptr_t base = (uintptr_t)1 << 40;
    rog_plan_info info;
    /* streamed (8 x 48 MiB + 5 >= 384 MiB), sources 1 byte and output 3 bytes past
     * 256-byte boundaries: body head 253, m = (1 + 253) % 16 = 14 -> shared granules */
    const size_t S = ((size_t)48 << 20) + 5;
    for (int r = 0; r < 8; ++r) srcs[r] = (const void *)(base + ((uintptr_t)r << 30) + 1);
    const void *out = (const void *)(base + ((uintptr_t)16 << 30) + 3);
    if (rog_plan(srcs, 8, S, out, ROG_PATH_AUTO, &info) != ROG_OK || info.kernel != ROG_KERNEL_PEER ||
        info.flags != (ROG_PLAN_NT_LOADS | ROG_PLAN_SHIFTED_LOADS)) {
        fprintf(stderr, "plan flags: streamed misaligned gather got kernel %d flags %u\n", info.kernel, info.flags);
        ++failures;
    }
    /* the same layout at 8 MiB per payload: cached loads, unaligned loads kept */
    if (rog_plan(srcs, 8, (size_t)8 << 20, out, ROG_PATH_AUTO, &info) != ROG_OK || info.flags != 0) {
        fprintf(stderr, "plan flags: cached misaligned gather got flags %u\n", info.flags);
        ++failures;
    }
    /* sums: 8 x 24 Mi bf16 (384 MiB) -> granule form; 2 x 1 Mi -> plain */
    for (int r = 0; r < 8; ++r) srcs[r] = (const void *)(base + ((uintptr_t)r << 30));
    out = (const void *)(base + ((uintptr_t)16 << 30));
    if (rog_reduce_plan(srcs, 8, (size_t)24 << 20, ROG_DTYPE_BF16, out, ROG_PATH_AUTO, &info) != ROG_OK ||
        info.flags != (ROG_PLAN_NT_LOADS | ROG_PLAN_SHIFTED_LOADS)) {
        fprintf(stderr, "plan flags: streamed sum got flags %u\n", info.flags);
        ++failures;
    }
    if (rog_reduce_plan(srcs, 2, (size_t)1 << 20, ROG_DTYPE_BF16, out, ROG_PATH_AUTO, &info) != ROG_OK ||
        info.flags != 0) {
        fprintf(stderr, "plan flags: cached sum got flags %u\n", info.flags);
        ++failures;
    }
}

int main(void) {
    plan_flag_cases();
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    const rog_path paths[3] = {ROG_PATH_AUTO, ROG_PATH_SINGLE_WG, ROG_PATH_MULTI_WG};
    const size_t sizes[] = {1, 16, 1024, 4095, 65536, 262151, 1 << 20};
    const size_t offs[][2] = {{0, 0}, {1, 3}, {8, 8}, {0, 5}};
    const int Ws[] = {1, 2, 8};
    for (int p = 0; p < 3; ++p)
        for (unsigned w = 0; w < sizeof Ws / sizeof Ws[0]; ++w)
            for (unsigned s = 0; s < sizeof sizes / sizeof sizes[0]; ++s)
                for (unsigned o = 0; o < sizeof offs / sizeof offs[0]; ++o)
                    gather_case(Ws[w], sizes[s], offs[o][0], offs[o][1], paths[p], st);
    batch_case(st);
    error_cases(st);
    const size_t counts[] = {1, 9, 1000, 32769, 300001};
    const int rWs[] = {1, 3, 8};
    for (int p = 0; p < 3; ++p)
        for (int bf16 = 0; bf16 < 2; ++bf16)
            for (unsigned w = 0; w < sizeof rWs / sizeof rWs[0]; ++w)
                for (unsigned c = 0; c < sizeof counts / sizeof counts[0]; ++c) {
                    reduce_case(rWs[w], counts[c], bf16, (size_t)c % 4, -1, paths[p], st);
                    if (rWs[w] > 1) reduce_case(rWs[w], counts[c], bf16, 0, rWs[w] - 1, paths[p], st);
                }
    reduce_batch_case(st);
    CHECK_HIP(hipStreamDestroy(st));
    printf("abi_c_check: %d failures; single-WG bound %zu bytes, max W %d\n", failures,
           rog_single_wg_max_bytes(), rog_max_peers());
    return failures ? 1 : 0;
}
