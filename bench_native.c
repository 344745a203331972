/*
 * bench_native.c -- the small-gather latency of librog.so timed from C, with
 * no Python between the event records: the same cases as bench.py's latency
 * sweep (W in {2, 8}, 1 - 128 KiB per payload, aligned), each call bracketed
 * by its own pair of HIP events on one stream, as the pages time a call.  Also
 * the floor of the timing method itself: an event pair with nothing between
 * and one around a 4-byte hipMemsetAsync.  Prints one JSON object.
 * Built by __graft_entry__.build() into _build/bench_native; bench.py runs it.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "rog.h"

#define N_CALLS 200
#define N_WARM 20

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %d at line %d: %s\n", (int)e_, __LINE__, #x);   \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

static int cmp_float(const void *a, const void *b) {
    const float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

static hipEvent_t e0[N_CALLS], e1[N_CALLS];
static float us[N_CALLS];

/* what: 0 = rog_gather, 1 = nothing, 2 = hipMemsetAsync of 4 bytes */
static void timed(int what, const void *const *srcs, int W, size_t S, void *out, hipStream_t st,
                  float *p10, float *p50, float *p90) {
    for (int i = 0; i < N_WARM + N_CALLS; ++i) {
        const int k = i - N_WARM;
        if (k >= 0) CHECK(hipEventRecord(e0[k], st));
        if (what == 0) {
            if (rog_gather(srcs, W, S, out, st) != ROG_OK) { fprintf(stderr, "rog_gather failed\n"); exit(3); }
        } else if (what == 2) {
            CHECK(hipMemsetAsync(out, 0, 4, st));
        }
        if (k >= 0) CHECK(hipEventRecord(e1[k], st));
    }
    CHECK(hipStreamSynchronize(st));
    for (int k = 0; k < N_CALLS; ++k) {
        CHECK(hipEventElapsedTime(&us[k], e0[k], e1[k]));
        us[k] *= 1000.0f;
    }
    qsort(us, N_CALLS, sizeof us[0], cmp_float);
    *p10 = us[N_CALLS / 10];
    *p50 = us[N_CALLS / 2];
    *p90 = us[N_CALLS * 9 / 10];
}

int main(void) {
    hipStream_t st;
    CHECK(hipStreamCreate(&st));
    for (int k = 0; k < N_CALLS; ++k) {
        CHECK(hipEventCreate(&e0[k]));
        CHECK(hipEventCreate(&e1[k]));
    }
    const int Ws[] = {2, 8};
    const size_t kib[] = {1, 8, 32, 128};
    float p10, p50, p90;
    printf("{\"calls\": %d, \"warmup\": %d, \"cases\": [", N_CALLS, N_WARM);
    int first = 1;
    for (int w = 0; w < 2; ++w) {
        for (int s = 0; s < 4; ++s) {
            const int W = Ws[w];
            const size_t S = kib[s] * 1024;
            void *buf[8];
            const void *srcs[8];
            void *out;
            for (int r = 0; r < W; ++r) {
                CHECK(hipMalloc(&buf[r], S));
                CHECK(hipMemset(buf[r], r + 1, S));
                srcs[r] = buf[r];
            }
            CHECK(hipMalloc(&out, (size_t)W * S));
            timed(0, srcs, W, S, out, st, &p10, &p50, &p90);
            printf("%s{\"W\": %d, \"S_KiB\": %zu, \"p10_us\": %.2f, \"p50_us\": %.2f, \"p90_us\": %.2f}",
                   first ? "" : ", ", W, kib[s], p10, p50, p90);
            first = 0;
            for (int r = 0; r < W; ++r) CHECK(hipFree(buf[r]));
            CHECK(hipFree(out));
        }
    }
    void *tiny;
    CHECK(hipMalloc(&tiny, 64));
    timed(1, NULL, 0, 0, tiny, st, &p10, &p50, &p90);
    printf("], \"empty_event_pair\": {\"p10_us\": %.2f, \"p50_us\": %.2f, \"p90_us\": %.2f}", p10, p50, p90);
    timed(2, NULL, 0, 0, tiny, st, &p10, &p50, &p90);
    printf(", \"memset_4_bytes\": {\"p10_us\": %.2f, \"p50_us\": %.2f, \"p90_us\": %.2f}}\n", p10, p50, p90);
    CHECK(hipFree(tiny));
    for (int k = 0; k < N_CALLS; ++k) {
        CHECK(hipEventDestroy(e0[k]));
        CHECK(hipEventDestroy(e1[k]));
    }
    CHECK(hipStreamDestroy(st));
    return 0;
}
