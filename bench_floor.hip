// bench_floor.hip -- the fixed cost of a launch on this GPU, for comparison
// with the gathers' own launches: kernels of the multi-workgroup gather's
// shape (one 64-lane wave per workgroup, one 1 KiB chunk each) that do
// nothing, only load their chunk, or only store it, at the grids of the
// gathers the benchmark times (1 KiB - 1 MiB outputs for the small gathers,
// 64 - 512 MiB for the bandwidth sweep).  Each case is launched 100 times back
// to back on one stream, timed with a pair of HIP events around the 100, and
// again replayed from a HIP graph of the same 100 launches (no host launch
// path between kernels).  Run it under rocprofv3 --kernel-trace for the
// kernel-only durations.  Prints one JSON line per case.
//
// Built by __graft_entry__.build() (bench.build_native) into _build/bench_floor.
// The load-only and store-only kernels touch exactly grid KiB of one buffer;
// the host allocates that many bytes before launching.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                     \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "HIP error %d at line %d: %s\n", (int)e_, __LINE__, #x); \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

// Nothing at all.
__global__ __launch_bounds__(64) void floor_null(v4u *, const v4u *) {}

// Each wave reads its 1 KiB chunk and keeps it only if it holds a value the
// host never writes (the buffer is all zeros), so the loads cannot be dropped
// and nothing is stored.
__global__ __launch_bounds__(64) void floor_load(v4u *out, const v4u *in) {
    const size_t i = size_t(blockIdx.x) * 64 + threadIdx.x;
    const v4u v = __builtin_nontemporal_load(in + i);
    if (v.x == 0x9E3779B9u && v.y == 0x7F4A7C15u) out[i] = v;
}

// Each wave writes its 1 KiB chunk with streamed, write-through stores (the
// gathers' store policy).
__global__ __launch_bounds__(64) void floor_store(v4u *out, const v4u *) {
    const size_t i = size_t(blockIdx.x) * 64 + threadIdx.x;
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(out + size_t(blockIdx.x) * 64, 0, 1024, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v4u{uint32_t(i), 1u, 2u, 3u}, r, int(threadIdx.x * 16), 0, 18);
}

enum { kCalls = 100, kWarm = 10 };

typedef void (*kernel_fn)(v4u *, const v4u *);

static void launch(kernel_fn k, unsigned grid, v4u *out, const v4u *in, hipStream_t st) {
    hipLaunchKernelGGL(k, dim3(grid), dim3(64), 0, st, out, in);
    CHECK(hipGetLastError());
}

int main(void) {
    static const unsigned grids[] = {1, 8, 64, 1024, 65536, 131072, 262144, 524288};
    static const char *names[] = {"null", "load", "store"};
    static const kernel_fn kernels[] = {floor_null, floor_load, floor_store};
    const unsigned max_grid = grids[sizeof grids / sizeof grids[0] - 1];
    const size_t bytes = size_t(max_grid) * 1024;
    v4u *a, *b;
    CHECK(hipMalloc((void **)&a, bytes));
    CHECK(hipMalloc((void **)&b, bytes));
    CHECK(hipMemset(a, 0, bytes));
    CHECK(hipMemset(b, 0, bytes));
    hipStream_t st;
    CHECK(hipStreamCreate(&st));
    hipEvent_t t0, t1;
    CHECK(hipEventCreate(&t0));
    CHECK(hipEventCreate(&t1));
    for (unsigned k = 0; k < 3; ++k) {
        for (unsigned g = 0; g < sizeof grids / sizeof grids[0]; ++g) {
            const unsigned grid = grids[g];
            // every access of a launch lies in [0, grid KiB) of a or b
            if (size_t(grid) * 1024 > bytes) return 3;
            for (int i = 0; i < kWarm; ++i) launch(kernels[k], grid, b, a, st);
            CHECK(hipStreamSynchronize(st));
            CHECK(hipEventRecord(t0, st));
            for (int i = 0; i < kCalls; ++i) launch(kernels[k], grid, b, a, st);
            CHECK(hipEventRecord(t1, st));
            CHECK(hipStreamSynchronize(st));
            float eager_ms = 0.f;
            CHECK(hipEventElapsedTime(&eager_ms, t0, t1));
            hipGraph_t graph;
            hipGraphExec_t exec;
            CHECK(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
            for (int i = 0; i < kCalls; ++i) launch(kernels[k], grid, b, a, st);
            CHECK(hipStreamEndCapture(st, &graph));
            CHECK(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
            CHECK(hipGraphLaunch(exec, st));
            CHECK(hipStreamSynchronize(st));
            CHECK(hipEventRecord(t0, st));
            CHECK(hipGraphLaunch(exec, st));
            CHECK(hipEventRecord(t1, st));
            CHECK(hipStreamSynchronize(st));
            float graph_ms = 0.f;
            CHECK(hipEventElapsedTime(&graph_ms, t0, t1));
            CHECK(hipGraphExecDestroy(exec));
            CHECK(hipGraphDestroy(graph));
            printf("{\"kernel\": \"%s\", \"grid\": %u, \"block\": 64, \"calls\": %d, "
                   "\"eager_us_per_launch\": %.3f, \"graph_us_per_launch\": %.3f}\n",
                   names[k], grid, kCalls, 1000.0 * eager_ms / kCalls, 1000.0 * graph_ms / kCalls);
            fflush(stdout);
        }
    }
    CHECK(hipEventDestroy(t0));
    CHECK(hipEventDestroy(t1));
    CHECK(hipStreamDestroy(st));
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    return 0;
}
