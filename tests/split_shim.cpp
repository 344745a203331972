// Host shim over the PEER kernel's payload cut (split_payload in
// csrc/rog_internal.h), so the CPU tests check the very code the kernels run.
#include "rog_internal.h"

extern "C" void rog_test_split(uint64_t da, uint64_t S, uint64_t *out2) {
    const rog::PeerSplit p = rog::split_payload(da, S);
    out2[0] = p.lo;
    out2[1] = p.hi;
}

extern "C" uint64_t rog_test_body_align(void) { return rog::kBodyAlign; }

// The workgroup-to-chunk remapping of the PEER, BATCH and REDUCE kernels,
// over a whole launch of n chunks: out[b] = xcd_grouped(b, n).
extern "C" void rog_test_xcd_grouped(uint32_t n, uint32_t *out) {
    for (uint32_t b = 0; b < n; ++b) out[b] = rog::xcd_grouped(b, n);
}

extern "C" uint32_t rog_test_xcd_run(void) { return rog::kXcdRun; }
