// Host shim over the PEER kernel's payload cut (split_payload in
// csrc/rog_internal.h), so the CPU tests check the very code the kernels run.
#include "rog_internal.h"

extern "C" void rog_test_split(uint64_t da, uint64_t S, uint64_t *out2) {
    const rog::PeerSplit p = rog::split_payload(da, S);
    out2[0] = p.lo;
    out2[1] = p.hi;
}

extern "C" uint64_t rog_test_body_align(void) { return rog::kBodyAlign; }
