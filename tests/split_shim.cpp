// Host shim over the PEER kernel's payload cut (split_payload in
// csrc/rog_internal.h), so the CPU tests check the very code the kernels run.
#include "rog_internal.h"

extern "C" void rog_test_split(uint64_t sa, uint64_t da, uint64_t S, uint64_t *out3) {
    const rog::PeerSplit p = rog::split_payload(sa, da, S);
    out3[0] = p.lo;
    out3[1] = p.hi;
    out3[2] = p.delta;
}

extern "C" uint64_t rog_test_body_align(void) { return rog::kBodyAlign; }
