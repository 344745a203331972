// Host shim over the PEER kernel's payload cut (split_payload in
// csrc/rog_internal.h), so the CPU tests check the very code the kernels run.
#include "rog_internal.h"

extern "C" void rog_test_split(uint64_t da, uint64_t S, uint64_t *out2) {
    const rog::PeerSplit p = rog::split_payload(da, S);
    out2[0] = p.lo;
    out2[1] = p.hi;
}

extern "C" uint64_t rog_test_body_align(void) { return rog::kBodyAlign; }

// The sum's granule-form cut (split_anchored).
extern "C" void rog_test_split_anchored(uint64_t da, uint64_t S, uint64_t anchor, uint64_t *out2) {
    const rog::PeerSplit p = rog::split_anchored(da, S, anchor);
    out2[0] = p.lo;
    out2[1] = p.hi;
}

// The workgroup-to-chunk remapping of the FLAT, PEER, BATCH and REDUCE kernels,
// over a whole launch of n chunks: out[b] = xcd_grouped(b, n).
extern "C" void rog_test_xcd_grouped(uint32_t n, uint32_t *out) {
    for (uint32_t b = 0; b < n; ++b) out[b] = rog::xcd_grouped(b, n);
}

extern "C" uint32_t rog_test_xcd_run(void) { return rog::kXcdRun; }

// The FLAT kernels' chunk cut: chunk c = flat_span(c, chunk, shift, n_vec),
// flat_chunk_count chunks, and the planner's shift for an output address.
extern "C" void rog_test_flat_span(uint32_t c, uint32_t chunk, uint32_t shift, uint32_t n_vec, uint32_t *out2) {
    const rog::ChunkSpan s = rog::flat_span(c, chunk, shift, n_vec);
    out2[0] = s.b;
    out2[1] = s.n;
}
extern "C" uint32_t rog_test_flat_chunk_count(uint32_t n_vec, uint32_t chunk, uint32_t shift) {
    return rog::flat_chunk_count(n_vec, chunk, shift);
}
extern "C" uint32_t rog_test_flat_shift(uint64_t out, uint64_t n_vec) { return rog::flat_shift(out, n_vec); }

// The PEER body's byte-window cut (cut16 in csrc/rog_device.h): bytes
// [m, m + 16) of the 32 bytes lo then hi.
#include "rog_device.h"

extern "C" void rog_test_cut16(const uint8_t *lo16, const uint8_t *hi16, uint32_t m, uint8_t *out16) {
    rog::vec16 lo, hi;
    __builtin_memcpy(&lo, lo16, 16);
    __builtin_memcpy(&hi, hi16, 16);
    const rog::vec16 v = rog::cut16(lo, hi, m);
    __builtin_memcpy(out16, &v, 16);
}

extern "C" int rog_test_peer_shift(void) { return rog::kPeerShift; }
