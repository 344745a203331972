/*
 * rog_oracle.c -- CPU oracle for the rank-ordered gather.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library, and the library never
 * calls it.
 *
 * What is computed.  The pages "perf(cuda): vectorize the deterministic
 * all-gather copy and right-size its single-block path" (RL-Align/RL-Kernel
 * PR #491, section "What", the copy_rank_ordered bullet) state that the
 * optimised copy is still a plain rank-ordered copy whose result is
 * byte-identical to the old one, and the size test in the same PR ("Tests")
 * compares it with NCCL's all-gather.  An all-gather of W payloads of S bytes
 * each places payload r at byte offset r*S of the W*S-byte output.  The oracle
 * is that definition written out as a per-peer byte loop, peers in rank order.
 *
 * Parity pins (tests/test_oracle.py): the closed form b"".join(payloads),
 * numpy.concatenate, the per-segment invariant, peer-tagged byte patterns,
 * guard bytes around the output, unchanged sources, brute force over tiny
 * sizes and offsets against an independent pure-Python loop, and planted
 * mistakes that each pin must catch.
 */
#include <stddef.h>

/* out[r*S + i] = srcs[r][i] for r in [0, W), i in [0, S).  Host memory. */
void rog_oracle_gather(const unsigned char *const *srcs, int W, size_t S,
                       unsigned char *out)
{
    for (int r = 0; r < W; ++r) {
        const unsigned char *src = srcs[r];
        unsigned char *dst = out + (size_t)r * S;
        for (size_t i = 0; i < S; ++i)
            dst[i] = src[i];
    }
}

/*
 * Batched form: n independent gathers that share W, taken in order.  The
 * pages' all_gather_many (same PR, review thread on the benchmark's
 * all_gather_many row) gathers each tensor of a list into its own output with
 * one handshake and no packing; each output is its own rank-ordered
 * concatenation.  srcs holds n*W pointers, tensor t's payloads at
 * srcs[t*W .. t*W+W-1]; bytes_per_rank[t] is that tensor's S.
 */
void rog_oracle_gather_many(const unsigned char *const *srcs, unsigned char *const *outs,
                            const size_t *bytes_per_rank, int n, int W)
{
    for (int t = 0; t < n; ++t)
        rog_oracle_gather(srcs + (size_t)t * W, W, bytes_per_rank[t], outs[t]);
}
