/*
 * rog_oracle.c -- CPU oracle for the rank-ordered gather and the rank-ordered sum.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library, and the library never
 * calls it.
 *
 * What is computed.  The pages "perf(cuda): vectorize the deterministic
 * all-gather copy and right-size its single-block path" (RL-Align/RL-Kernel
 * PR #491, section "What", the copy_rank_ordered bullet) say that the faster
 * copy moves the same bytes to the same places as the copy it replaces, and
 * the size test in the same PR ("Tests")
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
#include <stdint.h>
#include <string.h>

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
 * all_gather_many row) gathers each tensor of a list into an output of its
 * own, synchronising the ranks once for the whole list and without first
 * copying the tensors into one buffer; each output is its own rank-ordered
 * concatenation.  srcs holds n*W pointers, tensor t's payloads at
 * srcs[t*W .. t*W+W-1]; bytes_per_rank[t] is that tensor's S.
 */
void rog_oracle_gather_many(const unsigned char *const *srcs, unsigned char *const *outs,
                            const size_t *bytes_per_rank, int n, int W)
{
    for (int t = 0; t < n; ++t)
        rog_oracle_gather(srcs + (size_t)t * W, W, bytes_per_rank[t], outs[t]);
}

/*
 * Deterministic sum of W payloads (the reduction at the heart of a
 * deterministic all-reduce or reduce-scatter).  The pages name these
 * collectives beside the gather and say only that their results must not
 * depend on timing (RL-Align/RL-Kernel PR #491, section "Not in this PR", on
 * the all_reduce / reduce_scatter single-block paths); they print no
 * arithmetic; they name the backend a fixed tree (cuda_ipc_fixed_tree, the
 * author's replies on the benchmark's recorded backend) and leave its
 * reduction untouched and unprinted.  PARITY UNPINNED against the pages' own
 * reduction order: the tests pin this definition, not the backend's tree.
 * The reading taken here is the plainest deterministic one, a left-deep
 * chain in rank order:
 *
 *     out[i] = round( ((x_0[i] + x_1[i]) + x_2[i]) + ... + x_{W-1}[i] )
 *
 * with the sum taken in rank order, every addition in IEEE binary32 rounded
 * to nearest-even, the first term taken as it is (not added to a zero, so a
 * lone -0 stays -0), bf16 and binary16 inputs widened to binary32 exactly,
 * and the result rounded once to the element type (bf16: nearest-even on the
 * 16 dropped bits; binary16: nearest-even with gradual underflow and overflow
 * to infinity; a NaN stays a NaN).  Host memory; elements aligned to their
 * size.
 * Built with -ffp-contract=off; x86-64 evaluates float in float (SSE).
 */

static float oracle_bf16_to_f32(uint16_t h)
{
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even.  A NaN keeps its sign and
 * top payload bits and is made quiet. */
uint16_t rog_oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    const uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (upper & 1u)))
        upper += 1u;    /* a carry into the exponent is the right result */
    return (uint16_t)upper;
}

void rog_oracle_reduce_f32(const float *const *srcs, int W, size_t count, float *out)
{
    for (size_t i = 0; i < count; ++i) {
        float acc = srcs[0][i];
        for (int r = 1; r < W; ++r)
            acc = acc + srcs[r][i];
        out[i] = acc;
    }
}

void rog_oracle_reduce_bf16(const uint16_t *const *srcs, int W, size_t count, uint16_t *out)
{
    for (size_t i = 0; i < count; ++i) {
        float acc = oracle_bf16_to_f32(srcs[0][i]);
        for (int r = 1; r < W; ++r)
            acc = acc + oracle_bf16_to_f32(srcs[r][i]);
        out[i] = rog_oracle_f32_to_bf16(acc);
    }
}

/* IEEE binary16 -> binary32, exact (subnormals, infinities and NaNs kept). */
static float oracle_f16_to_f32(uint16_t h)
{
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t expo = (h >> 10) & 0x1Fu;
    uint32_t mant = h & 0x3FFu;
    uint32_t u;
    if (expo == 0x1Fu) {
        u = sign | 0x7F800000u | (mant << 13);              /* infinity or NaN */
    } else if (expo != 0) {
        u = sign | ((expo + 112u) << 23) | (mant << 13);    /* normal: rebias 15 -> 127 */
    } else if (mant == 0) {
        u = sign;                                           /* signed zero */
    } else {
        /* subnormal: mant * 2^-24; normalise into binary32 */
        uint32_t e = 113u;                                  /* 127 - 14 */
        while (!(mant & 0x400u)) { mant <<= 1; --e; }
        u = sign | (e << 23) | ((mant & 0x3FFu) << 13);
    }
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> IEEE binary16, round to nearest, ties to even, with gradual
 * underflow and overflow to infinity; a NaN stays a (quiet) NaN.
 *
 * A finite binary32 value is sig * 2^(e - 150) (sig the 24-bit significand,
 * e the biased exponent; binary32 subnormals have e = 1 and no hidden bit).
 * binary16 numbers of unbiased exponent E >= -14 are multiples of 2^(E - 10);
 * below 2^-14 they are multiples of 2^-24.  So the value is rounded to a whole
 * number q of quanta 2^qe, qe = max(E, -14) - 10, by dropping `shift` bits of
 * sig.  A q that reaches the next power of two moves to the next binade; past
 * the largest finite binary16 (E = 15) the result is infinity. */
uint16_t rog_oracle_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t expo = (u >> 23) & 0xFFu;
    const uint32_t mant = u & 0x7FFFFFu;
    if (expo == 0xFFu)                                      /* infinity, or a NaN made quiet */
        return (uint16_t)(sign | 0x7C00u | (mant ? 0x0200u | (mant >> 13) : 0u));
    const int32_t e = expo ? (int32_t)expo : 1;
    const uint32_t sig = expo ? (mant | 0x800000u) : mant;
    const int32_t E = e - 127;
    const int32_t qe = (E < -14 ? -14 : E) - 10;
    const int32_t shift = qe - (e - 150);                   /* >= 13 */
    if (shift >= 25)                                        /* below half the smallest quantum */
        return sign;
    uint32_t q = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1;
    if (E < -14)                            /* q quanta of 2^-24; q = 2^10 is the smallest normal */
        return (uint16_t)(sign | q);
    int32_t Eq = E;
    if (q == 0x800u) {                      /* rounded up into the next binade */
        Eq += 1;
        q = 0x400u;
    }
    if (Eq > 15)
        return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((uint32_t)(Eq + 15) << 10) | (q & 0x3FFu));
}

void rog_oracle_reduce_f16(const uint16_t *const *srcs, int W, size_t count, uint16_t *out)
{
    for (size_t i = 0; i < count; ++i) {
        float acc = oracle_f16_to_f32(srcs[0][i]);
        for (int r = 1; r < W; ++r)
            acc = acc + oracle_f16_to_f32(srcs[r][i]);
        out[i] = rog_oracle_f32_to_f16(acc);
    }
}
