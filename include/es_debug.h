/*
 * es_debug.h -- test hooks into the host big-integer code of libexact_solve.
 *
 * For the test suite only: they expose the bignum routines that the host
 * reconstruction stage uses, so that they can be checked against Python
 * integers without a GPU.  Integers are passed sign-magnitude: little-endian
 * uint64 limbs plus a sign flag (1 = negative).  Output buffers hold `cap`
 * limbs; the call returns ES_EINVAL (-1) if a result does not fit, else 0.
 */
#ifndef ES_DEBUG_H
#define ES_DEBUG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ES_DBG_MUL = 0, ES_DBG_DIVMOD = 1, ES_DBG_GCD = 2, ES_DBG_ADD = 3, ES_DBG_SUB = 4, ES_DBG_DIVEXACT1 = 5 };

/* op(a, b): MUL r1 = a*b; DIVMOD r1 = trunc(a/b), r2 = a - r1*b (b != 0);
 * GCD r1 = gcd(a, b) >= 0; ADD r1 = a + b; SUB r1 = a - b; DIVEXACT1
 * r1 = a / b for a positive one-limb b that divides a (the one-word Hensel
 * division of the lowest-terms step; -1 otherwise). */
int es_dbg_bignum(int op, const uint64_t *a, int32_t la, int a_neg, const uint64_t *b, int32_t lb,
                  int b_neg, uint64_t *r1, int32_t *l1, int *n1, uint64_t *r2, int32_t *l2, int *n2,
                  int32_t cap);

/* Wang rational reconstruction of a (0 <= a < M) with bounds N, D: returns 0
 * and num/den (den > 0) if a fraction exists, 1 if none, -1 on bad input.
 * The reconstruction runs twice, once on the calling thread alone and once
 * with the cofactor updates on a second thread; -2 if the two disagree. */
int es_dbg_ratrec(const uint64_t *a, int32_t la, const uint64_t *M, int32_t lM, const uint64_t *N,
                  int32_t lN, const uint64_t *D, int32_t lD, uint64_t *num, int32_t *lnum, int *nneg,
                  uint64_t *den, int32_t *lden, int32_t cap);

/* The lift's step count for live-prime set `mask` (bit j: the j-th odd
 * prime below 256) and bounds of nbits / dbits bits: m_exact and bits_exact
 * from P^m formed exactly, m_fast and bits_fast (the bit length of P^m) as
 * the solve takes them, from log2 P without forming P^m.  Returns 0, or -1
 * for an empty mask or bounds below 1. */
int es_dbg_step_count(uint64_t mask, int32_t nbits, int32_t dbits, int32_t *m_exact, int64_t *bits_exact,
                      int32_t *m_fast, int64_t *bits_fast);

/* X_k = sum_{i<m} x_{k,i} P^i for `count` components of m digits each
 * (int64 [count][m][6]: balanced 384-bit two's-complement digits), the way
 * the sample is assembled: each whole, and cut into `parts` ranges (a power
 * of two) assembled on the pool's threads and joined pairwise.  X_k goes to
 * out + k cap (lens[k] limbs, neg[k] its sign).  Returns 0, -1 on bad input
 * or a result wider than cap, -2 if the two ways disagree. */
int es_dbg_assemble(const uint64_t *P, int32_t lP, const int64_t *digits, int32_t m, int32_t count,
                    int32_t parts, uint64_t *out, int32_t *lens, int *neg, int32_t cap);

/* For the last solve on the calling thread that took the GPU
 * reconstruction: `alone` = components whose GPU numerator fell outside the
 * bound and were reconstructed alone on the host; `host_gcds` = components
 * whose gcd the host finished.  Both -1 if no such solve has run on this
 * thread.  Returns 0, or -1 for a null pointer. */
int es_dbg_last_recon_counts(int64_t *alone, int64_t *host_gcds);

#ifdef __cplusplus
}
#endif

#endif /* ES_DEBUG_H */
