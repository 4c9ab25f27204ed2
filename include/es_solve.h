/*
 * es_solve.h -- exact rational solution of an integer system A x = b on one
 * MI355X (gfx950) by multi-prime Dixon p-adic lifting.
 *
 * Method (exact-solve card, phanerozoic/exact-solve, section "Method"):
 * B = A^-1 mod P for a squarefree odd P = prod q_j over primes q_j < 256,
 * r_0 = b, x_i = B r_i mod P, r_{i+1} = (r_i - A x_i) / P; m digits
 * determine x once P^m is larger than 2 N D, N and D being Hadamard-type
 * bounds on the numerators and the denominator.  A^-1 mod q_j comes from a batched Gauss-Jordan inverse (all
 * primes at once; one launch per elimination step, or blocked 32 steps per
 * panel with an int8-MFMA rank-32 update; Barrett-style reduction); each
 * step's x_i is one int8 contraction per prime, a balanced CRT into the
 * wide base-P digit, and a one-limb residual update
 * (r_i - A x_i) P^-1 mod 2^64.  A host stage does the rational
 * reconstruction (common denominator from a sample, then one modular
 * multiply per numerator; the multiplies of all components run on the GPU
 * as one int8 GEMM, the sample and the final gcds on the host).
 *
 * Range (card, "Method" and "Requirements and limits"): A is n x n and b is
 * n x c, both int64 row-major; n * max|A_ij| < 2^63 and 1 <= n <= 2^17.
 *
 * Conventions for every entry point:
 *  - Status is returned as int: ES_OK (0), ES_SINGULAR (1), or a negative
 *    error code.  No entry point throws or aborts; es_strerror names a code.
 *  - "device pointer" means memory on the current HIP device; "host pointer"
 *    means ordinary host memory.  Input pointers are borrowed and never
 *    written.  Device work is enqueued on the given HIP stream (NULL = the
 *    null stream); calls return only after their results are ready.
 *  - Calls are re-entrant; two calls sharing one workspace must not overlap.
 */
#ifndef ES_SOLVE_H
#define ES_SOLVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ES_OK = 0,
    ES_SINGULAR = 1,    /* A is singular over the rationals (card, "API": None) */
    ES_EINVAL = -1,     /* bad size, null pointer or workspace too small */
    ES_ERANGE = -2,     /* n * max|A_ij| >= 2^63 */
    ES_ENOPRIME = -3,   /* det A is a nonzero multiple of every odd prime < 256 */
    ES_EHIP = -4,       /* a HIP runtime call failed */
    ES_ENOMEM = -5,     /* host or device allocation failed */
    ES_EINTERNAL = -6,  /* an internal consistency check failed */
    ES_ETOOBIG = -7     /* n beyond es_noalloc_max_n() for es_batched_inverse_noalloc */
};

#define ES_NUM_PRIMES 53      /* odd primes 3 .. 251 */
#define ES_MAX_N (1 << 17)    /* int8 products accumulate in int32 without overflow */
#define ES_DIGIT_LIMBS 6      /* one base-P digit: 384-bit two's complement */

typedef struct es_solution es_solution;

/* Static name of a status code. */
const char *es_strerror(int status);

/* The odd primes below 256 in ascending order; writes min(cap, 53) of them
 * to q (host pointer) and returns 53. */
int es_primes(int32_t *q, int32_t cap);

/* Bytes of device workspace es_solve_device needs for an n x n system with c
 * right-hand sides; 0 if n or c is out of range.  Depends on (n, c) only,
 * the same on every thread.  It holds the lift's buffers and the scratch of
 * the GPU reconstruction, sized for the largest case over every input within
 * the range limit for which at most five primes divide det A (at n = 1024,
 * c = 1 about 0.9 GB; at n = 2048, c = 16 about 2.6 GB).  An input outside
 * that case is still solved, with the reconstruction on the host.  The
 * library allocates no device memory of its own in es_solve_device. */
size_t es_workspace_bytes(int32_t n, int32_t c);

/*
 * Solve A x = b (card, "Usage"/"API").  dA [n][n] and db [n][c] are device
 * pointers, int64 row-major.  d_ws is caller-owned device memory of at least
 * es_workspace_bytes(n, c) bytes (contents on entry are ignored).  All device
 * work runs on `stream` (a hipStream_t, NULL for the null stream).  On ES_OK
 * *out receives a solution owned by the caller (release with
 * es_solution_free); on any other status *out is NULL.
 */
int es_solve_device(const int64_t *dA, const int64_t *db, int32_t n, int32_t c,
                    void *d_ws, size_t ws_bytes, void *stream, es_solution **out);

/* Same with host pointers A [n][n] and b [n][c]; the library allocates and
 * frees its own device memory and uses the null stream. */
int es_solve(const int64_t *A, const int64_t *b, int32_t n, int32_t c, es_solution **out);

/* Shape of a solution. */
int32_t es_solution_rows(const es_solution *s);
int32_t es_solution_cols(const es_solution *s);

/*
 * Component x[i][k] of a solution, in lowest terms with a positive
 * denominator (zero is 0/1).  *num_sign is -1, 0 or 1; magnitudes are
 * little-endian uint64 limbs, *num_len == 0 for zero, *den_len >= 1.  The
 * limb pointers stay valid until es_solution_free.  ES_EINVAL if (i, k) is
 * out of range or a pointer is NULL.
 */
int es_solution_get(const es_solution *s, int32_t i, int32_t k, int *num_sign,
                    const uint64_t **num, int32_t *num_len,
                    const uint64_t **den, int32_t *den_len);

/* Per-solve facts: live primes (those not dividing det A), step count m,
 * and the bit sizes of the numerator and denominator bounds used. */
int es_solution_info(const es_solution *s, int32_t *live_primes, int32_t *m,
                     int32_t *num_bound_bits, int32_t *den_bound_bits);

/* Bit length of the lifting modulus M = P^m of a solution (0 for NULL). */
int32_t es_solution_modulus_bits(const es_solution *s);

/* Frees everything the library allocated for a solution; NULL is a no-op. */
void es_solution_free(es_solution *s);

/* Host wall-clock stage timings of the last es_solve_device call on this
 * thread, in ms: [0] checks and bounds, [1] residues + batched inverse,
 * [2] lift (with its device-to-host digit copies on the host-reconstruction
 * path), [3] the GPU part of the reconstruction (weights, GEMM, numerators
 * and their copy to the host; 0 on the host path), [4] the whole
 * reconstruction. */
int es_last_timings(double *ms5);

/*
 * How the batched inverse eliminates, for later calls on the calling thread.
 * on = 1 (the default): blocked, 32 elimination steps per panel launch (one
 * workgroup per prime) followed by one int8-MFMA launch that applies them to
 * the rest of every prime's matrix as a rank-32 update; taken when n <= 4096.
 * on = 0 (or n > 4096): one launch per elimination step across all primes.
 * Both choose the same pivots and give identical results.  Without a call,
 * the environment variable ES_INVERSE=stepwise selects the step-wise form.
 */
int es_set_blocked_inverse(int on);

/*
 * Where the reconstruction runs for later solves on the calling thread.
 * on = 1 (the default): the modular multiplies of all components run on the
 * GPU as one int8 GEMM and the gcds that bring them to lowest terms run on
 * the GPU too (the sample stays on the host, and so does any gcd whose
 * Euclidean quotients the GPU rounds cannot handle); the host path is taken anyway when the GPU path does not
 * apply (a modulus P^m of fewer than 65 bits, wider than 131072 bits, more
 * than 1365 lift steps, more than 16 GiB of scratch, or more scratch than
 * the workspace reserves).  on = 0: every digit goes to the host and the
 * host reconstructs.  Both give the same result.  The GPU path's scratch is
 * part of the caller's workspace.  Without a call, the environment variable
 * ES_RECON=host selects the host path.
 */
int es_set_gpu_reconstruction(int on);

/*
 * For later solves on the calling thread with one right-hand side and
 * n > 512: each lift step stores, per component, its balanced residues and
 * the CRT quotient k in a 64-byte record on the device, and one launch turns
 * up to `steps` steps' records into their digits.  steps = 0 restores the
 * default (16 MiB of records); a larger value than the default is taken as
 * the default.  Results are unchanged: smaller values only add launches (the
 * workspace size does not depend on it).  Returns ES_EINVAL for steps < 0.
 */
int es_set_lift_record_steps(int32_t steps);

/*
 * Opt-in kernel timing for measurement.  With es_set_profiling(1) on a
 * thread, later solves on that thread bracket every launch of the hot
 * kernels with a pair of HIP events on the solve's stream (small added gaps
 * between launches; results are unchanged); while it is on, the blocked
 * elimination runs one kernel at a time instead of overlapping each panel
 * with the previous panel's update.  es_kernel_profile then gives,
 * for the last solve, the summed event time in ms and the launch count per
 * kernel class: [0] Gauss-Jordan step, [1] lift contraction (GEMV / GEMM),
 * [2] CRT of the digit, [3] residual update, [4] residues of A, [5] reconstruction
 * GEMM, [6] other reconstruction kernels (weight rows, digit bytes,
 * numerators), [7] the gcds that bring the numerators to lowest terms,
 * [8] panel and [9] update launches of the blocked elimination.  Writes
 * min(cap, 10) entries and returns 10.
 */
int es_set_profiling(int on);
int es_kernel_profile(double *total_ms, int32_t *counts, int32_t cap);

/* ------------------------------------------------------------------------
 * Stage entry points: the hot path's steps, exposed for tests and
 * measurement.  They use the same kernels as es_solve_device.
 * ------------------------------------------------------------------------ */

/*
 * Batched modular inverse (card, "Method": the inverse of A modulo each
 * prime q_j by Gauss-Jordan elimination of [A | I], each elimination step one launch
 * over every prime, reductions by precomputed reciprocals rather than the
 * hardware remainder).
 * dA: device int64 [n][n]; d_ws: workspace as for es_solve_device with c = 1.
 * dB_out: device int8 [53][n][n]; row-major A^-1 mod q_j with entries in the
 * balanced range [-(q_j-1)/2, (q_j-1)/2]; rows of a prime with flag 1 are
 * left unspecified.  flags_host: host int32 [53], 1 where A is singular mod
 * q_j, else 0.  ES_ERANGE as for es_solve_device.
 */
int es_batched_inverse(const int64_t *dA, int32_t n, void *d_ws, size_t ws_bytes,
                       void *stream, int8_t *dB_out, int32_t *flags_host);

/*
 * es_batched_inverse for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and the same results, with no workspace
 * argument.  Its kernels work in a fixed scratch array of 24 MiB that the
 * library holds on each device until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  n must not
 * exceed es_noalloc_max_n() (512): larger n returns ES_ETOOBIG.  dA, dB_out,
 * flags_host and stream as for es_batched_inverse.  Every call on one device
 * shares that device's scratch (each call overwrites it), so calls that
 * overlap on one device, from several threads or streams, race.
 */
int es_batched_inverse_noalloc(const int64_t *dA, int32_t n, void *stream, int8_t *dB_out,
                               int32_t *flags_host);

/* Largest n that es_batched_inverse_noalloc takes. */
int32_t es_noalloc_max_n(void);

/*
 * The lift alone (card, "Method"): runs the batched inverse, drops primes
 * dividing det A, then m lift steps on the live primes and copies the digits
 * x_0 .. x_{m-1} to digits_host, host int64 [n*c][m][6]: component (i, t) at
 * index i*c + t, each digit a little-endian 384-bit two's-complement integer
 * in [-(P-1)/2, (P-1)/2].  If m_req > 0 exactly m_req steps run, else m is
 * chosen from the Hadamard bound.  digits_cap is the capacity of digits_host
 * in int64 words.  live_mask_host (host uint64 [1]) receives bit j set for
 * each live prime index j; m_out receives m.  With digits_host == NULL the
 * call stops after choosing m (nothing is lifted), so a caller can size the
 * buffer.  ES_SINGULAR / ES_ENOPRIME as for es_solve_device; ES_EINVAL if
 * digits_cap is too small.
 */
int es_lift_digits(const int64_t *dA, const int64_t *db, int32_t n, int32_t c,
                   void *d_ws, size_t ws_bytes, void *stream, int32_t m_req,
                   int64_t *digits_host, size_t digits_cap, uint64_t *live_mask_host,
                   int32_t *m_out);

/*
 * Host rational reconstruction (card, "Method": common denominator from a
 * few components, then each numerator by one product modulo P^m).
 * digits: host int64 [n*c][m][6] as written by es_lift_digits; live_mask
 * selects the primes whose product is P; x = A^-1 b is recovered from
 * X = sum x_i P^i given |numerators| <= 2^num_bits and
 * 0 < denominators <= 2^den_bits, which requires P^m > 2^(num_bits+den_bits+1)
 * (ES_EINVAL otherwise).  nthreads <= 0 picks the host core count.
 * ES_EINTERNAL if some component has no fraction within the bounds.
 */
int es_reconstruct(const int64_t *digits, int32_t n, int32_t c, int32_t m,
                   uint64_t live_mask, int32_t num_bits, int32_t den_bits,
                   int32_t nthreads, es_solution **out);

#ifdef __cplusplus
}
#endif

#endif /* ES_SOLVE_H */
