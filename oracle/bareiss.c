/*
 * The solution of A x = b as exact fractions, by fraction-free Bareiss elimination,
 * in plain C with its own arbitrary-precision integers and POSIX threads.
 *
 * TEST INFRASTRUCTURE ONLY: this is the CPU oracle for the exact solver.  Only
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * load it.  It shares no code with the HIP library.
 *
 * What it computes is the definition of the result in the exact-solve card
 * (phanerozoic/exact-solve), sections "API" and "Correctness": x = A^-1 b over
 * the rationals, each component in lowest terms with a positive denominator,
 * or "singular" when det A = 0.  The algorithm is the same as the Python
 * oracle (oracle/exact.py) and is checked bit for bit against it:
 *   1. Bareiss elimination of [A | b]; pivot = lowest row >= k with a nonzero
 *      entry in column k; every division by the previous pivot is exact.
 *   2. d = M[n-1][n-1] = +-det A; back substitution
 *      N_i = (d M[i][n+t] - sum_{j>i} M[i][j] N_j) / M[i][i], exact by Cramer.
 *   3. x_i = N_i / d reduced by gcd, sign moved to the numerator.
 * Big integers: sign-magnitude, 64-bit limbs, schoolbook multiplication.
 * Every division the method makes is exact (Bareiss's quotients, the back
 * substitution by Cramer's rule, lowest terms by the gcd), so division is
 * the 2-adic exact division, checked; the gcd is the binary algorithm.
 * Nothing is tuned.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

typedef struct {
    uint64_t *d; /* little-endian magnitude limbs */
    int len;     /* 0 means zero */
    int cap;
    int neg;     /* 1 if negative (never set for zero) */
} bz;

static void die(const char *msg) {
    fprintf(stderr, "oracle: %s\n", msg);
    abort();
}

static void bz_reserve(bz *x, int cap) {
    if (x->cap >= cap) return;
    x->d = (uint64_t *)realloc(x->d, (size_t)cap * sizeof(uint64_t));
    if (!x->d) die("out of memory");
    x->cap = cap;
}

static void bz_clear(bz *x) {
    free(x->d);
    x->d = NULL;
    x->len = x->cap = x->neg = 0;
}

static void bz_norm(bz *x) {
    while (x->len > 0 && x->d[x->len - 1] == 0) x->len--;
    if (x->len == 0) x->neg = 0;
}

static void bz_set_i64(bz *x, int64_t v) {
    bz_reserve(x, 1);
    x->neg = v < 0;
    x->d[0] = v < 0 ? (uint64_t)0 - (uint64_t)v : (uint64_t)v;
    x->len = 1;
    bz_norm(x);
}

static void bz_copy(bz *r, const bz *a) {
    if (r == a) return;
    bz_reserve(r, a->len > 0 ? a->len : 1);
    if (a->len) memcpy(r->d, a->d, (size_t)a->len * sizeof(uint64_t));
    r->len = a->len;
    r->neg = a->neg;
}

static int mag_cmp(const uint64_t *a, int la, const uint64_t *b, int lb) {
    if (la != lb) return la < lb ? -1 : 1;
    for (int i = la - 1; i >= 0; i--)
        if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
    return 0;
}

/* r = a + b, r has room for max(la, lb) + 1 limbs; returns length */
static int mag_add(uint64_t *r, const uint64_t *a, int la, const uint64_t *b, int lb) {
    if (la < lb) { const uint64_t *t = a; a = b; b = t; int tl = la; la = lb; lb = tl; }
    uint64_t carry = 0;
    for (int i = 0; i < la; i++) {
        u128 s = (u128)a[i] + (i < lb ? b[i] : 0) + carry;
        r[i] = (uint64_t)s;
        carry = (uint64_t)(s >> 64);
    }
    r[la] = carry;
    return la + 1;
}

/* r = a - b with a >= b; returns length (not normalised) */
static int mag_sub(uint64_t *r, const uint64_t *a, int la, const uint64_t *b, int lb) {
    uint64_t borrow = 0;
    for (int i = 0; i < la; i++) {
        uint64_t bi = i < lb ? b[i] : 0;
        uint64_t t = a[i] - bi;
        uint64_t b1 = a[i] < bi;
        uint64_t t2 = t - borrow;
        uint64_t b2 = t < borrow;
        r[i] = t2;
        borrow = b1 | b2;
    }
    if (borrow) die("mag_sub underflow");
    return la;
}

/* r[0 .. la+lb) = a * b (schoolbook); r must not alias a or b */
static void mag_mul(uint64_t *r, const uint64_t *a, int la, const uint64_t *b, int lb) {
    memset(r, 0, (size_t)(la + lb) * sizeof(uint64_t));
    for (int i = 0; i < la; i++) {
        uint64_t carry = 0;
        for (int j = 0; j < lb; j++) {
            u128 p = (u128)a[i] * b[j] + r[i + j] + carry;
            r[i + j] = (uint64_t)p;
            carry = (uint64_t)(p >> 64);
        }
        r[i + lb] = carry;
    }
}

/* r = a * b */
static void bz_mul(bz *r, const bz *a, const bz *b, bz *tmp) {
    if (a->len == 0 || b->len == 0) { r->len = 0; r->neg = 0; return; }
    bz_reserve(tmp, a->len + b->len);
    mag_mul(tmp->d, a->d, a->len, b->d, b->len);
    tmp->len = a->len + b->len;
    tmp->neg = a->neg ^ b->neg;
    bz_norm(tmp);
    bz_copy(r, tmp);
}

/* r = a + sgn*b, with sgn = +1 or -1; r may alias a */
static void bz_addsub(bz *r, const bz *a, const bz *b, int sgn, bz *tmp) {
    int bneg = b->len ? (b->neg ^ (sgn < 0)) : 0;
    if (b->len == 0) { bz_copy(r, a); return; }
    if (a->len == 0) { bz_copy(r, b); r->neg = bneg; return; }
    int ml = (a->len > b->len ? a->len : b->len) + 1;
    bz_reserve(tmp, ml);
    if (a->neg == bneg) {
        tmp->len = mag_add(tmp->d, a->d, a->len, b->d, b->len);
        tmp->neg = a->neg;
    } else {
        int c = mag_cmp(a->d, a->len, b->d, b->len);
        if (c == 0) { r->len = 0; r->neg = 0; return; }
        if (c > 0) { tmp->len = mag_sub(tmp->d, a->d, a->len, b->d, b->len); tmp->neg = a->neg; }
        else       { tmp->len = mag_sub(tmp->d, b->d, b->len, a->d, a->len); tmp->neg = bneg; }
    }
    bz_norm(tmp);
    bz_copy(r, tmp);
}

/* number of trailing zero bits of a nonzero magnitude */
static long mag_ctz(const uint64_t *a, int la) {
    long z = 0;
    int i = 0;
    while (i < la && a[i] == 0) { i++; z += 64; }
    if (i == la) die("trailing zeros of zero");
    return z + __builtin_ctzll(a[i]);
}

/* r = a >> sh (r may be a itself: limb i reads limbs at or above i); returns
   the normalised length */
static int mag_shr(uint64_t *r, const uint64_t *a, int la, long sh) {
    int limbs = (int)(sh / 64), bits = (int)(sh % 64);
    int lr = la - limbs;
    if (lr <= 0) return 0;
    for (int i = 0; i < lr; i++) {
        uint64_t v = a[i + limbs] >> bits;
        if (bits && i + limbs + 1 < la) v |= a[i + limbs + 1] << (64 - bits);
        r[i] = v;
    }
    while (lr > 0 && r[lr - 1] == 0) lr--;
    return lr;
}

/* r = a << sh, r has room for la + sh/64 + 1 limbs and does not alias a;
   returns the normalised length */
static int mag_shl(uint64_t *r, const uint64_t *a, int la, long sh) {
    int limbs = (int)(sh / 64), bits = (int)(sh % 64);
    memset(r, 0, (size_t)(la + limbs + 1) * sizeof(uint64_t));
    for (int i = 0; i < la; i++) {
        r[i + limbs] |= a[i] << bits;
        r[i + limbs + 1] = bits ? a[i] >> (64 - bits) : 0;
    }
    int lr = la + limbs + 1;
    while (lr > 0 && r[lr - 1] == 0) lr--;
    return lr;
}

typedef struct {
    bz t1, w, v, q;
} scratch;

static void scratch_free(scratch *s) {
    bz_clear(&s->t1); bz_clear(&s->w); bz_clear(&s->v); bz_clear(&s->q);
}

/*
 * Exact division by the 2-adic method (Jebelean, "An algorithm for exact
 * division", 1993): q = |a| / |b| when |b| divides |a|.  Both are shifted
 * right by the divisor's trailing zero bits, which makes the divisor odd and
 * so invertible modulo 2^64; then the quotient is built from its lowest limb
 * up: limb i is the running remainder's limb i times that inverse (mod 2^64),
 * and that multiple of the divisor, shifted by i limbs, is subtracted.  When
 * the division is exact the remainder ends at zero; any other outcome
 * (a bit of |a| below the divisor's lowest set bit, a borrow out of the top,
 * or a nonzero limb left over) means it was not.  Returns 0 and sets q's
 * magnitude, or -1 if |b| does not divide |a|.
 */
static int mag_divexact(bz *q, const bz *a, const bz *b, scratch *s) {
    if (b->len == 0) die("division by zero");
    if (a->len == 0) { q->len = 0; q->neg = 0; return 0; }
    long sh = mag_ctz(b->d, b->len);
    if (mag_ctz(a->d, a->len) < sh) return -1;
    bz_reserve(&s->w, a->len);
    bz_reserve(&s->v, b->len);
    int la = mag_shr(s->w.d, a->d, a->len, sh);
    int lb = mag_shr(s->v.d, b->d, b->len, sh);
    uint64_t *w = s->w.d;
    const uint64_t *v = s->v.d;
    if (la < lb) return -1;
    int lq = la - lb + 1;
    /* Newton's iteration x <- x (2 - v0 x) doubles the correct low bits of
       an inverse of the odd v0; v0 itself is one modulo 8 */
    uint64_t inv = v[0];
    for (int it = 0; it < 5; it++) inv *= 2 - v[0] * inv;
    bz_reserve(&s->q, lq);
    uint64_t *qd = s->q.d;
    for (int i = 0; i < lq; i++) {
        uint64_t qi = w[i] * inv;
        qd[i] = qi;
        /* w -= qi * v * 2^(64 i), with a signed running carry */
        __int128 acc = 0;
        for (int j = 0; j < lb; j++) {
            u128 p = (u128)qi * v[j];
            acc += (__int128)w[i + j] - (__int128)(uint64_t)p;
            w[i + j] = (uint64_t)acc;
            acc >>= 64;
            acc -= (__int128)(uint64_t)(p >> 64);
        }
        for (int k = i + lb; acc != 0 && k < la; k++) {
            acc += (__int128)w[k];
            w[k] = (uint64_t)acc;
            acc >>= 64;
        }
        if (acc != 0) return -1;          /* the remainder went negative */
    }
    for (int k = 0; k < la; k++)
        if (w[k] != 0) return -1;
    bz_reserve(q, lq);
    memcpy(q->d, qd, (size_t)lq * sizeof(uint64_t));
    q->len = lq;
    q->neg = 0;
    bz_norm(q);
    return 0;
}

/* q = a / b, the division being exact (checked) */
static void bz_divexact(bz *q, const bz *a, const bz *b, scratch *s) {
    int neg = a->neg ^ b->neg;
    if (mag_divexact(q, a, b, s) != 0) die("inexact division");
    q->neg = q->len ? neg : 0;
}

/*
 * g = gcd(|a|, |b|) by the binary algorithm (Stein, 1967; Knuth, TAOCP
 * vol. 2, 4.5.2, Algorithm B): the common power of two is set aside, both
 * numbers are made odd, and the smaller is subtracted from the larger, whose
 * factors of two are then removed, until the two are equal.
 */
static void bz_gcd(bz *g, const bz *a, const bz *b, scratch *s) {
    (void)s;
    if (a->len == 0 || b->len == 0) {
        bz_copy(g, a->len ? a : b);
        g->neg = 0;
        return;
    }
    bz x = {0}, y = {0};
    bz_copy(&x, a); x.neg = 0;
    bz_copy(&y, b); y.neg = 0;
    long za = mag_ctz(x.d, x.len), zb = mag_ctz(y.d, y.len);
    long common = za < zb ? za : zb;
    x.len = mag_shr(x.d, x.d, x.len, za);
    y.len = mag_shr(y.d, y.d, y.len, zb);
    for (;;) {
        int c = mag_cmp(x.d, x.len, y.d, y.len);
        if (c == 0) break;
        if (c < 0) { bz t = x; x = y; y = t; }
        x.len = mag_sub(x.d, x.d, x.len, y.d, y.len);   /* even and nonzero */
        while (x.len > 0 && x.d[x.len - 1] == 0) x.len--;
        x.len = mag_shr(x.d, x.d, x.len, mag_ctz(x.d, x.len));
    }
    bz_reserve(g, x.len + (int)(common / 64) + 2);
    g->len = mag_shl(g->d, x.d, x.len, common);
    g->neg = 0;
    bz_clear(&x); bz_clear(&y);
}

/* ------------------------------------------------------------------------ */

typedef struct {
    int n, c, T, max_steps;
    bz **M;          /* row pointers, n rows of n + c entries */
    bz *N;           /* numerators [n][c] */
    bz d;            /* +-det A */
    bz *partial;     /* per-thread partial sums for back substitution */
    bz *num, *den;   /* reduced output [n][c] */
    int singular, stopped;
    int cur_i, cur_t;
    double *step_seconds; /* optional: wall time of each elimination step */
    pthread_barrier_t bar;
} job;

#include <time.h>
static double now_s(void) {
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return ts.tv_sec + 1e-9 * ts.tv_nsec;
}

typedef struct { job *J; int tid; } warg;

static void *worker(void *arg) {
    warg *w = (warg *)arg;
    job *J = w->J;
    int tid = w->tid, T = J->T, n = J->n, c = J->c, W = n + c;
    scratch s;
    memset(&s, 0, sizeof s);
    bz a = {0}, b = {0};

    /* forward elimination */
    double t_step = now_s();
    for (int k = 0; k < n; k++) {
        if (tid == 0) {
            if (J->step_seconds && k > 0) {
                double t = now_s();
                J->step_seconds[k - 1] = t - t_step;
                t_step = t;
            }
            if (J->max_steps >= 0 && k >= J->max_steps) {
                J->stopped = 1;
            } else {
                int piv = -1;
                for (int i = k; i < n; i++)
                    if (J->M[i][k].len != 0) { piv = i; break; }
                if (piv < 0) J->singular = 1;
                else if (piv != k) { bz *t = J->M[k]; J->M[k] = J->M[piv]; J->M[piv] = t; }
            }
        }
        pthread_barrier_wait(&J->bar);
        if (J->singular || J->stopped) goto done;
        const bz *rk = J->M[k];
        const bz *akk = &rk[k];
        const bz *prev = k > 0 ? &J->M[k - 1][k - 1] : NULL;
        for (int i = k + 1 + tid; i < n; i += T) {
            bz *ri = J->M[i];
            const bz *aik = &ri[k];
            for (int j = k + 1; j < W; j++) {
                bz_mul(&a, akk, &ri[j], &s.t1);
                bz_mul(&b, aik, &rk[j], &s.t1);
                bz_addsub(&a, &a, &b, -1, &s.t1);
                if (prev) bz_divexact(&ri[j], &a, prev, &s);
                else bz_copy(&ri[j], &a);
            }
        }
        pthread_barrier_wait(&J->bar);
        if (tid == 0)
            for (int i = k + 1; i < n; i++) bz_clear(&J->M[i][k]);
    }

    if (tid == 0) bz_copy(&J->d, &J->M[n - 1][n - 1]);
    pthread_barrier_wait(&J->bar);

    /* fraction-free back substitution */
    for (int t = 0; t < c; t++) {
        for (int i = n - 1; i >= 0; i--) {
            bz *acc = &J->partial[tid];
            acc->len = 0; acc->neg = 0;
            const bz *ri = J->M[i];
            for (int j = i + 1 + tid; j < n; j += T) {
                bz_mul(&a, &ri[j], &J->N[(size_t)j * c + t], &s.t1);
                bz_addsub(acc, acc, &a, +1, &s.t1);
            }
            pthread_barrier_wait(&J->bar);
            if (tid == 0) {
                bz_mul(&a, &J->d, &ri[n + t], &s.t1);
                for (int u = 0; u < T; u++) bz_addsub(&a, &a, &J->partial[u], -1, &s.t1);
                bz_divexact(&J->N[(size_t)i * c + t], &a, &ri[i], &s);
            }
            pthread_barrier_wait(&J->bar);
        }
    }

    /* lowest terms, positive denominator */
    for (int idx = tid; idx < n * c; idx += T) {
        bz *num = &J->num[idx], *den = &J->den[idx];
        bz_gcd(&a, &J->N[idx], &J->d, &s);
        bz_divexact(num, &J->N[idx], &a, &s);
        bz_divexact(den, &J->d, &a, &s);
        if (den->neg) {
            den->neg = 0;
            if (num->len) num->neg ^= 1;
        }
        if (num->len == 0) { bz_set_i64(den, 1); }
    }
done:
    bz_clear(&a); bz_clear(&b);
    scratch_free(&s);
    return NULL;
}

static size_t put_hex(char *o, const bz *x) {
    size_t k = 0;
    if (x->len == 0) { o[k++] = '0'; return k; }
    if (x->neg) o[k++] = '-';
    k += (size_t)sprintf(o + k, "%llx", (unsigned long long)x->d[x->len - 1]);
    for (int i = x->len - 2; i >= 0; i--)
        k += (size_t)sprintf(o + k, "%016llx", (unsigned long long)x->d[i]);
    return k;
}

/*
 * Solve A x = b (A row-major n x n, b row-major n x c, int64).
 * nthreads >= 1.  max_steps < 0 runs to completion; otherwise elimination
 * stops after that many steps (used to time a bounded sample of the work).
 * Returns 0 and *out = malloc'd text "num den\n" per component (hex, row-major)
 * on success, 1 if A is singular, 2 if stopped by max_steps.  If step_seconds
 * is not NULL it receives the wall time of each elimination step that ran
 * (n doubles; only timing, the arithmetic is the same).
 */
int oracle_solve_timed(const int64_t *A, const int64_t *b, int n, int c, int nthreads,
                       int max_steps, char **out, double *step_seconds) {
    *out = NULL;
    if (n < 1 || c < 1 || nthreads < 1) return -1;
    job J;
    memset(&J, 0, sizeof J);
    J.n = n; J.c = c; J.T = nthreads; J.max_steps = max_steps;
    J.step_seconds = step_seconds;
    int W = n + c;
    J.M = (bz **)calloc((size_t)n, sizeof(bz *));
    for (int i = 0; i < n; i++) {
        J.M[i] = (bz *)calloc((size_t)W, sizeof(bz));
        for (int j = 0; j < n; j++) bz_set_i64(&J.M[i][j], A[(size_t)i * n + j]);
        for (int t = 0; t < c; t++) bz_set_i64(&J.M[i][n + t], b[(size_t)i * c + t]);
    }
    J.N = (bz *)calloc((size_t)n * c, sizeof(bz));
    J.num = (bz *)calloc((size_t)n * c, sizeof(bz));
    J.den = (bz *)calloc((size_t)n * c, sizeof(bz));
    J.partial = (bz *)calloc((size_t)nthreads, sizeof(bz));
    pthread_barrier_init(&J.bar, NULL, (unsigned)nthreads);
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    warg *wa = (warg *)calloc((size_t)nthreads, sizeof(warg));
    for (int t = 0; t < nthreads; t++) {
        wa[t].J = &J; wa[t].tid = t;
        if (t > 0) pthread_create(&th[t], NULL, worker, &wa[t]);
    }
    worker(&wa[0]);
    for (int t = 1; t < nthreads; t++) pthread_join(th[t], NULL);
    pthread_barrier_destroy(&J.bar);

    int status = J.singular ? 1 : (J.stopped ? 2 : 0);
    if (status == 0) {
        size_t cap = 64;
        for (int idx = 0; idx < n * c; idx++)
            cap += (size_t)(J.num[idx].len + J.den[idx].len + 2) * 16 + 8;
        char *o = (char *)malloc(cap);
        size_t k = 0;
        for (int idx = 0; idx < n * c; idx++) {
            k += put_hex(o + k, &J.num[idx]);
            o[k++] = ' ';
            k += put_hex(o + k, &J.den[idx]);
            o[k++] = '\n';
        }
        o[k] = 0;
        *out = o;
    }
    for (int i = 0; i < n; i++) {
        for (int j = 0; j < W; j++) bz_clear(&J.M[i][j]);
        free(J.M[i]);
    }
    free(J.M);
    for (int idx = 0; idx < n * c; idx++) { bz_clear(&J.N[idx]); bz_clear(&J.num[idx]); bz_clear(&J.den[idx]); }
    for (int t = 0; t < nthreads; t++) bz_clear(&J.partial[t]);
    free(J.N); free(J.num); free(J.den); free(J.partial);
    bz_clear(&J.d);
    free(th); free(wa);
    return status;
}

/* Same as oracle_solve_timed without the per-step timing. */
int oracle_solve(const int64_t *A, const int64_t *b, int n, int c, int nthreads,
                 int max_steps, char **out) {
    return oracle_solve_timed(A, b, n, c, nthreads, max_steps, out, NULL);
}

void oracle_free(char *p) { free(p); }

/* ------------------------------------------------------------------------
 * Test hooks: the exact division and the gcd on magnitudes given as
 * little-endian uint64 limbs, so the tests can check them against Python
 * integers.  The result is written to r (room for cap limbs), its length to
 * *lr.  oracle_dbg_divexact returns 0, or 1 when b does not divide a exactly;
 * oracle_dbg_gcd returns 0.  Both return -1 when b is zero (divexact) or the
 * result does not fit.
 */
static void bz_from_limbs(bz *x, const uint64_t *a, int la) {
    bz_reserve(x, la > 0 ? la : 1);
    if (la) memcpy(x->d, a, (size_t)la * sizeof(uint64_t));
    x->len = la;
    x->neg = 0;
    bz_norm(x);
}

int oracle_dbg_divexact(const uint64_t *a, int la, const uint64_t *b, int lb, uint64_t *r, int *lr, int cap) {
    bz A = {0}, B = {0}, Q = {0};
    scratch s;
    memset(&s, 0, sizeof s);
    bz_from_limbs(&A, a, la);
    bz_from_limbs(&B, b, lb);
    int rc = -1;
    if (B.len != 0) {
        rc = mag_divexact(&Q, &A, &B, &s) == 0 ? 0 : 1;
        if (rc == 0) {
            if (Q.len > cap) rc = -1;
            else { memcpy(r, Q.d, (size_t)Q.len * sizeof(uint64_t)); *lr = Q.len; }
        }
    }
    bz_clear(&A); bz_clear(&B); bz_clear(&Q);
    scratch_free(&s);
    return rc;
}

int oracle_dbg_gcd(const uint64_t *a, int la, const uint64_t *b, int lb, uint64_t *r, int *lr, int cap) {
    bz A = {0}, B = {0}, G = {0};
    scratch s;
    memset(&s, 0, sizeof s);
    bz_from_limbs(&A, a, la);
    bz_from_limbs(&B, b, lb);
    bz_gcd(&G, &A, &B, &s);
    int rc = 0;
    if (G.len > cap) rc = -1;
    else { if (G.len) memcpy(r, G.d, (size_t)G.len * sizeof(uint64_t)); *lr = G.len; }
    bz_clear(&A); bz_clear(&B); bz_clear(&G);
    scratch_free(&s);
    return rc;
}

/* ------------------------------------------------------------------------
 * Measurement hook for the CPU baseline: the wall time of one entry update of
 * the elimination -- the two products of L-limb numbers, their difference
 * and the exact division by an Lp-limb number -- averaged over `reps` updates
 * on each of `nthreads` threads that run at once (so the figure includes
 * what running every core costs each one).  The operands are arbitrary
 * numbers of those sizes, built as multiples of the divisor so that the
 * division is exact.  Returns the mean over the threads, in seconds.
 */
typedef struct {
    int L, Lp, reps;
    unsigned long long seed;
    double seconds;
} ubench_arg;

static uint64_t ub_next(unsigned long long *s) {
    /* xorshift64* */
    *s ^= *s >> 12; *s ^= *s << 25; *s ^= *s >> 27;
    return *s * 2685821657736338717ULL;
}

static void ub_random(bz *x, int limbs, unsigned long long *s) {
    bz_reserve(x, limbs);
    for (int i = 0; i < limbs; i++) x->d[i] = ub_next(s);
    x->d[limbs - 1] |= 1ULL << 62;
    x->len = limbs;
    x->neg = 0;
}

static void *ubench_worker(void *p) {
    ubench_arg *u = (ubench_arg *)p;
    scratch s;
    memset(&s, 0, sizeof s);
    bz prev = {0}, f1 = {0}, f2 = {0}, akk = {0}, aik = {0}, rij = {0}, rkj = {0}, a = {0}, b = {0}, q = {0};
    int Lf = u->L - u->Lp + 1 > 1 ? u->L - u->Lp + 1 : 1;
    ub_random(&prev, u->Lp, &u->seed);
    ub_random(&f1, Lf, &u->seed);
    ub_random(&f2, Lf, &u->seed);
    bz_mul(&akk, &prev, &f1, &s.t1);           /* akk, aik multiples of prev: the */
    bz_mul(&aik, &prev, &f2, &s.t1);           /* difference below divides exactly */
    ub_random(&rij, u->L, &u->seed);
    ub_random(&rkj, u->L, &u->seed);
    aik.neg = 1;
    double t0 = now_s();
    for (int r = 0; r < u->reps; r++) {
        bz_mul(&a, &akk, &rij, &s.t1);
        bz_mul(&b, &aik, &rkj, &s.t1);
        bz_addsub(&a, &a, &b, -1, &s.t1);
        bz_divexact(&q, &a, &prev, &s);
    }
    u->seconds = (now_s() - t0) / u->reps;
    bz_clear(&prev); bz_clear(&f1); bz_clear(&f2); bz_clear(&akk); bz_clear(&aik);
    bz_clear(&rij); bz_clear(&rkj); bz_clear(&a); bz_clear(&b); bz_clear(&q);
    scratch_free(&s);
    return NULL;
}

double oracle_entry_update_seconds(int L, int Lp, int reps, int nthreads) {
    if (L < 1 || Lp < 1 || Lp > L || reps < 1 || nthreads < 1) return -1.0;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    ubench_arg *ua = (ubench_arg *)calloc((size_t)nthreads, sizeof(ubench_arg));
    for (int t = 0; t < nthreads; t++) {
        ua[t].L = L; ua[t].Lp = Lp; ua[t].reps = reps;
        ua[t].seed = 0x9e3779b97f4a7c15ULL * (unsigned long long)(t + 1);
        if (t > 0) pthread_create(&th[t], NULL, ubench_worker, &ua[t]);
    }
    ubench_worker(&ua[0]);
    double sum = ua[0].seconds;
    for (int t = 1; t < nthreads; t++) {
        pthread_join(th[t], NULL);
        sum += ua[t].seconds;
    }
    free(th); free(ua);
    return sum / nthreads;
}
