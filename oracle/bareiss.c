/*
 * Exact rational solution of A x = b by fraction-free Bareiss elimination,
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
 * Big integers: sign-magnitude, 64-bit limbs, schoolbook multiplication,
 * Knuth's Algorithm D for division, Euclid for gcd.  Nothing is tuned.
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

static int clz64(uint64_t x) { return __builtin_clzll(x); }

/*
 * Knuth, TAOCP vol. 2, 4.3.1, Algorithm D on 64-bit limbs.
 * q gets la - lb + 1 limbs, rem gets lb limbs.  Requires lb >= 1, la >= lb,
 * b[lb-1] != 0.  Scratch: un (la + 1 limbs), vn (lb limbs).
 */
static void mag_divmod(uint64_t *q, uint64_t *rem, const uint64_t *a, int la,
                       const uint64_t *b, int lb, uint64_t *un, uint64_t *vn) {
    if (lb == 1) {
        uint64_t r = 0;
        for (int i = la - 1; i >= 0; i--) {
            u128 cur = ((u128)r << 64) | a[i];
            q[i] = (uint64_t)(cur / b[0]);
            r = (uint64_t)(cur % b[0]);
        }
        rem[0] = r;
        return;
    }
    int s = clz64(b[lb - 1]);
    for (int i = lb - 1; i > 0; i--)
        vn[i] = s ? (b[i] << s) | (b[i - 1] >> (64 - s)) : b[i];
    vn[0] = b[0] << s;
    un[la] = s ? a[la - 1] >> (64 - s) : 0;
    for (int i = la - 1; i > 0; i--)
        un[i] = s ? (a[i] << s) | (a[i - 1] >> (64 - s)) : a[i];
    un[0] = a[0] << s;

    for (int j = la - lb; j >= 0; j--) {
        u128 num = ((u128)un[j + lb] << 64) | un[j + lb - 1];
        u128 qhat = num / vn[lb - 1];
        u128 rhat = num % vn[lb - 1];
        while (qhat >> 64 || qhat * vn[lb - 2] > ((rhat << 64) | un[j + lb - 2])) {
            qhat--;
            rhat += vn[lb - 1];
            if (rhat >> 64) break;
        }
        /* multiply and subtract */
        uint64_t borrow = 0, carry = 0;
        for (int i = 0; i < lb; i++) {
            u128 p = qhat * vn[i] + carry;
            carry = (uint64_t)(p >> 64);
            uint64_t plo = (uint64_t)p;
            uint64_t t = un[i + j] - plo;
            uint64_t b1 = un[i + j] < plo;
            uint64_t t2 = t - borrow;
            uint64_t b2 = t < borrow;
            un[i + j] = t2;
            borrow = b1 | b2;
        }
        uint64_t top = un[j + lb];
        uint64_t t = top - carry;
        uint64_t b1 = top < carry;
        uint64_t t2 = t - borrow;
        uint64_t b2 = t < borrow;
        un[j + lb] = t2;
        if (b1 | b2) {
            /* qhat was one too large: add back */
            qhat--;
            uint64_t c = 0;
            for (int i = 0; i < lb; i++) {
                u128 sum = (u128)un[i + j] + vn[i] + c;
                un[i + j] = (uint64_t)sum;
                c = (uint64_t)(sum >> 64);
            }
            un[j + lb] += c;
        }
        q[j] = (uint64_t)qhat;
    }
    for (int i = 0; i < lb - 1; i++)
        rem[i] = s ? (un[i] >> s) | (un[i + 1] << (64 - s)) : un[i];
    rem[lb - 1] = un[lb - 1] >> s;
}

typedef struct {
    bz t1, t2, t3, un, vn;
} scratch;

static void scratch_free(scratch *s) {
    bz_clear(&s->t1); bz_clear(&s->t2); bz_clear(&s->t3); bz_clear(&s->un); bz_clear(&s->vn);
}

/* truncated division of magnitudes: q = |a| / |b|, r = |a| % |b| (signs set by caller) */
static void bz_divmod_mag(bz *q, bz *r, const bz *a, const bz *b, scratch *s) {
    if (b->len == 0) die("division by zero");
    if (mag_cmp(a->d, a->len, b->d, b->len) < 0) {
        if (q) { q->len = 0; q->neg = 0; }
        if (r) { bz_copy(r, a); r->neg = 0; }
        return;
    }
    int la = a->len, lb = b->len;
    bz_reserve(&s->un, la + 1);
    bz_reserve(&s->vn, lb);
    bz_reserve(&s->t2, la - lb + 1);
    bz_reserve(&s->t3, lb);
    mag_divmod(s->t2.d, s->t3.d, a->d, la, b->d, lb, s->un.d, s->vn.d);
    s->t2.len = la - lb + 1; s->t2.neg = 0; bz_norm(&s->t2);
    s->t3.len = lb; s->t3.neg = 0; bz_norm(&s->t3);
    if (q) bz_copy(q, &s->t2);
    if (r) bz_copy(r, &s->t3);
}

/* q = a / b, the division being exact (checked) */
static void bz_divexact(bz *q, const bz *a, const bz *b, scratch *s) {
    if (a->len == 0) { q->len = 0; q->neg = 0; return; }
    bz_reserve(&s->t1, 1);
    bz_divmod_mag(q, &s->t1, a, b, s);
    if (s->t1.len != 0) die("inexact division");
    int neg = a->neg ^ b->neg;
    q->neg = q->len ? neg : 0;
}

/* g = gcd(|a|, |b|) by Euclid's algorithm */
static void bz_gcd(bz *g, const bz *a, const bz *b, scratch *s) {
    bz x = {0}, y = {0}, r = {0};
    bz_copy(&x, a); x.neg = 0;
    bz_copy(&y, b); y.neg = 0;
    while (y.len != 0) {
        bz_divmod_mag(NULL, &r, &x, &y, s);
        bz_copy(&x, &y);
        bz_copy(&y, &r);
    }
    bz_copy(g, &x);
    bz_clear(&x); bz_clear(&y); bz_clear(&r);
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
