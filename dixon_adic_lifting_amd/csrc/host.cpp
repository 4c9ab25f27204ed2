// Host-side stages of the solver (see host.h).
//
// Prime set and step count follow the exact-solve card (phanerozoic/
// exact-solve), section "Method": P is a squarefree product of odd primes
// below 256 (odd so that P^-1 mod 2^64 exists), and the lift runs until P^m
// is larger than 2 N D, with N and D the Hadamard-type bounds on the
// numerators and the denominator.  Reconstruction follows the same section:
// the shared denominator is found from a few components, and each numerator
// then takes one product modulo P^m.
#include "host.h"

#include <sched.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <functional>
#include <mutex>
#include <thread>

#include "../../include/es_solve.h"

namespace es {

typedef unsigned __int128 u128;

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

LaunchEvents& pending_launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

static thread_local int g_krec_cap = 0;  // 0: the default record chunk

void set_lift_record_cap(int steps) { g_krec_cap = steps; }

int lift_record_steps(const Layout& L) { return g_krec_cap > 0 ? std::min(L.krec, g_krec_cap) : L.krec; }

Layout make_layout(int n, int c) {
    Layout L{};
    L.n = n;
    L.c = c;
    if (n <= 1024) {
        int p = 64;
        while (p < n) p <<= 1;
        L.pitch = p;
    } else {
        L.pitch = (int)align_up((size_t)n, 64);
    }
    L.lpr = std::min(64, L.pitch / 16);
    const size_t NC = (size_t)n * c;
    const size_t per_step = NC * kDigitLimbs * sizeof(uint64_t);
    size_t kc = ((size_t)64 << 20) / per_step;
    L.kchunk = (int)std::max<size_t>(1, std::min<size_t>(kc, 4096));
    const size_t E = kNumPrimes, nrb = ((size_t)n + 63) / 64;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    L.off_S = take(E * n * (size_t)L.pitch);
    L.off_piv = take(E * (n + 1) * sizeof(int32_t));
    L.off_rowpos = take(E * n * sizeof(int32_t));
    L.off_pend = take(2 * E * (size_t)L.pitch);
    L.off_GT = take(n <= 4096 ? E * (size_t)L.pitch * kPanel : 0);  // blocked elimination only
    L.off_flags = take(E * sizeof(int32_t));
    L.off_wq = take((size_t)work_queue_rows(n) * 8 * sizeof(int32_t));
    L.off_rowmax = take((size_t)n * sizeof(uint64_t));
    L.off_rownorm = take((size_t)n * sizeof(double));
    L.off_colpart = take(nrb * n * sizeof(double));
    L.off_colnorm = take((size_t)n * sizeof(double));
    L.off_bpart = take(nrb * c * sizeof(double));
    L.off_bnorm = take((size_t)c * sizeof(double));
    L.off_A32 = take((size_t)n * n * sizeof(int32_t));
    L.off_R = take(NC * sizeof(int64_t));
    L.off_rho = take(E * c * (size_t)L.pitch);
    L.off_U = take(E * NC);
    L.off_xlow = take(NC * sizeof(uint64_t));
    L.off_rpos = take(c == 1 ? (size_t)n * 64 * sizeof(int32_t) : 0);
    L.off_Ab = take(c > 1 ? 4 * (size_t)n * L.pitch : 0);
    L.off_xp = take(c > 1 ? 8 * (size_t)c * L.pitch : 0);
    const bool fused = fused_lift_shape(n, c, L.pitch);
    L.off_Sperm = take(fused ? E * n * (size_t)L.pitch : 0);
    const size_t kr = std::min<size_t>(((size_t)16 << 20) / ((size_t)n * 64), (size_t)L.kchunk);
    L.krec = (int)std::max<size_t>(1, kr);
    L.off_urec = take(fused ? (size_t)L.krec * n * 64 : 0);
    L.off_digits = take(NC * (size_t)L.kchunk * kDigitLimbs * sizeof(uint64_t));
    L.off_params = take(sizeof(LiftParams));
    L.total = o;
    return L;
}

size_t inverse_bytes(const Layout& L) {
    return align_up(L.off_rho + (size_t)kNumPrimes * L.c * L.pitch, 256);
}

// ---------------------------------------------------------------- primes

LiveSet make_live_set(const int* flags) {
    LiveSet ls;
    ls.P = BigInt::from_u64(1);
    for (int j = 0; j < kNumPrimes; j++) {
        if (flags[j]) continue;
        ls.idx[ls.E++] = j;
        ls.P = mul_small(ls.P, kPrimeTable.q[j]);
    }
    // P^-1 mod 2^64 by Newton's iteration x <- x (2 - P x); P x = 1 mod 8 at x = P
    uint64_t p0 = ls.P.is_zero() ? 1 : ls.P.d[0];
    uint64_t x = p0;
    for (int it = 0; it < 6; it++) x *= 2 - p0 * x;
    ls.Pinv = x;
    return ls;
}

LiveSet live_set_from_mask(uint64_t mask) {
    int flags[kNumPrimes];
    for (int j = 0; j < kNumPrimes; j++) flags[j] = ((mask >> j) & 1) ? 0 : 1;
    return make_live_set(flags);
}

static uint32_t inv_mod_small(uint32_t a, uint32_t q) {
    // extended Euclid on small integers
    int64_t t0 = 0, t1 = 1, r0 = q, r1 = a % q;
    while (r1) {
        int64_t qt = r0 / r1, tmp;
        tmp = r0 - qt * r1; r0 = r1; r1 = tmp;
        tmp = t0 - qt * t1; t0 = t1; t1 = tmp;
    }
    return (uint32_t)((t0 % (int64_t)q + q) % q);
}

void fill_lift_params(const LiveSet& ls, LiftParams* prm) {
    std::memset(prm, 0, sizeof *prm);
    prm->E = ls.E;
    prm->Pinv = ls.Pinv;
    for (int l = 0; l < ls.E; l++) {
        const int j = ls.idx[l];
        prm->qidx[l] = (uint32_t)j;
        prm->q[l] = kPrimeTable.q[j];
        prm->mu16[l] = kPrimeTable.mu16[j];
        prm->mu32[l] = kPrimeTable.mu32[j];
        prm->r32[l] = kPrimeTable.r32[j];
    }
    // CRT constants: W_l = P / q_l, its inverse mod q_l, the words of P and
    // of (P - 1) / 2
    BigInt P = BigInt::from_u64(1);
    for (int l = 0; l < ls.E; l++) P = mul_small(P, prm->q[l]);
    auto word = [](const BigInt& v, int w) -> uint32_t {
        const size_t limb = (size_t)w / 2;
        const uint64_t x = limb < v.size() ? v.d[limb] : 0;
        return (uint32_t)(w % 2 ? x >> 32 : x);
    };
    for (int l = 0; l < ls.E; l++) {
        const uint32_t q = prm->q[l];
        const BigInt W = divexact(P, BigInt::from_u64(q));
        uint64_t wmod = 0;  // W mod q, from the words
        for (int w = kDigitWords - 1; w >= 0; w--) wmod = ((wmod << 32) | word(W, w)) % q;
        prm->cinv[l] = (uint32_t)inv_mod_small((uint32_t)wmod, q);
        prm->qrec[l] = 1.0 / (double)q;
        for (int w = 0; w < kDigitWords; w++) prm->Wd[l][w] = (double)word(W, w);
    }
    const BigInt Ph = shr_abs(P, 1);
    for (int w = 0; w < kDigitWords; w++) {
        prm->Pw[w] = word(P, w);
        prm->Phw[w] = word(Ph, w);
    }
}

// ---------------------------------------------------------------- bounds

void hadamard_bits(const double* rownorm, const double* colnorm, const double* bnorm, int n, int c,
                   int* nbits, int* dbits) {
    double lr = 0, lc = 0, lcmin = INFINITY, lb = -INFINITY;
    for (int i = 0; i < n; i++) lr += 0.5 * std::log2(rownorm[i]);
    for (int j = 0; j < n; j++) {
        double v = 0.5 * std::log2(colnorm[j]);
        lc += v;
        lcmin = std::min(lcmin, v);
    }
    for (int t = 0; t < c; t++)
        if (bnorm[t] > 0) lb = std::max(lb, 0.5 * std::log2(bnorm[t]));
    // |det A| <= min(prod row norms, prod column norms); each numerator is a
    // determinant with one column replaced by a column of b (Cramer), so
    // |num| <= ||b_t|| prod_j ||A_j|| / min_j ||A_j||.  Two bits of margin
    // absorb the rounding of the fp64 sums and logarithms.
    const double ld = std::min(lr, lc);
    *dbits = std::max(1, (int)std::ceil(ld + 2.0));
    if (lb == -INFINITY) {
        *nbits = 1;  // b = 0: every numerator is 0
    } else {
        const double ln = lb + lc - lcmin;
        *nbits = std::max(1, (int)std::ceil(ln + 2.0));
    }
}

int choose_m(const BigInt& P, int nbits, int dbits, BigInt* M) {
    // P^m > 2^B with B = nbits + dbits + 1 holds exactly when the odd number
    // P^m has bit length >= B + 1.  Start from a float estimate just below
    // and confirm with exact powers.
    const size_t need = (size_t)nbits + dbits + 2;
    const size_t bl = P.bit_length();
    const BigInt top = shr_abs(P, bl > 64 ? bl - 64 : 0);
    const double l2p = std::log2((double)top.d[0]) + (double)(bl > 64 ? bl - 64 : 0);
    int m = std::max(1, (int)std::floor((double)need / l2p) - 1);
    BigInt Pm = pow_u(P, (unsigned)m);
    while (Pm.bit_length() < need) {
        Pm = mul(Pm, P);
        m++;
    }
    *M = std::move(Pm);
    return m;
}

int choose_m_bits(const BigInt& P, int nbits, int dbits, size_t* mbits) {
    // The same m without forming P^m: P^k has bit length floor(k log2 P) + 1.
    // log2 P from P's top 64 bits is within about 1e-13 (the rounding of the
    // top word to a double and of log2 itself), so k log2 P is within 2e-9
    // for k up to 2^14; where it lies within 1e-6 of an integer the exact
    // power decides.
    const size_t need = (size_t)nbits + dbits + 2;
    const size_t bl = P.bit_length();
    const BigInt top = shr_abs(P, bl > 64 ? bl - 64 : 0);
    const double l2p = std::log2((double)top.d[0]) + (double)(bl > 64 ? bl - 64 : 0);
    auto bits = [&](int k, size_t* out) {
        const double x = (double)k * l2p, f = std::floor(x);
        if (x - f < 1e-6 || f + 1.0 - x < 1e-6 || k > (1 << 14)) return false;
        *out = (size_t)f + 1;
        return true;
    };
    auto exact = [&]() {
        BigInt M;
        const int m = choose_m(P, nbits, dbits, &M);
        *mbits = M.bit_length();
        return m;
    };
    int m = std::max(1, (int)std::floor((double)(need - 1) / l2p));
    size_t b = 0;
    for (;;) {
        if (!bits(m, &b)) return exact();
        if (b >= need) break;
        m++;
    }
    while (m > 1) {
        size_t b1;
        if (!bits(m - 1, &b1)) return exact();
        if (b1 < need) break;
        m--, b = b1;
    }
    *mbits = b;
    return m;
}

// ---------------------------------------------------------------- singular decision

static uint64_t mulmod62(uint64_t a, uint64_t b, uint64_t p) { return (uint64_t)((u128)a * b % p); }

static uint64_t powmod62(uint64_t a, uint64_t e, uint64_t p) {
    uint64_t r = 1;
    while (e) {
        if (e & 1) r = mulmod62(r, a, p);
        a = mulmod62(a, a, p);
        e >>= 1;
    }
    return r;
}

bool full_rank_mod(const int64_t* A, int n, uint64_t p) {
    std::vector<uint64_t> M((size_t)n * n);
    for (size_t i = 0; i < (size_t)n * n; i++) {
        int64_t v = A[i];
        uint64_t u = v < 0 ? (uint64_t)0 - (uint64_t)v : (uint64_t)v;
        u %= p;
        M[i] = (v < 0 && u) ? p - u : u;
    }
    for (int k = 0; k < n; k++) {
        int piv = -1;
        for (int i = k; i < n; i++)
            if (M[(size_t)i * n + k]) { piv = i; break; }
        if (piv < 0) return false;
        if (piv != k)
            for (int j = 0; j < n; j++) std::swap(M[(size_t)k * n + j], M[(size_t)piv * n + j]);
        const uint64_t inv = powmod62(M[(size_t)k * n + k], p - 2, p);
        for (int i = k + 1; i < n; i++) {
            const uint64_t f = mulmod62(M[(size_t)i * n + k], inv, p);
            if (!f) continue;
            for (int j = k; j < n; j++) {
                uint64_t t = mulmod62(f, M[(size_t)k * n + j], p);
                uint64_t& x = M[(size_t)i * n + j];
                x = x >= t ? x - t : x + p - t;
            }
        }
    }
    return true;
}

// ---------------------------------------------------------------- reconstruction

int default_threads() {
    if (const char* e = std::getenv("ES_THREADS")) {
        int v = std::atoi(e);
        if (v > 0) return v;
    }
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        int cnt = CPU_COUNT(&set);
        if (cnt > 0) return cnt;
    }
    unsigned h = std::thread::hardware_concurrency();
    return h ? (int)h : 1;
}

// A pool of worker threads started on first use and kept for the life of
// the process (thread start-up costs far more than the short host phases of
// a solve).  One job at a time: a caller that finds the pool busy, or that
// is itself a pool worker, runs its loop alone.  The caller works on its
// own job and returns once every item is done, without waiting for workers
// that have not woken yet (a wake-up can take tens of microseconds): items
// are claimed through a ticket that carries the job's generation, so a late
// worker finds the ticket moved on and claims nothing.  Items are claimed a
// chunk at a time (a quarter of an even share), so that short items do not
// queue on the ticket, and a worker that has finished a job watches for the
// next one for a short while before it sleeps (the host phases of a solve
// come in quick succession).  The first exception thrown by the loop body
// is rethrown in the caller (the items after it are skipped).
namespace {
thread_local bool t_pool_worker = false;

struct ThreadPool {
    static constexpr int64_t kWatchNs = 60000;  // how long an idle worker watches for the next job
    std::mutex mu, serial;
    std::condition_variable cv_work, cv_done;
    uint32_t gen = 0;                  // current job (under mu)
    std::atomic<uint32_t> pub{0};      // gen, for workers watching without the lock
    const std::function<void(size_t)>* job = nullptr;
    size_t count = 0, chunk = 1;
    std::atomic<uint64_t> ticket{0};  // gen << 32 | next item
    std::atomic<size_t> done{0};      // items of the current job finished or skipped
    std::atomic<bool> stop{false};
    std::exception_ptr error;
    const int workers;

    explicit ThreadPool(int n) : workers(n) {
        for (int i = 0; i < n; i++) std::thread([this] { run(); }).detach();
    }
    // claims and runs chunks of job g until none is left
    void drain(uint32_t g, const std::function<void(size_t)>* f, size_t cnt, size_t ch) {
        for (;;) {
            uint64_t t = ticket.load(std::memory_order_acquire);
            const size_t i0 = (size_t)(uint32_t)t;
            if ((uint32_t)(t >> 32) != g || i0 >= cnt) return;
            const size_t i1 = std::min(cnt, i0 + ch);
            if (!ticket.compare_exchange_weak(t, ((uint64_t)g << 32) | (uint64_t)i1, std::memory_order_acq_rel))
                continue;
            for (size_t i = i0; i < i1; i++) {
                if (stop.load(std::memory_order_relaxed)) break;
                try {
                    (*f)(i);
                } catch (...) {
                    std::lock_guard<std::mutex> lk(mu);
                    if (!error) error = std::current_exception();
                    stop = true;
                }
            }
            if (done.fetch_add(i1 - i0, std::memory_order_acq_rel) + (i1 - i0) == cnt) {
                std::lock_guard<std::mutex> lk(mu);
                cv_done.notify_all();
            }
        }
    }
    void run() {
        t_pool_worker = true;
        uint32_t seen = 0;
        for (;;) {
            // watch for the next job a while, then sleep until one comes
            const auto t0 = std::chrono::steady_clock::now();
            for (int k = 0; pub.load(std::memory_order_acquire) == seen; k++) {
                __builtin_ia32_pause();
                if ((k & 255) == 255 &&
                    std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0)
                            .count() > kWatchNs)
                    break;
            }
            const std::function<void(size_t)>* f;
            size_t cnt, ch;
            uint32_t g;
            {
                std::unique_lock<std::mutex> lk(mu);
                cv_work.wait(lk, [&] { return gen != seen; });
                seen = g = gen;
                f = job;
                cnt = count;
                ch = chunk;
            }
            // *f is only used for an item claimed under generation g, and
            // the caller waits for every such item: it is still alive then
            drain(g, f, cnt, ch);
        }
    }
    // false when the pool is busy with another caller's job
    bool parallel(size_t cnt, const std::function<void(size_t)>& f, size_t grain) {
        if (cnt >= ((size_t)1 << 32)) return false;
        std::unique_lock<std::mutex> one(serial, std::try_to_lock);
        if (!one.owns_lock()) return false;
        uint32_t g;
        const size_t ch = grain > 0 ? grain : std::max<size_t>(1, cnt / (4 * (size_t)(workers + 1)));
        {
            std::lock_guard<std::mutex> lk(mu);
            job = &f;
            count = cnt;
            chunk = ch;
            done = 0;
            stop = false;
            error = nullptr;
            g = ++gen;
            ticket.store((uint64_t)g << 32, std::memory_order_release);
            pub.store(g, std::memory_order_release);
        }
        cv_work.notify_all();
        drain(g, &f, cnt, ch);
        std::exception_ptr e;
        {
            std::unique_lock<std::mutex> lk(mu);
            cv_done.wait(lk, [&] { return done.load(std::memory_order_acquire) >= cnt; });
            e = error;
            error = nullptr;
        }
        if (e) std::rethrow_exception(e);
        return true;
    }
};

ThreadPool* pool() {
    // never destroyed: its workers wait on it until the process ends.  A
    // forked child has none of the parent's workers and starts its own pool.
    static std::mutex mu;
    static ThreadPool* p = nullptr;
    static pid_t owner = 0;
    std::lock_guard<std::mutex> lk(mu);
    if (!p || owner != getpid()) {
        p = new ThreadPool(std::max(0, default_threads() - 1));
        owner = getpid();
    }
    return p;
}
}  // namespace

template <class F>
static void parallel_for(size_t count, int nthreads, F&& fn, size_t grain = 0) {
    if (count == 0) return;
    if (nthreads > 1 && count > 1 && !t_pool_worker) {
        const std::function<void(size_t)> f = fn;
        if (pool()->parallel(count, f, grain)) return;
    }
    for (size_t i = 0; i < count; i++) fn(i);
}

// X = sum_{i<m} x_i P^i from balanced 384-bit two's-complement digits (Horner).
BigInt assemble(const int64_t* dig, int m, const BigInt& P) {
    BigInt X;
    for (int i = m - 1; i >= 0; i--)
        X = add(mul(X, P), BigInt::from_twos((const uint64_t*)(dig + (size_t)i * kDigitLimbs), kDigitLimbs));
    return X;
}

// digits [lo, hi) as sum_i x_i P^(i - lo): halves joined by one product with
// a power of P, so the long products are balanced (and use Karatsuba)
static BigInt assemble_range(const int64_t* dig, int lo, int hi, const std::vector<BigInt>& pw) {
    if (hi - lo <= 8) {
        BigInt X;
        for (int i = hi - 1; i >= lo; i--)
            X = add(mul(X, pw[1]),
                    BigInt::from_twos((const uint64_t*)(dig + (size_t)i * kDigitLimbs), kDigitLimbs));
        return X;
    }
    const int mid = lo + (hi - lo) / 2;
    return add(assemble_range(dig, lo, mid, pw), mul(pw[mid - lo], assemble_range(dig, mid, hi, pw)));
}

BigInt assemble(const int64_t* dig, int m, const std::vector<BigInt>& pw) {
    if (m < 1) return BigInt();
    if (pw.size() < 2 || (int)pw.size() <= m / 2 + 1) return assemble(dig, m, pw.empty() ? BigInt() : pw.back());
    return assemble_range(dig, 0, m, pw);
}

void assemble_split(const int64_t* dig, size_t stride, size_t count, int m, const std::vector<BigInt>& pw,
                    int parts, int nthreads, BigInt* out) {
    if (m < 1 || count == 0) return;
    if (parts < 2 || m < 8 * parts || (int)pw.size() <= m) {
        parallel_for(count, nthreads, [&](size_t k) { out[k] = assemble(dig + k * stride, m, pw); });
        return;
    }
    // ranges [m q / parts, m (q + 1) / parts), then pairs joined level by
    // level: the left part plus P^(start of right - start of left) times the right
    std::vector<BigInt> X(count * (size_t)parts);
    std::vector<int> start(parts + 1);
    for (int q = 0; q <= parts; q++) start[q] = (int)((long)m * q / parts);
    parallel_for(X.size(), nthreads, [&](size_t t) {
        const size_t k = t / parts;
        const int q = (int)(t % parts);
        X[t] = assemble_range(dig + k * stride, start[q], start[q + 1], pw);
    });
    for (int w = 1; w < parts; w *= 2) {
        const size_t joins = count * (size_t)(parts / (2 * w));
        parallel_for(joins, nthreads, [&](size_t t) {
            const size_t k = t / (parts / (2 * w));
            const int q = (int)(t % (parts / (2 * w))) * 2 * w;
            BigInt& left = X[k * parts + q];
            left = add(left, mul(pw[start[q + w] - start[q]], X[k * parts + q + w]));
        });
    }
    for (size_t k = 0; k < count; k++) out[k] = std::move(X[k * parts]);
}

static bool verbose() {
    static const bool v = [] {
        const char* e = std::getenv("ES_VERBOSE");
        return e && *e && *e != '0';
    }();
    return v;
}

void parallel_for_each(size_t count, int nthreads, const std::function<void(size_t)>& fn, size_t grain) {
    parallel_for(count, nthreads, fn, grain);
}

std::vector<size_t> sample_indices(size_t NC, int c) {
    // the first row (one component of every right-hand side: their
    // denominators can differ), then eight components spread over the rows,
    // the k-th at index floor(k NC / 8) + (k mod c)
    std::vector<size_t> sample;
    for (size_t t = 0; t < (size_t)c && t < NC; t++) sample.push_back(t);
    for (size_t k = 1; k < 8; k++) {
        const size_t j = k * NC / 8 + k % (size_t)c;
        if (j >= (size_t)c && j < NC && std::find(sample.begin(), sample.end(), j) == sample.end())
            sample.push_back(j);
    }
    return sample;
}

bool sample_denominator(const std::vector<BigInt>& xs, const BigInt& M, int nbits, int dbits, int nthreads,
                        BigInt* d) {
    const BigInt Nb = shl(BigInt::from_u64(1), (size_t)nbits);
    const BigInt Db = shl(BigInt::from_u64(1), (size_t)dbits);
    std::vector<BigInt> sden(xs.size());
    std::atomic<int> bad{0};
    // a second thread per reconstruction only while the samples leave most
    // cores idle (both threads of every sample busy otherwise crowd them out)
    const bool split = 4 * xs.size() <= (size_t)nthreads;
    parallel_for(xs.size(), nthreads, [&](size_t s) {
        // the remainder / cofactor pair where the Euclidean sequence first
        // drops to N: its cofactor is x's denominator (a solution within the
        // bounds exists), and every numerator formed with d is checked
        // against N afterwards, so the coprimality test is not needed here
        BigInt a = mod_floor(xs[s], M), nu, de;
        if (!rational_reconstruct(a, M, Nb, Db, &nu, &de, false, split)) bad = 1;
        else sden[s] = de;
    });
    if (bad) return false;
    *d = BigInt::from_u64(1);
    for (auto& v : sden) *d = lcm(*d, v);
    return true;
}

int reconstruct(const int64_t* digits, size_t stride_m, int n, int c, int m, const BigInt& P,
                const BigInt& M, int nbits, int dbits, int nthreads, SolutionData* out) {
    const size_t NC = (size_t)n * c;
    typedef std::chrono::steady_clock clk;
    auto t0 = clk::now();
    auto lap = [&](const char* what) {
        if (!verbose()) return;
        auto t1 = clk::now();
        fprintf(stderr, "[es] reconstruct %-10s %8.3f ms\n", what,
                std::chrono::duration<double, std::milli>(t1 - t0).count());
        t0 = t1;
    };
    std::vector<BigInt> X(NC);
    parallel_for(NC, nthreads, [&](size_t j) { X[j] = assemble(digits + j * stride_m * kDigitLimbs, m, P); });
    lap("assemble");
    const BigInt Nb = shl(BigInt::from_u64(1), (size_t)nbits);
    const BigInt Db = shl(BigInt::from_u64(1), (size_t)dbits);
    BigInt Mhalf = shr_abs(M, 1);

    // common denominator from the sample
    std::vector<BigInt> xs;
    for (size_t j : sample_indices(NC, c)) xs.push_back(X[j]);
    BigInt d;
    if (!sample_denominator(xs, M, nbits, dbits, nthreads, &d)) return ES_EINTERNAL;
    lap("sample");

    out->n = n;
    out->c = c;
    out->num.assign(NC, BigInt());
    out->dens.assign(1, d);  // entry 0: d itself
    out->den_of.assign(NC, 0);
    std::vector<BigInt> own(NC);  // a component's own denominator (when not d)
    std::vector<char> failed(NC, 0);
    parallel_for(NC, nthreads, [&](size_t j) {
        BigInt y = mod_floor(mul(d, X[j]), M);
        if (cmp_abs(y, Mhalf) > 0) y = sub(y, M);  // balanced representative
        if (cmp_abs(y, Nb) > 0) {
            failed[j] = 1;
            return;
        }
        BigInt g = gcd(y, d);
        if (g.size() == 1 && g.d[0] == 1) {
            out->num[j] = y;
            return;
        }
        out->num[j] = divexact(y, g);
        own[j] = divexact(d, g);
    });
    lap("numerators");
    for (size_t j = 0; j < NC; j++) {
        if (failed[j]) {
            BigInt a = mod_floor(X[j], M), nu;
            if (!rational_reconstruct(a, M, Nb, Db, &nu, &own[j])) return ES_EINTERNAL;
            out->num[j] = nu;
        }
        if (own[j].is_zero()) continue;
        out->den_of[j] = (uint32_t)out->dens.size();
        out->dens.push_back(std::move(own[j]));
    }
    return ES_OK;
}

}  // namespace es
