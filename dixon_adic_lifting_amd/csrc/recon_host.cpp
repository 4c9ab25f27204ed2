// Host side of the GPU reconstruction path (kernels in recon.hip).
//
// Method (exact-solve card, phanerozoic/exact-solve, section "Method"): the
// denominator d shared by the components is found from a few of them (Wang
// reconstruction on the host), then each numerator is one modular multiply
// y = d X mods M, accepted when |y| <= N, and reduced to lowest terms by
// gcd(y, d).  The modular multiplies of all components run on the GPU as one
// int8 GEMM against weights 256^b P^i d mod M; this file computes the weight
// seeds P^i d mod M, drives the kernels, and finishes each component.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <thread>
#include <stdexcept>
#include <vector>

#include "../../include/es_solve.h"
#include "es_internal.h"
#include "host.h"
#include "recon_host.h"

namespace es {

namespace {

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Pinned host staging for the device-to-host copies, per thread.
struct PinnedStage {
    void* p = nullptr;
    size_t bytes = 0;
    ~PinnedStage() {
        if (p) (void)hipHostFree(p);
    }
    void* get(size_t need) {
        if (need <= bytes) return p;
        if (p) (void)hipHostFree(p);
        p = nullptr;
        bytes = 0;
        if (hipHostMalloc(&p, need, hipHostMallocDefault) != hipSuccess) {
            p = nullptr;
            return nullptr;
        }
        bytes = need;
        return p;
    }
};
thread_local PinnedStage g_pinned_stage;

// A second stream for the numerator words' copies to the host, per thread
// (kept until the process ends; default priority): the gcd kernel reads the
// same words on the solve's stream meanwhile.
struct CopyStream {
    hipStream_t s = nullptr;
    hipStream_t get() {
        if (!s && hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) s = nullptr;
        return s;
    }
};
thread_local CopyStream g_copy_stream;

// Marks the arrival of the numerator words on the host, per thread (kept
// until the process ends).
struct ReadyEvent {
    hipEvent_t e = nullptr;
    hipEvent_t get() {
        if (!e && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) e = nullptr;
        return e;
    }
};
thread_local ReadyEvent g_words_ready;
// Marks the arrival on the host of the first gcd launch's results.
thread_local ReadyEvent g_first_gcds;
// Marks a chunk's numerators on the device, for the copy stream to wait on.
thread_local ReadyEvent g_numer_done;

// little-endian 32-bit words of a nonnegative BigInt, zero-padded to nw
void to_words(const BigInt& v, uint32_t* w, int nw) {
    for (int i = 0; i < nw; i++) {
        const size_t limb = (size_t)i / 2;
        const uint64_t x = limb < v.size() ? v.d[limb] : 0;
        w[i] = (uint32_t)(i % 2 ? x >> 32 : x);
    }
}

// signed integer from nw two's-complement words (negative when neg)
BigInt from_words(const uint32_t* w, int nw, bool neg) {
    std::vector<uint32_t> mag(w, w + nw);
    if (neg) {  // magnitude = 2^(32 nw) - value
        uint64_t carry = 1;
        for (int i = 0; i < nw; i++) {
            const uint64_t v = (uint64_t)(uint32_t)~mag[i] + carry;
            mag[i] = (uint32_t)v;
            carry = v >> 32;
        }
    }
    BigInt r;
    r.d.resize((size_t)(nw + 1) / 2);
    for (int i = 0; i < nw; i++) r.d[(size_t)i / 2] |= (uint64_t)mag[i] << (32 * (i % 2));
    r.trim();
    r.neg = neg && !r.is_zero();
    return r;
}

// floor(a / b) for a >= 0, b > 0
BigInt shr_pow(const BigInt& a, const BigInt& b) {
    BigInt q;
    divmod_trunc(a, b, &q, nullptr);
    return q;
}

// t <- P t - q M, for t of n limbs (zero padded) in [0, M) and the quotient
// q = floor(P t / M), so that the result lies in [0, M) too (n = M's limbs):
// one pass over the columns with a signed three-word accumulator, the old
// limbs of t the column needs kept in a ring.  Throws if the result does
// not fit (a wrong q).
void seed_step(uint64_t* t, size_t n, const uint64_t* p, size_t lp, const uint64_t* q, size_t lq,
               const uint64_t* M) {
    typedef unsigned __int128 u128;
    if (lp > 8) throw std::logic_error("seed multiplier too wide");
    uint64_t old[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // old[k] = t[i - k] before this step
    uint64_t a0 = 0, a1 = 0;
    int64_t a2 = 0;
    const size_t cols = n + std::max(lp, lq) + 1;
    for (size_t i = 0; i < cols; i++) {
        for (size_t k = lp - 1; k > 0; k--) old[k] = old[k - 1];
        old[0] = i < n ? t[i] : 0;
        for (size_t k = 0; k < lp && k <= i; k++) {
            const u128 pr = (u128)p[k] * old[k];
            const u128 s0 = (u128)a0 + (uint64_t)pr;
            a0 = (uint64_t)s0;
            const u128 s1 = (u128)a1 + (uint64_t)(pr >> 64) + (uint64_t)(s0 >> 64);
            a1 = (uint64_t)s1;
            a2 += (int64_t)(uint64_t)(s1 >> 64);
        }
        for (size_t k = 0; k < lq && k <= i; k++) {
            if (i - k >= n) continue;
            const u128 pr = (u128)q[k] * M[i - k];
            const uint64_t lo = (uint64_t)pr, hi = (uint64_t)(pr >> 64);
            const uint64_t b0 = a0 < lo;
            a0 -= lo;
            const u128 sub = (u128)hi + b0;
            const uint64_t b1 = (u128)a1 < sub;
            a1 = (uint64_t)((u128)a1 - sub);
            a2 -= (int64_t)b1;
        }
        if (i < n) t[i] = a0;
        else if (a0 != 0) throw std::logic_error("seed step out of range");
        a0 = a1;
        a1 = (uint64_t)a2;
        a2 = a2 < 0 ? -1 : 0;
    }
    if (a0 != 0 || a1 != 0 || a2 != 0) throw std::logic_error("seed step out of range");
}

bool verbose() {
    static const bool v = [] {
        const char* e = std::getenv("ES_VERBOSE");
        return e && *e && *e != '0';
    }();
    return v;
}

}  // namespace

namespace {
thread_local int g_gpu_recon = -1;  // -1: not set on this thread (environment decides)
}

void set_gpu_recon(bool on) { g_gpu_recon = on ? 1 : 0; }

bool gpu_recon_disabled() {
    static const bool env_off = [] {
        const char* e = std::getenv("ES_RECON");
        return e && std::strcmp(e, "host") == 0;
    }();
    return g_gpu_recon < 0 ? env_off : g_gpu_recon == 0;
}

GpuReconPlan plan_gpu_recon(int n, int c, int m, size_t mbits, int nbits) {
    GpuReconPlan pl;
    pl.n = n;
    pl.c = c;
    pl.m = m;
    pl.NC = (size_t)n * c;
    // words 0 .. TM hold every value in [0, 2M) (weights and numerators are
    // kept in that range), so M's own top word may be zero: the three-word
    // windows of M below then still carry at least 63 bits
    pl.TM = (int)(mbits / 32);
    pl.NW = pl.TM + 1;
    pl.nw = nbits / 32 + 1;
    // the quotient window needs three words of M; a weight row must fit one
    // wave; 48 m contraction bytes keep every GEMM column sum within int32
    if (pl.TM < 2 || wchain_words_per_lane(pl.NW) == 0 || numer_words_per_lane(pl.NW) == 0 || 48 * (size_t)m > 65536 ||
        pl.nw > pl.NW)
        return pl;
    pl.Ncolsp = (int)round_up((size_t)4 * pl.NW, 256);
    pl.Kpad = (int)round_up((size_t)48 * m, 192);
    pl.NCc = (int)std::min<size_t>(pl.NC, 8192);
    pl.NCcp = (int)round_up((size_t)pl.NCc, 128);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = round_up(o + bytes, 256);
        return at;
    };
    pl.off_digits = take(pl.NC * (size_t)m * kDigitLimbs * sizeof(uint64_t));
    pl.off_S = take((size_t)pl.NCcp * pl.Kpad);
    pl.off_rowsum = take((size_t)pl.NCcp * sizeof(int));
    pl.off_T = take((size_t)m * pl.NW * sizeof(uint32_t));
    pl.off_Mw = take((size_t)pl.NW * sizeof(uint32_t));
    pl.off_W = take((size_t)pl.Kpad * pl.Ncolsp);
    pl.off_WT = take((size_t)pl.Kpad * pl.Ncolsp);
    pl.off_VT = take((size_t)pl.Ncolsp * pl.NCcp * sizeof(int));
    // numerators, their status and the gcds for every component: the GEMM
    // runs chunk by chunk, the gcd kernel once over all of them
    const size_t NCp = round_up(pl.NC, 128);
    pl.off_Y = take(NCp * pl.nw * sizeof(uint32_t));
    pl.off_status = take(NCp * sizeof(int));
    pl.off_Dw = take((size_t)pl.NW * sizeof(uint32_t));
    pl.off_G = take(NCp * sizeof(uint64_t));
    pl.off_gstat = take(NCp * sizeof(int));
    pl.total = o;
    pl.ok = pl.total <= ((size_t)16 << 30);
    return pl;
}

size_t gpu_recon_reserve(int n, int c) {
    // The largest bounds within the range limit n max|A| < 2^63: every entry
    // of A at 2^63 / n and every entry of b at 2^63 in magnitude.
    const double amax = std::ldexp(1.0, 63) / n;
    std::vector<double> an((size_t)n, (double)n * amax * amax), bn((size_t)c, (double)n * std::ldexp(1.0, 126));
    int nb = 0, db = 0;
    hadamard_bits(an.data(), an.data(), bn.data(), n, c, &nb, &db);
    // The smallest P with at most kReserveDrops primes dropped: the product
    // of the others, the largest ones dropped.
    BigInt P = BigInt::from_u64(1);
    for (int j = 0; j < kNumPrimes - kReserveDrops; j++) P = mul_small(P, kPrimeTable.q[j]);
    const double l2p = std::log2((double)shr_abs(P, P.bit_length() - 64).d[0]) + (double)(P.bit_length() - 64);
    const size_t need = (size_t)nb + db + 2;
    // The least m with P^m of bit length >= need has P^(m - 1) < 2^need, so
    // M = P^m < 2^need P: at most need + 334 bits whatever the live primes.
    size_t mb = need + 335;
    // the widest M the GPU path takes (its weight and numerator rows fit one wave)
    size_t mb_cap = 0;
    for (size_t w = 3; wchain_words_per_lane((int)w) != 0 && numer_words_per_lane((int)w) != 0; w++)
        mb_cap = 32 * w - 1;
    mb = std::min(mb, mb_cap);
    // steps for any P at least as large, at the capped width
    int m = (int)std::min<double>(std::ceil((double)need / l2p) + 1.0, std::floor((double)mb / l2p) + 2.0);
    m = std::min(m, 65536 / 48);
    nb = (int)std::min<size_t>((size_t)nb, mb);
    const GpuReconPlan pl = plan_gpu_recon(n, c, m, mb, nb);
    return pl.ok ? pl.total : 0;
}

#define HIPOK(expr)                                   \
    do {                                              \
        if ((expr) != hipSuccess) return ES_EHIP;     \
    } while (0)

int reconstruct_gpu(const GpuReconPlan& pl, uint8_t* scr, const BigInt& P, const std::vector<BigInt>& pw,
                    int nbits, int dbits, int nthreads, hipStream_t st, SolutionData* out, GpuReconTimes* tm,
                    KernelTimer* kt) {
    if ((int)pw.size() != pl.m + 1) return ES_EINTERNAL;
    const BigInt& M = pw[pl.m];
    typedef std::chrono::steady_clock clk;
    auto t0 = clk::now();
    auto lap = [&](double* slot, const char* what) {
        auto t1 = clk::now();
        const double ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
        if (slot) *slot = ms;
        if (verbose()) fprintf(stderr, "[es] gpu reconstruct %-12s %8.3f ms\n", what, ms);
        t0 = t1;
    };
    // parts of a stage, printed only (the stage's lap keeps its total)
    auto ts = clk::now();
    auto sublap = [&](const char* what) {
        const auto t1 = clk::now();
        if (verbose())
            fprintf(stderr, "[es] gpu reconstruct   %-10s %8.3f ms\n", what,
                    std::chrono::duration<double, std::milli>(t1 - ts).count());
        ts = t1;
    };
    const int m = pl.m, NW = pl.NW, TM = pl.TM, nw = pl.nw;
    const size_t NC = pl.NC;
    const uint64_t* dig = (const uint64_t*)(scr + pl.off_digits);
    const size_t dig_comp = (size_t)m * kDigitLimbs;  // int64 per component

    // 1. common denominator from the sample (host)
    const std::vector<size_t> sidx = sample_indices(NC, pl.c);
    const size_t y_bytes = round_up(NC * nw * sizeof(uint32_t), 256), st_bytes = round_up(NC * sizeof(int), 256);
    const size_t g_bytes = round_up(NC * sizeof(uint64_t), 256);
    const size_t sd_bytes = sidx.size() * dig_comp * sizeof(int64_t);
    // the copy stream is idle whenever this returns (every exit waits for
    // it), so the pinned stage and the caller's workspace are free to reuse
    hipStream_t cst = g_copy_stream.get();
    if (!cst) return ES_EHIP;
    struct SyncOnExit {
        hipStream_t s;
        ~SyncOnExit() { (void)hipStreamSynchronize(s); }
    } sync_copies{cst};
    uint8_t* pin = (uint8_t*)g_pinned_stage.get(y_bytes + 2 * st_bytes + g_bytes + sd_bytes);
    if (!pin) return ES_ENOMEM;
    uint32_t* Yh = (uint32_t*)pin;
    int* sth = (int*)(pin + y_bytes);
    int* gsth = (int*)(pin + y_bytes + st_bytes);
    uint64_t* Gh = (uint64_t*)(pin + y_bytes + 2 * st_bytes);
    int64_t* sd = (int64_t*)(pin + y_bytes + 2 * st_bytes + g_bytes);
    for (size_t k = 0; k < sidx.size(); k++)
        HIPOK(hipMemcpyAsync(sd + k * dig_comp, dig + sidx[k] * dig_comp, dig_comp * sizeof(int64_t),
                             hipMemcpyDeviceToHost, st));
    HIPOK(hipStreamSynchronize(st));
    sublap("digits");
    // The sample's denominators (Wang reconstruction of each X mod M; their
    // lcm is d).  With one right-hand side the first two run first, with a
    // second thread each for the cofactors, and the GPU pass starts from
    // their lcm; the others finish on threads of their own meanwhile, and if
    // the whole sample's lcm differs the pass is run again with it before any
    // of its results are used.  With several right-hand sides (whose
    // denominators differ, so a part of the sample misses factors far more
    // often) the whole sample runs first.  The first ones' X are assembled
    // each in parts on the pool's threads, the others' on their own threads.
    const size_t nfirst = pl.c == 1 ? std::min<size_t>(2, sidx.size()) : sidx.size();
    std::vector<BigInt> xs(sidx.size());
    {
        int parts = 1;
        while (parts < 8 && (size_t)parts * 2 * nfirst <= (size_t)nthreads) parts *= 2;
        assemble_split(sd, dig_comp, nfirst, m, pw, parts, nthreads, xs.data());
    }
    sublap("assemble");
    const BigInt Nb = shl(BigInt::from_u64(1), (size_t)nbits);
    const BigInt Db = shl(BigInt::from_u64(1), (size_t)dbits);
    std::vector<BigInt> sden(xs.size());
    std::atomic<int> bad{0};
    auto sample_rr = [&](size_t k, bool split) {
        try {
            BigInt a = mod_floor(k < nfirst ? xs[k] : assemble(sd + k * dig_comp, m, pw), M), nu, de;
            if (!rational_reconstruct(a, M, Nb, Db, &nu, &de, false, split)) bad = 1;
            else sden[k] = de;
        } catch (...) {
            bad = 1;
        }
    };
    const bool split_first = 4 * nfirst <= (size_t)nthreads;
    std::vector<std::thread> rest;
    struct Joiner {
        std::vector<std::thread>& v;
        void join() {
            for (auto& t : v)
                if (t.joinable()) t.join();
        }
        ~Joiner() { join(); }
    } rest_join{rest};
    auto start_rest = [&]() {
        for (size_t k = nfirst; k < xs.size(); k++) rest.emplace_back(sample_rr, k, false);
    };
    // the others start at once when they and the first ones fit the cores
    const bool rest_now = nfirst * (split_first ? 2 : 1) + (xs.size() - nfirst) <= (size_t)nthreads;
    if (rest_now) start_rest();
    if (nfirst <= 2) {
        std::thread second;
        if (nfirst > 1) second = std::thread(sample_rr, (size_t)1, split_first);
        sample_rr(0, split_first);
        if (second.joinable()) second.join();
    } else {
        parallel_for_each(nfirst, nthreads, [&](size_t k) { sample_rr(k, split_first); });
    }
    sublap("wang");
    if (!rest_now) start_rest();
    if (bad) return ES_EINTERNAL;
    // dbase: the lcm of the denominators known so far; d, the pass's
    // common denominator, is a multiple of it
    BigInt dbase = sden[0];
    for (size_t k = 1; k < nfirst; k++) dbase = lcm(dbase, sden[k]);
    BigInt d = dbase;
    bool sample_checked = rest.empty();
    // d also takes the small factors a sample most often misses: a
    // component's y = d x in the bound is exact whatever multiple of its
    // denominator d is, as long as d stays within the denominator bound
    // (both are below the bounds that M separates), and the gcd takes the
    // extra factors out again.  When the pass starts from part of the
    // sample, 2^6, and 3^2, 5^2 and 7 when they are not among the lift's
    // primes (so that they may divide det A): a pass whose d the whole
    // sample's denominators divide is kept.  Otherwise (the whole sample
    // comes first) 2^2: on random systems with sixteen right-hand sides the
    // sample's lcm lacked a factor 2 of other components' denominators in
    // about one system in twenty, and 2^2 keeps the one-word gcds
    // d / (denominator) well inside 64 bits.
    const BigInt Dcap = shl(BigInt::from_u64(1), (size_t)dbits);
    {
        uint64_t s = 4;
        if (!sample_checked) {
            s = 64;
            const uint64_t qs[3] = {3, 5, 7}, pe[3] = {9, 25, 7};
            for (int i = 0; i < 3; i++)
                if (!mod_floor(P, BigInt::from_u64(qs[i])).is_zero()) s *= pe[i];
        }
        const BigInt ds = mul_small(dbase, (int64_t)s);
        if (cmp(ds, Dcap) <= 0) d = ds;
    }
    lap(tm ? &tm->sample_ms : nullptr, "sample");

    uint32_t* Td = (uint32_t*)(scr + pl.off_T);
    uint32_t* Mwd = (uint32_t*)(scr + pl.off_Mw);
    uint8_t* W = scr + pl.off_W;
    int8_t* WT = (int8_t*)(scr + pl.off_WT);
    int8_t* S = (int8_t*)(scr + pl.off_S);
    int* rowsum = (int*)(scr + pl.off_rowsum);
    int* VT = (int*)(scr + pl.off_VT);
    uint32_t* Yd = (uint32_t*)(scr + pl.off_Y);
    int* std_ = (int*)(scr + pl.off_status);
    uint32_t* Dwd = (uint32_t*)(scr + pl.off_Dw);
    uint64_t* Gd = (uint64_t*)(scr + pl.off_G);
    int* gstd = (int*)(scr + pl.off_gstat);
    std::vector<uint32_t> T((size_t)m * NW), Mw(NW), Dwords(NW);
    to_words(M, Mw.data(), NW);
    HIPOK(hipMemcpyAsync(Mwd, Mw.data(), Mw.size() * sizeof(uint32_t), hipMemcpyHostToDevice, st));
    const double Md = (double)Mw[TM] + (double)Mw[TM - 1] * 0x1p-32 + (double)Mw[TM - 2] * 0x1p-64;
    const double Mtop = (double)Mw[TM] * 0x1p64 + (double)Mw[TM - 1] * 0x1p32 + (double)Mw[TM - 2];

    // One pass of the numerators for every component under the current d:
    // weight seeds T_i = P^i d mod M (host), weight rows, GEMM, numerators
    // and gcds (GPU), results to the pinned arrays.
    bool gpu_gcd = false;
    size_t gcd_first = NC;  // components of the first gcd launch
    hipEvent_t words_ready = g_words_ready.get(), first_gcds = g_first_gcds.get();
    hipEvent_t numer_done = g_numer_done.get();
    if (!words_ready || !first_gcds || !numer_done || !cst) return ES_EHIP;
    auto gpu_pass = [&]() -> int {
        // The chain T_{i+1} = T_i P mod M, cut into segments that each start
        // from P^{i0} d mod M = (d mod P^{m - i0}) P^{i0} (M = P^m: the
        // product is below M, no division by M) and run in parallel.  With
        // T_i = P^i D_i, D_i = d mod P^{m - i}, the step's quotient
        // floor(P T_i / M) is D_i's base-P digit m - i - 1, so each step is
        // T_{i+1} = P T_i - delta M with no division: a segment takes its
        // digits from one division of D_{i0} by a power of P.
        const int nseg = std::max(1, std::min(nthreads, m / 8));
        parallel_for_each((size_t)nseg, nthreads, [&](size_t sg) {
            const int i0 = (int)(sg * (size_t)m / nseg), i1 = (int)((sg + 1) * (size_t)m / nseg);
            const BigInt D = mod_floor(d, pw[m - i0]);
            // digits m - i1 + 1 .. m - i0 - 1 of D, lowest first
            std::vector<BigInt> delta;
            if (i1 - i0 >= 2) {
                BigInt Q = shr_pow(D, pw[m - i1 + 1]);
                for (int k = 0; k < i1 - i0 - 1; k++) {
                    BigInt qq, r;
                    divmod_trunc(Q, P, &qq, &r);
                    delta.push_back(std::move(r));
                    Q = std::move(qq);
                }
                if (!Q.is_zero()) throw std::logic_error("seed digits left over");
            }
            BigInt Ti = mul(D, pw[i0]);
            Ti.d.resize(M.size(), 0);
            for (int i = i0; i < i1; i++) {
                to_words(Ti, &T[(size_t)i * NW], NW);
                if (i + 1 < i1) {
                    const BigInt& q = delta[(size_t)(i1 - 2 - i)];
                    seed_step(Ti.d.data(), M.size(), P.d.data(), P.size(), q.d.data(), q.size(), M.d.data());
                }
            }
        });
        lap(tm ? &tm->seeds_ms : nullptr, "seeds");
        const int nwd = (int)((d.bit_length() + 31) / 32);
        gpu_gcd = nwd <= NW && gcd_words_per_lane(std::max(nw, nwd)) != 0;
        to_words(d, Dwords.data(), NW);
        HIPOK(hipMemcpyAsync(Td, T.data(), T.size() * sizeof(uint32_t), hipMemcpyHostToDevice, st));
        HIPOK(hipMemcpyAsync(Dwd, Dwords.data(), Dwords.size() * sizeof(uint32_t), hipMemcpyHostToDevice, st));
        long ev = kt->start(KC_RECON_OTHER);
        HIPOK(launch_wchain(Td, Mwd, m, TM, Md, pl.Ncolsp, W, st));
        HIPOK(launch_transpose_offset(W, pl.Kpad, pl.Ncolsp, WT, st));
        kt->stop(ev);
        for (size_t j0 = 0; j0 < NC; j0 += (size_t)pl.NCc) {
            const int rows = (int)std::min<size_t>((size_t)pl.NCc, NC - j0);
            ev = kt->start(KC_RECON_OTHER);
            HIPOK(launch_digit_bytes(dig, m, m, (int)j0, rows, pl.NCcp, pl.Kpad, S, rowsum, st));
            kt->stop(ev);
            ev = kt->start_one(KC_RECON_GEMM);
            HIPOK(launch_recon_gemm(S, WT, pl.Kpad, pl.NCcp, pl.Ncolsp, VT, st));
            kt->stop(ev);
            ev = kt->start(KC_RECON_OTHER);
            HIPOK(launch_numer(VT, pl.Ncolsp, rowsum, rows, Mwd, TM, Mtop, nbits, Yd + j0 * nw, std_ + j0, st));
            kt->stop(ev);
            // the numerator words leave on the copy stream while the gcds
            // run, and the host converts them meanwhile
            HIPOK(hipEventRecord(numer_done, st));
            HIPOK(hipStreamWaitEvent(cst, numer_done, 0));
            HIPOK(hipMemcpyAsync(Yh + j0 * nw, Yd + j0 * nw, (size_t)rows * nw * sizeof(uint32_t),
                                 hipMemcpyDeviceToHost, cst));
            HIPOK(hipMemcpyAsync(sth + j0, std_ + j0, (size_t)rows * sizeof(int), hipMemcpyDeviceToHost, cst));
        }
        HIPOK(hipEventRecord(words_ready, cst));
        gcd_first = NC;
        if (gpu_gcd) {
            // over every component at once (the blocks fill the CUs in fewer
            // rounds than chunk by chunk), as two launches when the blocks
            // take many rounds: the host brings the first launch's
            // components to lowest terms while the second runs
            int grp = 0;
            gcd_first = (size_t)gcd_split((int)NC, nw, nwd, &grp);
            if (gcd_first > NC) gcd_first = NC;
            const size_t bounds[3] = {0, gcd_first, NC};
            for (int part = 0; part < 2; part++) {
                const size_t j0 = bounds[part], rows = bounds[part + 1] - j0;
                if (rows == 0) continue;
                long ev = kt->start_one(KC_RECON_GCD);
                HIPOK(launch_gcd(Yd + j0 * nw, nw, std_ + j0, (int)rows, Dwd, nwd, Gd + j0, gstd + j0, grp, st));
                kt->stop(ev);
                HIPOK(hipMemcpyAsync(Gh + j0, Gd + j0, rows * sizeof(uint64_t), hipMemcpyDeviceToHost, st));
                HIPOK(hipMemcpyAsync(gsth + j0, gstd + j0, rows * sizeof(int), hipMemcpyDeviceToHost, st));
                if (part == 0) HIPOK(hipEventRecord(first_gcds, st));
            }
        }
        return ES_OK;
    };

    // The components of `which` that the last pass accepted: first y / d
    // from the numerator words (while the gcds run), then lowest terms
    // where the gcd is not 1.
    std::atomic<size_t> host_gcds{0};
    auto convert = [&](const std::vector<size_t>& which) {
        const uint32_t di = (uint32_t)out->dens.size();  // this pass's d
        out->dens.push_back(d);
        parallel_for_each(which.size(), nthreads, [&](size_t k) {
            const size_t j = which[k];
            if (sth[j] != 0 && sth[j] != 1) return;
            out->num[j] = from_words(Yh + j * nw, nw, sth[j] == 1);
            out->den_of[j] = di;
        });
    };
    auto reduce = [&](const std::vector<size_t>& which) {
        // the components whose gcd the host computes (long) are listed
        // first, one item each, so that the pool's threads share them; the
        // one-word divisions follow in batches
        std::vector<size_t> need;
        std::vector<uint64_t> gs;  // the distinct one-word gcds other than 1
        for (size_t j : which)
            if ((sth[j] == 0 || sth[j] == 1) && gsth[j] != 0) need.push_back(j);
        const size_t nlong = need.size();
        for (size_t j : which) {
            if ((sth[j] != 0 && sth[j] != 1) || gsth[j] != 0 || Gh[j] == 1) continue;
            need.push_back(j);
            gs.push_back(Gh[j]);
        }
        std::sort(gs.begin(), gs.end());
        gs.erase(std::unique(gs.begin(), gs.end()), gs.end());
        // d / g for each of them (a few: on this thread), as new entries of
        // the denominator table
        const size_t base = out->dens.size();
        out->dens.resize(base + gs.size());
        parallel_for_each(gs.size(), gs.size() <= 8 ? 1 : nthreads,
                          [&](size_t k) { out->dens[base + k] = divexact_u64(d, gs[k]); });
        std::vector<BigInt> own(nlong);  // denominators of the host gcds
        const size_t kBatch = 32, nbatch = (need.size() - nlong + kBatch - 1) / kBatch;
        parallel_for_each(nlong + nbatch, nthreads, [&](size_t it) {
            if (it >= nlong) {
                const size_t k0 = nlong + (it - nlong) * kBatch, k1 = std::min(need.size(), k0 + kBatch);
                for (size_t k = k0; k < k1; k++) {
                    const size_t j = need[k];
                    divexact_u64_inplace(out->num[j], Gh[j]);
                    out->den_of[j] =
                        (uint32_t)(base + (size_t)(std::lower_bound(gs.begin(), gs.end(), Gh[j]) - gs.begin()));
                }
                return;
            }
            const size_t j = need[it];
            const BigInt g = gcd(out->num[j], d);
            host_gcds++;
            if (g.size() == 1 && g.d[0] == 1) return;
            out->num[j] = divexact(out->num[j], g);
            own[it] = divexact(d, g);
        }, 1);
        for (size_t k = 0; k < nlong; k++) {
            if (own[k].is_zero()) continue;
            out->den_of[need[k]] = (uint32_t)out->dens.size();
            out->dens.push_back(std::move(own[k]));
        }
    };

    out->n = pl.n;
    out->c = pl.c;
    out->num.assign(NC, BigInt());
    out->dens.clear();
    out->den_of.assign(NC, 0);
    std::vector<size_t> todo(NC);
    for (size_t j = 0; j < NC; j++) todo[j] = j;
    // Digits of the listed components, copied to the host on the solve's stream.
    auto fetch = [&](const std::vector<size_t>& which, std::vector<int64_t>* buf) -> int {
        buf->resize(which.size() * dig_comp);
        for (size_t k = 0; k < which.size(); k++)
            HIPOK(hipMemcpyAsync(buf->data() + k * dig_comp, dig + which[k] * dig_comp, dig_comp * sizeof(int64_t),
                                 hipMemcpyDeviceToHost, st));
        HIPOK(hipStreamSynchronize(st));
        return ES_OK;
    };
    // Reconstructs one component on its own from its digits (card, "Method": a
    // numerator outside the bound means the sample missed part of its
    // denominator).
    auto alone = [&](const int64_t* digs, BigInt* nu, BigInt* de, bool split) -> bool {
        BigInt a = mod_floor(assemble(digs, m, pw), M);
        return rational_reconstruct(a, M, Nb, Db, nu, de, true, split);
    };
    size_t failed_total = 0;
    for (int pass = 0;; pass++) {
        int rc = gpu_pass();
        if (rc != ES_OK) return rc;
        if (!sample_checked) {
            rest_join.join();
            sample_checked = true;
            if (bad) return ES_EINTERNAL;
            for (size_t k = nfirst; k < sden.size(); k++) dbase = lcm(dbase, sden[k]);
            const BigInt dall = lcm(d, dbase);
            if (cmp(dall, d) != 0) {
                // d missed part of the sample's denominators: this pass is
                // dropped and run again with their lcm (with d's extra
                // factors while that stays within the bound)
                if (verbose()) {
                    const BigInt f = divexact(dall, d);
                    fprintf(stderr, "[es] gpu reconstruct: the sample widened d by a %zu-bit factor (%llu if one word), pass again\n",
                            f.bit_length(), f.size() == 1 ? (unsigned long long)f.d[0] : 0ULL);
                }
                HIPOK(hipStreamSynchronize(st));
                d = cmp(dall, Dcap) <= 0 ? dall : dbase;
                pass--;
                continue;
            }
        }
        HIPOK(hipEventSynchronize(words_ready));
        convert(todo);
        std::vector<size_t> later;  // components of the second gcd launch
        if (gpu_gcd && gcd_first < NC) {
            std::vector<size_t> early;
            for (size_t j : todo) (j < gcd_first ? early : later).push_back(j);
            HIPOK(hipEventSynchronize(first_gcds));
            reduce(early);
        } else {
            later = todo;
        }
        HIPOK(hipStreamSynchronize(st));
        if (!gpu_gcd)
            for (size_t j = 0; j < NC; j++) gsth[j] = 1;
        lap(tm ? &tm->gpu_ms : nullptr, "gpu");
        reduce(later);
        std::vector<size_t> failed;
        for (size_t j : todo)
            if (sth[j] != 0 && sth[j] != 1) failed.push_back(j);
        lap(tm ? &tm->finish_ms : nullptr, "lowest terms");
        if (failed.empty()) break;
        failed_total += failed.size();
        if (verbose()) fprintf(stderr, "[es] gpu reconstruct: %zu components outside the bound\n", failed.size());
        std::vector<int64_t> digs;
        if (failed.size() <= (size_t)(2 * nthreads) || pass >= 3) {
            // few left: each on its own, in parallel
            rc = fetch(failed, &digs);
            if (rc != ES_OK) return rc;
            std::atomic<int> bad{0};
            std::vector<BigInt> own(failed.size());
            parallel_for_each(failed.size(), nthreads, [&](size_t k) {
                BigInt nu;
                if (!alone(digs.data() + k * dig_comp, &nu, &own[k], 4 * failed.size() <= (size_t)nthreads)) bad = 1;
                out->num[failed[k]] = nu;
            });
            if (bad) return ES_EINTERNAL;
            for (size_t k = 0; k < failed.size(); k++) {
                out->den_of[failed[k]] = (uint32_t)out->dens.size();
                out->dens.push_back(std::move(own[k]));
            }
            break;
        }
        // many left: d becomes the lcm of the known denominators and the
        // first one's (any extra factors dropped: they may have pushed the
        // numerators past the bound), and they run again
        rc = fetch(std::vector<size_t>{failed[0]}, &digs);
        if (rc != ES_OK) return rc;
        BigInt nu, de;
        if (!alone(digs.data(), &nu, &de, true)) return ES_EINTERNAL;
        dbase = lcm(dbase, de);
        d = dbase;
        todo.swap(failed);
    }
    if (verbose())
        fprintf(stderr, "[es] gpu reconstruct: %zu gcds finished on the host, %zu components alone\n",
                (size_t)host_gcds, failed_total);
    if (tm) {
        tm->failed = failed_total;
        tm->host_gcds = host_gcds;
    }
    return ES_OK;
}

}  // namespace es
