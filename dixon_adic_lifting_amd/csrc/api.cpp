// C ABI of the exact solver (include/es_solve.h): argument checks, the order
// of the stages on one HIP stream, and the solution object.
//
// Stages (exact-solve card, phanerozoic/exact-solve, section "Method"):
//   checks + bounds -> residues of A -> batched Gauss-Jordan inverse (one
//   launch per elimination step, all 53 primes) -> prime-set selection and
//   step count -> m lift steps (contraction, CRT, residual) -> one
//   device-to-host copy of the digits per chunk of steps -> host rational
//   reconstruction.
#include <hip/hip_runtime.h>

#include <chrono>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <new>
#include <future>
#include <vector>

#include "../../include/es_solve.h"
#include "es_internal.h"
#include "host.h"
#include "recon_host.h"

using namespace es;

struct es_solution {
    SolutionData data;
};

namespace {

thread_local double g_timings[5] = {0, 0, 0, 0, 0};

typedef std::chrono::steady_clock clk;
double ms_since(clk::time_point t0) {
    return std::chrono::duration<double, std::milli>(clk::now() - t0).count();
}

#define HIP_CHECK(expr)                          \
    do {                                         \
        if ((expr) != hipSuccess) return ES_EHIP; \
    } while (0)

// Opt-in per-launch timing: a pair of HIP events on the solve's stream around
// every launch of the hot kernels; totals are read after the final sync.
// Classes 5, 6 and 7 (reconstruction GEMM, other reconstruction kernels,
// gcds) are declared with the reconstruction driver; 8 and 9 are the panel
// and update launches of the blocked elimination.
enum KernelClass {
    KC_GJ = 0, KC_CONTRACT = 1, KC_CRT = 2, KC_RESIDUAL = 3, KC_RESIDUES = 4,
    KC_PANEL = 8, KC_UPDATE = 9, KC_COUNT = 10
};

thread_local bool g_profiling = false;
// components the last GPU reconstruction on this thread finished on the host
// (outside the numerator bound: reconstructed alone; or gcds left to the host)
thread_local int64_t g_recon_alone = -1, g_recon_host_gcds = -1;
thread_local double g_kernel_ms[KC_COUNT] = {};
thread_local int32_t g_kernel_cnt[KC_COUNT] = {};

struct Profiler : KernelTimer {
    bool on = false;
    hipStream_t st = nullptr;
    std::vector<hipEvent_t> pool;
    size_t used = 0;
    std::vector<std::pair<int, size_t>> marks;  // (class, index of the start event)

    explicit Profiler(hipStream_t s) : on(g_profiling), st(s) {}
    ~Profiler() {
        for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    }
    hipEvent_t next() {
        if (used == pool.size()) {
            hipEvent_t e = nullptr;
            if (hipEventCreate(&e) != hipSuccess) return nullptr;
            pool.push_back(e);
        }
        return pool[used++];
    }
    // returns the index of the start event (or -1 when off)
    long start(int cls) override {
        if (!on) return -1;
        hipEvent_t e = next();
        if (!e) return -1;
        (void)hipEventRecord(e, st);
        marks.push_back({cls, used - 1});
        return (long)(used - 1);
    }
    // one kernel: the next launch records the pair itself; stop() records nothing
    long start_one(int cls) override {
        if (!on) return -1;
        hipEvent_t e0 = next();
        hipEvent_t e1 = e0 ? next() : nullptr;
        if (!e1) return -1;
        pending_launch_events() = LaunchEvents{e0, e1};
        marks.push_back({cls, used - 2});
        return -1;
    }
    void stop(long idx) override {
        pending_launch_events() = LaunchEvents{};  // unused if the launch did not happen
        if (idx < 0) return;
        hipEvent_t e = next();
        if (e) (void)hipEventRecord(e, st);
    }
    // after the stream has been synchronised
    void collect() {
        if (!on) return;
        for (int k = 0; k < KC_COUNT; k++) {
            g_kernel_ms[k] = 0;
            g_kernel_cnt[k] = 0;
        }
        for (auto& mk : marks) {
            if (mk.second + 1 >= used) continue;
            float ms = 0;
            if (hipEventElapsedTime(&ms, pool[mk.second], pool[mk.second + 1]) == hipSuccess) {
                g_kernel_ms[mk.first] += ms;
                g_kernel_cnt[mk.first] += 1;
            }
        }
    }
};

// Two 62-bit primes for the rank test that separates "singular" from "det A
// is a nonzero multiple of every odd prime below 256".
const uint64_t kRankPrimes[2] = {4611686018427387847ULL, 4611686018427387817ULL};  // 2^62-57, 2^62-87

bool valid_shape(int32_t n, int32_t c) { return n >= 1 && n <= ES_MAX_N && c >= 1 && (int64_t)n * c <= (1LL << 31); }

struct Prep {
    Layout L;
    uint64_t maxabs = 0;
    int nbits = 0, dbits = 0;
    bool a32 = false;
};

// Pinned host memory, kept per thread and grown on demand
// (device-to-host copies into pageable memory go through an extra staging
// copy, and pinned memory is allocated with hipHostMalloc, never registered).
struct PinnedBuffer {
    void* p = nullptr;
    size_t bytes = 0;
    ~PinnedBuffer() {
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
thread_local PinnedBuffer g_pinned;  // the digits
thread_local PinnedBuffer g_stats;   // the range statistics of A and b

// Initialise the workspace and enqueue the norms and their copy to the host;
// the elimination can be enqueued behind them before the host reads them.
int prepare_launch(const int64_t* dA, const int64_t* db, int32_t n, int32_t c, uint8_t* ws, hipStream_t st,
                   Prep* pr) {
    Layout& L = pr->L;
    HIP_CHECK(launch_fill_u32((uint32_t*)(ws + L.off_piv), (size_t)kNumPrimes * (n + 1), (uint32_t)INT_MAX, st));
    HIP_CHECK(launch_fill_u32((uint32_t*)(ws + L.off_rowpos), (size_t)kNumPrimes * n, 0xffffffffu, st));
    HIP_CHECK(launch_fill_u32((uint32_t*)(ws + L.off_flags), kNumPrimes, 0u, st));
    HIP_CHECK(launch_fill_u32((uint32_t*)(ws + L.off_rho), (size_t)kNumPrimes * c * L.pitch / 4, 0u, st));
    HIP_CHECK(launch_stats(dA, db, L, ws, st));
    uint8_t* h = (uint8_t*)g_stats.get(((size_t)3 * n + c) * 8);
    if (!h) return ES_ENOMEM;
    HIP_CHECK(hipMemcpyAsync(h, ws + L.off_rowmax, n * sizeof(uint64_t), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(h + (size_t)8 * n, ws + L.off_rownorm, n * sizeof(double), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(h + (size_t)16 * n, ws + L.off_colnorm, n * sizeof(double), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(h + (size_t)24 * n, ws + L.off_bnorm, c * sizeof(double), hipMemcpyDeviceToHost, st));
    return ES_OK;
}

// After the stream has passed prepare_launch's copies: check the range and
// bound the solution's size.
int prepare_finish(int32_t n, int32_t c, Prep* pr) {
    const uint8_t* h = (const uint8_t*)g_stats.p;
    const uint64_t* rowmax = (const uint64_t*)h;
    const double* rn = (const double*)(h + (size_t)8 * n);
    const double* cn = (const double*)(h + (size_t)16 * n);
    const double* bn = (const double*)(h + (size_t)24 * n);
    uint64_t mx = 0;
    for (int i = 0; i < n; i++) mx = rowmax[i] > mx ? rowmax[i] : mx;
    pr->maxabs = mx;
    if ((unsigned __int128)mx * (unsigned)n >= ((unsigned __int128)1 << 63)) return ES_ERANGE;
    for (int i = 0; i < n; i++)
        if (rn[i] == 0.0 || cn[i] == 0.0) return ES_SINGULAR;  // a zero row or column
    hadamard_bits(rn, cn, bn, n, c, &pr->nbits, &pr->dbits);
    pr->a32 = mx < (1ULL << 31);
    return ES_OK;
}

// Blocked elimination (default) or one launch per elimination step, per thread.
thread_local int g_blocked = -1;  // -1: not set on this thread (environment decides)

bool use_blocked(const Layout& L) {
    static const bool env_step = [] {
        const char* e = std::getenv("ES_INVERSE");
        return e && std::strcmp(e, "stepwise") == 0;
    }();
    const bool want = g_blocked < 0 ? !env_step : g_blocked == 1;
    return want && blocked_inverse_fits(L);
}

// The blocked inverse overlaps each panel with the previous panel's update
// unless ES_LOOKAHEAD=0.
bool use_lookahead() {
    static const bool v = [] {
        const char* e = std::getenv("ES_LOOKAHEAD");
        return !(e && e[0] == '0');
    }();
    return v;
}

// Residues and the Gauss-Jordan elimination; flags to the host.
int run_inverse(const int64_t* dA, uint8_t* ws, hipStream_t st, Prep* pr, int* flags, Profiler* prof) {
    const Layout& L = pr->L;
    const bool blocked = use_blocked(L);
    long ev = prof->start(KC_RESIDUES);
    HIP_CHECK(launch_residues(dA, L, ws, st, blocked));
    prof->stop(ev);
    if (blocked && !prof->on && use_lookahead()) {
        // panel K runs together with the update of panel K - 32 (the columns
        // the next panel needs are updated first, in the gather launch)
        for (int K = 0; K < L.n + kPanel; K += kPanel) {
            HIP_CHECK(launch_gj_panel_rest(L, ws, K, st));
            if (K < L.n) HIP_CHECK(launch_gj_gather_next(L, ws, K, st));
        }
    } else if (blocked) {
        // one kernel at a time (also the form that per-kernel timing measures)
        for (int K = 0; K < L.n; K += kPanel) {
            ev = prof->start_one(KC_PANEL);
            HIP_CHECK(launch_gj_panel(L, ws, K, st));
            prof->stop(ev);
            ev = prof->start_one(KC_UPDATE);
            HIP_CHECK(launch_gj_update(L, ws, K, st));
            prof->stop(ev);
        }
    } else {
        for (int k = 0; k < L.n; k++) {
            ev = prof->start(KC_GJ);
            HIP_CHECK(launch_gj_step(L, ws, k, st));
            prof->stop(ev);
        }
    }
    HIP_CHECK(hipMemcpyAsync(flags, ws + L.off_flags, kNumPrimes * sizeof(int), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipStreamSynchronize(st));
    return ES_OK;
}

// No prime survived: every q_j divides det A.  Decide singular vs ENOPRIME.
int no_prime_decision(const int64_t* dA, int32_t n, const Prep& pr, hipStream_t st) {
    // |det A| <= 2^dbits; if that is below the product of all 53 primes, the
    // only multiple of it within the bound is 0.
    BigInt all = BigInt::from_u64(1);
    for (int j = 0; j < kNumPrimes; j++) all = mul_small(all, kPrimeTable.q[j]);
    if ((size_t)pr.dbits + 1 < all.bit_length()) return ES_SINGULAR;
    std::vector<int64_t> A((size_t)n * n);
    HIP_CHECK(hipMemcpyAsync(A.data(), dA, A.size() * sizeof(int64_t), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipStreamSynchronize(st));
    for (uint64_t p : kRankPrimes)
        if (full_rank_mod(A.data(), n, p)) return ES_ENOPRIME;  // det != 0 for certain
    return ES_SINGULAR;  // singular modulo two 62-bit primes as well
}


// Lift m steps; digits land in host [n*c][m][6].
// With dig_dev set, the digits stay on the device ([n*c][m][6] at dig_dev)
// and digits_host is unused.
int run_lift(const int64_t* dA, const int64_t* db, uint8_t* ws, hipStream_t st, const Prep& pr,
             const LiveSet& ls, int m, int64_t* digits_host, Profiler* prof, uint64_t* dig_dev = nullptr) {
    Layout L = pr.L;
    L.krec = lift_record_steps(L);
    if (m <= L.kchunk || dig_dev) L.kchunk = m;  // one chunk: the device digits are laid out exactly as the host's
    L.dig_dev = dig_dev;
    LiftParams prm;
    fill_lift_params(ls, &prm);
    HIP_CHECK(hipMemcpyAsync(ws + L.off_params, &prm, sizeof prm, hipMemcpyHostToDevice, st));
    HIP_CHECK(launch_lift_positions(L, ws, st));
    // several right-hand sides with |A| < 2^30: the residual on MFMA, and
    // B_j's columns and the residues in natural row order
    const bool rmfma = residual_mfma_fits(L, pr.a32, pr.maxabs);
    if (rmfma) {
        HIP_CHECK(launch_a_planes(L, ws, st));
        HIP_CHECK(launch_natural_cols(L, ws, ls.E, st));
    }
    HIP_CHECK(launch_split_b(db, L, ws, ls.E, rmfma, st));
    const bool fused = lift_fused_fits(L);
    if (fused) HIP_CHECK(launch_lift_rows(L, ws, ls.E, st));
    const size_t NC = (size_t)L.n * L.c;
    for (int i0 = 0; i0 < m; i0 += L.kchunk) {
        const int cnt = std::min(L.kchunk, m - i0);
        for (int s = 0; s < cnt; s++) {
            long ev;
            if (fused) {
                ev = prof->start_one(KC_CONTRACT);
                HIP_CHECK(launch_lift_contract_crt(L, ws, ls.E, s % L.krec, st));
                prof->stop(ev);
            } else {
                ev = prof->start_one(KC_CONTRACT);
                HIP_CHECK(launch_lift_contract(L, ws, ls.E, st));
                prof->stop(ev);
                ev = prof->start_one(KC_CRT);
                HIP_CHECK(launch_lift_crt(L, ws, s, rmfma, st));
                prof->stop(ev);
            }
            ev = prof->start_one(KC_RESIDUAL);
            HIP_CHECK(launch_lift_residual(L, ws, pr.a32, dA, rmfma, st));
            prof->stop(ev);
            if (fused && (s % L.krec == L.krec - 1 || s == cnt - 1)) {
                // the digits of the steps whose records are held
                ev = prof->start_one(KC_CRT);
                HIP_CHECK(launch_lift_crt_records(L, ws, s % L.krec + 1, s - s % L.krec, st));
                prof->stop(ev);
            }
        }
        if (dig_dev) {
            // digits stay on the device for the GPU reconstruction
        } else if (cnt == m) {
            HIP_CHECK(hipMemcpyAsync(digits_host, ws + L.off_digits, NC * (size_t)m * kDigitLimbs * 8,
                                     hipMemcpyDeviceToHost, st));
        } else {
            HIP_CHECK(hipMemcpy2DAsync(digits_host + (size_t)i0 * kDigitLimbs, (size_t)m * kDigitLimbs * 8,
                                       ws + L.off_digits, (size_t)L.kchunk * kDigitLimbs * 8,
                                       (size_t)cnt * kDigitLimbs * 8, NC, hipMemcpyDeviceToHost, st));
        }
    }
    HIP_CHECK(hipStreamSynchronize(st));
    return ES_OK;
}

}  // namespace

extern "C" {

const char* es_strerror(int status) {
    switch (status) {
        case ES_OK: return "ok";
        case ES_SINGULAR: return "A is singular over the rationals";
        case ES_EINVAL: return "invalid argument (size, null pointer or workspace too small)";
        case ES_ERANGE: return "n * max|A_ij| >= 2^63";
        case ES_ENOPRIME: return "det A is a nonzero multiple of every odd prime below 256";
        case ES_EHIP: return "HIP runtime error";
        case ES_ENOMEM: return "out of memory";
        case ES_EINTERNAL: return "internal consistency check failed";
        case ES_ETOOBIG: return "n exceeds what the fixed scratch of the non-allocating entry point holds";
        default: return "unknown status";
    }
}

int es_primes(int32_t* q, int32_t cap) {
    for (int j = 0; j < kNumPrimes && j < cap; j++) q[j] = (int32_t)kPrimeTable.q[j];
    return kNumPrimes;
}

size_t es_workspace_bytes(int32_t n, int32_t c) {
    if (!valid_shape(n, c)) return 0;
    try {
        return make_layout(n, c).total + gpu_recon_reserve(n, c);
    } catch (...) {
        return 0;
    }
}

int es_set_lift_record_steps(int32_t steps) {
    if (steps < 0) return ES_EINVAL;
    set_lift_record_cap(steps);
    return ES_OK;
}

int es_set_blocked_inverse(int on) {
    g_blocked = on ? 1 : 0;
    return ES_OK;
}

int es_set_gpu_reconstruction(int on) {
    set_gpu_recon(on != 0);
    return ES_OK;
}

int es_set_profiling(int on) {
    g_profiling = on != 0;
    return ES_OK;
}

int es_kernel_profile(double* total_ms, int32_t* counts, int32_t cap) {
    if (!total_ms || !counts) return ES_EINVAL;
    for (int k = 0; k < KC_COUNT && k < cap; k++) {
        total_ms[k] = g_kernel_ms[k];
        counts[k] = g_kernel_cnt[k];
    }
    return KC_COUNT;
}

int es_dbg_last_recon_counts(int64_t* alone, int64_t* host_gcds) {
    if (!alone || !host_gcds) return ES_EINVAL;
    *alone = g_recon_alone;
    *host_gcds = g_recon_host_gcds;
    return ES_OK;
}

int es_last_timings(double* ms5) {
    if (!ms5) return ES_EINVAL;
    for (int i = 0; i < 5; i++) ms5[i] = g_timings[i];
    return ES_OK;
}

int es_solve_device(const int64_t* dA, const int64_t* db, int32_t n, int32_t c, void* d_ws, size_t ws_bytes,
                    void* stream, es_solution** out) {
    if (out) *out = nullptr;
    if (!out || !dA || !db || !d_ws || !valid_shape(n, c)) return ES_EINVAL;
    Prep pr;
    pr.L = make_layout(n, c);
    if (ws_bytes < es_workspace_bytes(n, c)) return ES_EINVAL;
    for (double& t : g_timings) t = 0;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    Profiler prof(st);
    try {
        auto t0 = clk::now();
        int rc = prepare_launch(dA, db, n, c, ws, st, &pr);
        g_timings[0] = ms_since(t0);
        if (rc != ES_OK) return rc;
        t0 = clk::now();
        int flags[kNumPrimes];
        rc = run_inverse(dA, ws, st, &pr, flags, &prof);
        g_timings[1] = ms_since(t0);
        if (rc != ES_OK) return rc;
        t0 = clk::now();
        rc = prepare_finish(n, c, &pr);
        g_timings[0] += ms_since(t0);
        if (rc != ES_OK) return rc;
        LiveSet ls = make_live_set(flags);
        if (ls.E == 0) return no_prime_decision(dA, n, pr, st);
        size_t mbits = 0;
        const int m = choose_m_bits(ls.P, pr.nbits, pr.dbits, &mbits);
        // P^0 .. P^m (M = P^m) are needed only by the reconstruction: formed
        // on a host thread while the GPU lifts
        std::future<std::vector<BigInt>> fpw = std::async(std::launch::async, [&ls, m] {
            std::vector<BigInt> pw((size_t)m + 1);
            pw[0] = BigInt::from_u64(1);
            for (int i = 1; i <= m; i++) pw[i] = mul(pw[i - 1], ls.P);
            return pw;
        });
        std::vector<BigInt> pw;
        auto take_M = [&](BigInt* M) {
            pw = fpw.get();
            *M = pw[(size_t)m];
            return M->bit_length() == mbits;
        };
        // the reconstruction's scratch follows the lift's part of the
        // workspace; an input whose plan outgrows the reserve (more than
        // kReserveDrops primes dividing det A near the range limit) takes
        // the host reconstruction
        GpuReconPlan plan;
        uint8_t* scr = nullptr;
        if (!gpu_recon_disabled()) {
            plan = plan_gpu_recon(n, c, m, mbits, pr.nbits);
            if (plan.ok && plan.total <= ws_bytes - pr.L.total) scr = ws + pr.L.total;
        }
        BigInt M;
        es_solution* sol = nullptr;
        if (scr) {
            // lift into device digits, then the GEMM-based reconstruction
            t0 = clk::now();
            rc = run_lift(dA, db, ws, st, pr, ls, m, nullptr, &prof, (uint64_t*)(scr + plan.off_digits));
            g_timings[2] = ms_since(t0);
            if (rc != ES_OK) return rc;
            t0 = clk::now();
            if (!take_M(&M)) return ES_EINTERNAL;
            sol = new es_solution;
            GpuReconTimes rt;
            rc = reconstruct_gpu(plan, scr, ls.P, pw, pr.nbits, pr.dbits, default_threads(), st, &sol->data, &rt,
                                 &prof);
            g_timings[3] = rt.gpu_ms;
            g_timings[4] = ms_since(t0);
            g_recon_alone = (int64_t)rt.failed;
            g_recon_host_gcds = (int64_t)rt.host_gcds;
            prof.collect();
        } else {
            int64_t* digits = (int64_t*)g_pinned.get((size_t)n * c * m * kDigitLimbs * sizeof(int64_t));
            if (!digits) return ES_ENOMEM;
            t0 = clk::now();
            rc = run_lift(dA, db, ws, st, pr, ls, m, digits, &prof);
            g_timings[2] = ms_since(t0);
            if (rc != ES_OK) return rc;
            prof.collect();
            t0 = clk::now();
            if (!take_M(&M)) return ES_EINTERNAL;
            sol = new es_solution;
            rc = reconstruct(digits, (size_t)m, n, c, m, ls.P, M, pr.nbits, pr.dbits, default_threads(),
                             &sol->data);
            g_timings[4] = ms_since(t0);
        }
        if (rc != ES_OK) {
            delete sol;
            return rc;
        }
        sol->data.live = ls.E;
        sol->data.m = m;
        sol->data.nbits = pr.nbits;
        sol->data.dbits = pr.dbits;
        sol->data.mbits = (int)M.bit_length();
        *out = sol;
        return ES_OK;
    } catch (const std::bad_alloc&) {
        return ES_ENOMEM;
    } catch (...) {
        return ES_EINTERNAL;
    }
}

int es_solve(const int64_t* A, const int64_t* b, int32_t n, int32_t c, es_solution** out) {
    if (out) *out = nullptr;
    if (!out || !A || !b || !valid_shape(n, c)) return ES_EINVAL;
    const size_t wsb = es_workspace_bytes(n, c);
    void *dA = nullptr, *db = nullptr, *ws = nullptr;
    int rc = ES_OK;
    if (hipMalloc(&dA, (size_t)n * n * 8) != hipSuccess || hipMalloc(&db, (size_t)n * c * 8) != hipSuccess ||
        hipMalloc(&ws, wsb) != hipSuccess) {
        rc = ES_ENOMEM;
    } else if (hipMemcpy(dA, A, (size_t)n * n * 8, hipMemcpyHostToDevice) != hipSuccess ||
               hipMemcpy(db, b, (size_t)n * c * 8, hipMemcpyHostToDevice) != hipSuccess) {
        rc = ES_EHIP;
    } else {
        rc = es_solve_device((const int64_t*)dA, (const int64_t*)db, n, c, ws, wsb, nullptr, out);
    }
    if (dA) (void)hipFree(dA);
    if (db) (void)hipFree(db);
    if (ws) (void)hipFree(ws);
    return rc;
}

int32_t es_solution_rows(const es_solution* s) { return s ? s->data.n : 0; }
int32_t es_solution_cols(const es_solution* s) { return s ? s->data.c : 0; }

int es_solution_get(const es_solution* s, int32_t i, int32_t k, int* num_sign, const uint64_t** num,
                    int32_t* num_len, const uint64_t** den, int32_t* den_len) {
    if (!s || !num_sign || !num || !num_len || !den || !den_len) return ES_EINVAL;
    if (i < 0 || i >= s->data.n || k < 0 || k >= s->data.c) return ES_EINVAL;
    const size_t idx = (size_t)i * s->data.c + k;
    const BigInt& nu = s->data.num[idx];
    const BigInt& de = s->data.den(idx);
    *num_sign = nu.is_zero() ? 0 : (nu.neg ? -1 : 1);
    *num = nu.d.data();
    *num_len = (int32_t)nu.size();
    *den = de.d.data();
    *den_len = (int32_t)de.size();
    return ES_OK;
}

int es_solution_info(const es_solution* s, int32_t* live_primes, int32_t* m, int32_t* num_bound_bits,
                     int32_t* den_bound_bits) {
    if (!s) return ES_EINVAL;
    if (live_primes) *live_primes = s->data.live;
    if (m) *m = s->data.m;
    if (num_bound_bits) *num_bound_bits = s->data.nbits;
    if (den_bound_bits) *den_bound_bits = s->data.dbits;
    return ES_OK;
}

int32_t es_solution_modulus_bits(const es_solution* s) { return s ? s->data.mbits : 0; }

void es_solution_free(es_solution* s) { delete s; }

}  // extern "C"

namespace {

// The batched inverse in the first inverse_bytes(L) bytes of ws.
int batched_inverse_in(const int64_t* dA, const Layout& L, uint8_t* ws, hipStream_t st, int8_t* dB_out,
                       int32_t* flags_host) {
    Prep pr;
    pr.L = L;
    // the norms of b are not needed here; A stands in for it
    int rc = prepare_launch(dA, dA, L.n, 1, ws, st, &pr);
    if (rc != ES_OK) return rc;
    int flags[kNumPrimes];
    Profiler prof(st);
    rc = run_inverse(dA, ws, st, &pr, flags, &prof);
    if (rc != ES_OK) return rc;
    rc = prepare_finish(L.n, 1, &pr);
    if (rc == ES_SINGULAR) rc = ES_OK;  // a zero row/column just makes every prime singular
    if (rc != ES_OK) return rc;
    HIP_CHECK(launch_export_inverse(pr.L, ws, dB_out, st));
    HIP_CHECK(hipStreamSynchronize(st));
    for (int j = 0; j < kNumPrimes; j++) flags_host[j] = flags[j] ? 1 : 0;
    return ES_OK;
}

}  // namespace

extern "C" {

int es_batched_inverse(const int64_t* dA, int32_t n, void* d_ws, size_t ws_bytes, void* stream, int8_t* dB_out,
                       int32_t* flags_host) {
    if (!dA || !d_ws || !dB_out || !flags_host || !valid_shape(n, 1)) return ES_EINVAL;
    const Layout L = make_layout(n, 1);
    if (ws_bytes < L.total) return ES_EINVAL;
    try {
        return batched_inverse_in(dA, L, (uint8_t*)d_ws, (hipStream_t)stream, dB_out, flags_host);
    } catch (...) {
        return ES_EINTERNAL;
    }
}

int32_t es_noalloc_max_n(void) {
    // the largest n whose inverse fits the fixed scratch (the bytes grow with n)
    int32_t lo = 0, hi = 1 << 16;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        if (inverse_bytes(make_layout(mid, 1)) <= fixed_scratch_bytes()) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

int es_batched_inverse_noalloc(const int64_t* dA, int32_t n, void* stream, int8_t* dB_out, int32_t* flags_host) {
    if (!dA || !dB_out || !flags_host || !valid_shape(n, 1)) return ES_EINVAL;
    try {
        const Layout L = make_layout(n, 1);
        if (inverse_bytes(L) > fixed_scratch_bytes()) return ES_ETOOBIG;
        uint8_t* ws = fixed_scratch();
        if (!ws) return ES_EHIP;
        return batched_inverse_in(dA, L, ws, (hipStream_t)stream, dB_out, flags_host);
    } catch (...) {
        return ES_EINTERNAL;
    }
}

int es_lift_digits(const int64_t* dA, const int64_t* db, int32_t n, int32_t c, void* d_ws, size_t ws_bytes,
                   void* stream, int32_t m_req, int64_t* digits_host, size_t digits_cap,
                   uint64_t* live_mask_host, int32_t* m_out) {
    if (!dA || !db || !d_ws || !live_mask_host || !m_out || !valid_shape(n, c)) return ES_EINVAL;
    Prep pr;
    pr.L = make_layout(n, c);
    if (ws_bytes < pr.L.total) return ES_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)d_ws;
    try {
        int rc = prepare_launch(dA, db, n, c, ws, st, &pr);
        if (rc != ES_OK) return rc;
        int flags[kNumPrimes];
        Profiler prof(st);
        rc = run_inverse(dA, ws, st, &pr, flags, &prof);
        if (rc != ES_OK) return rc;
        rc = prepare_finish(n, c, &pr);
        if (rc != ES_OK) return rc;
        LiveSet ls = make_live_set(flags);
        if (ls.E == 0) return no_prime_decision(dA, n, pr, st);
        int m = m_req;
        if (m <= 0) {
            BigInt M;
            m = choose_m(ls.P, pr.nbits, pr.dbits, &M);
        }
        uint64_t mask = 0;
        for (int l = 0; l < ls.E; l++) mask |= 1ULL << ls.idx[l];
        *live_mask_host = mask;
        *m_out = m;
        if (!digits_host) return ES_OK;  // query: m and the live set only
        if ((size_t)n * c * m * kDigitLimbs > digits_cap) return ES_EINVAL;
        rc = run_lift(dA, db, ws, st, pr, ls, m, digits_host, &prof);
        prof.collect();
        return rc;
    } catch (...) {
        return ES_EINTERNAL;
    }
}

int es_reconstruct(const int64_t* digits, int32_t n, int32_t c, int32_t m, uint64_t live_mask, int32_t num_bits,
                   int32_t den_bits, int32_t nthreads, es_solution** out) {
    if (out) *out = nullptr;
    if (!digits || !out || !valid_shape(n, c) || m < 1 || num_bits < 0 || den_bits < 0) return ES_EINVAL;
    if (live_mask == 0 || (live_mask >> kNumPrimes) != 0) return ES_EINVAL;
    try {
        LiveSet ls = live_set_from_mask(live_mask);
        BigInt M = pow_u(ls.P, (unsigned)m);
        if (M.bit_length() < (size_t)num_bits + den_bits + 2) return ES_EINVAL;
        es_solution* sol = new es_solution;
        int rc = reconstruct(digits, (size_t)m, n, c, m, ls.P, M, num_bits, den_bits,
                             nthreads > 0 ? nthreads : default_threads(), &sol->data);
        if (rc != ES_OK) {
            delete sol;
            return rc;
        }
        sol->data.live = ls.E;
        sol->data.m = m;
        sol->data.nbits = num_bits;
        sol->data.dbits = den_bits;
        *out = sol;
        return ES_OK;
    } catch (const std::bad_alloc&) {
        return ES_ENOMEM;
    } catch (...) {
        return ES_EINTERNAL;
    }
}

}  // extern "C"
