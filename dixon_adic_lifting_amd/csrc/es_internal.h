// Internal declarations shared by the host runtime (api.cpp, host.cpp) and
// the HIP kernels (kernels.hip).  Not part of the public C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace es {

// Events that the next kernel launched on this thread records at its own
// start and end (from its dispatch, with no marker packets around it); set
// by the per-kernel timer, empty otherwise.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& pending_launch_events();

// Every kernel launch of the library goes through here.
template <typename F, typename... Args>
inline void es_launch(F kernel, const dim3& grid, const dim3& block, uint32_t shmem, hipStream_t st, Args... args) {
    LaunchEvents& pe = pending_launch_events();
    const LaunchEvents ev = pe;
    pe = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, ev.start, ev.stop, 0u, args...);
}

constexpr int kNumPrimes = 53;   // odd primes below 256
constexpr int kDigitLimbs = 6;   // one base-P digit, 384-bit two's complement
constexpr int kDigitWords = 12;  // the same in 32-bit words

// Odd primes below 256 (Eratosthenes) with their Barrett constants:
// mu16 = floor(2^16 / q) reduces x < 2^16; mu32 = floor(2^32 / q) reduces
// x < 2^32; r32 = 2^32 mod q folds the high word of a 64-bit value.
// mq24 = ceil(2^24 / q) gives the exact quotient floor(x / q) =
// floor(x mq24 / 2^24) for every x < 2^16 (round-up reciprocal with
// 16 + 8 bits of precision, q <= 2^8), so no correction step follows.
struct PrimeTable {
    uint32_t q[kNumPrimes];
    uint32_t mu16[kNumPrimes];
    uint32_t mu32[kNumPrimes];
    uint32_t r32[kNumPrimes];
    uint32_t mq24[kNumPrimes];
};

constexpr PrimeTable make_prime_table() {
    PrimeTable t{};
    bool composite[256] = {};
    for (unsigned i = 2; i < 256; i++)
        if (!composite[i])
            for (unsigned j = i * i; j < 256; j += i) composite[j] = true;
    int cnt = 0;
    for (unsigned v = 3; v < 256; v++) {
        if (composite[v]) continue;
        t.q[cnt] = v;
        t.mu16[cnt] = 65536u / v;
        t.mu32[cnt] = (uint32_t)(4294967296ull / v);
        t.r32[cnt] = (uint32_t)(4294967296ull % v);
        t.mq24[cnt] = (uint32_t)((16777216ull + v - 1) / v);
        cnt++;
    }
    return t;
}

constexpr PrimeTable kPrimeTable = make_prime_table();

// Inverses modulo each prime: inv[j][a] = a^-1 mod q_j (inv[j][0] = 0), from
// the recurrence a^-1 = -(q div a) (q mod a)^-1 mod q.
struct InverseTable {
    uint8_t inv[kNumPrimes][256];
};

constexpr InverseTable make_inverse_table() {
    InverseTable t{};
    for (int j = 0; j < kNumPrimes; j++) {
        const uint32_t q = kPrimeTable.q[j];
        t.inv[j][1] = 1;
        for (uint32_t a = 2; a < q; a++)
            t.inv[j][a] = (uint8_t)((q - (q / a) * t.inv[j][q % a] % q) % q);
    }
    return t;
}

constexpr InverseTable kInverseTable = make_inverse_table();
static_assert(kInverseTable.inv[52][250] == 250 && kInverseTable.inv[0][2] == 2, "inverse table");
static_assert(kPrimeTable.q[0] == 3 && kPrimeTable.q[kNumPrimes - 1] == 251, "prime table");

// Per-solve constants of the lift, for the live primes in ascending order.
// Lives in the device workspace; kernels read it with uniform (scalar) loads.
struct LiftParams {
    int32_t E;                    // number of live primes
    int32_t pad0;
    uint64_t Pinv;                // P^-1 mod 2^64 (P odd)
    uint32_t qidx[kNumPrimes];    // index into the 53-prime table
    uint32_t q[kNumPrimes];
    uint32_t mu16[kNumPrimes];
    uint32_t mu32[kNumPrimes];
    uint32_t r32[kNumPrimes];
    uint32_t cinv[kNumPrimes];    // (P / q_l)^-1 mod q_l
    uint32_t Pw[kDigitWords];     // words of P
    uint32_t Phw[kDigitWords];    // words of (P - 1) / 2
    uint32_t pad1[1];
    double qrec[kNumPrimes];      // 1 / q_l
    double Wd[kNumPrimes][kDigitWords];  // words of P / q_l (exact in double)
};

// Device workspace layout for an n x n system with c right-hand sides.
struct Layout {
    int n, c;
    int pitch;            // row pitch of the residue matrices, bytes
    int lpr;              // lanes per row in the row kernels (4 .. 64)
    int kchunk;           // lift steps whose digits the device buffer holds
    size_t off_S;         // u8/int8 [53][n][pitch]   GJ matrix, then B_j
    size_t off_piv;       // int32 [53][n + 1]         pivot row per step
    size_t off_rowpos;    // int32 [53][n]             step at which a row pivoted
    size_t off_pend;      // u8 [2][53][pitch]         scaled pivot rows
    size_t off_GT;        // int8 [53][pitch][32]      old pivot rows of a panel, transposed
    size_t off_flags;     // int32 [53]                singular mod q_j
    size_t off_wq;        // int32 [n / 32 + 2][8]     blocked elimination: per panel, the update's per-XCD tile queues
    size_t off_rowmax;    // uint64 [n]                max |A_ij| per row
    size_t off_rownorm;   // double [n]                row norms^2 of A
    size_t off_colpart;   // double [ceil(n/64)][n]    column partial sums
    size_t off_colnorm;   // double [n]                column norms^2 of A
    size_t off_bpart;     // double [ceil(n/64)][c]
    size_t off_bnorm;     // double [c]                column norms^2 of b
    size_t off_A32;       // int32 [n][n]              A when |A| < 2^31
    size_t off_R;         // int64 [n][c]              residual r_i
    size_t off_rho;       // int8 [53][c][pitch]       r_i mods q_j, permuted
    size_t off_U;         // u8 [53][n*c]              (B_j r_i) mod q_j
    size_t off_xlow;      // uint64 [n][c]             x_i mod 2^64
    size_t off_rpos;      // int32 [n][64]             (c = 1) row i's position in live prime l's order, l < E
    size_t off_Ab;        // int8 [4][n][pitch]        (c > 1) A as four balanced byte planes, for the MFMA residual
    size_t off_xp;        // int8 [8 c][pitch]         (c > 1) x_low as eight balanced byte planes, row 8 b c + t
    size_t off_Sperm;     // int8 [53][n][pitch]       (c = 1, pitch >= 1024) B_j rows in component order, live primes
    size_t off_urec;      // u8 [krec][n][64]          (same condition) per step: balanced CRT residues, k at byte 63
    int krec;             // lift steps whose records the device buffer holds
    size_t off_digits;    // uint64 [n*c][kchunk][6]   digits of a chunk of steps
    size_t off_params;    // LiftParams
    size_t total;
    uint64_t* dig_dev;    // when set, the digits go here ([n*c][kchunk][6]) instead
};

// Shapes that take the fused lift (contraction and the step's CRT share in
// one kernel): one right-hand side, rows of at least 1 KB, and every prime's
// matrix within one 2 GiB buffer resource.
inline bool fused_lift_shape(int n, int c, int pitch) {
    return c == 1 && pitch >= 1024 && (size_t)kNumPrimes * n * pitch <= (size_t)0x7fffffff;
}

// The layout depends on (n, c) only.
Layout make_layout(int n, int c);
// bytes at the start of a layout that the batched inverse touches (its
// matrices, pivots, panels, norms, the int32 copy of A and the residues the
// set-up clears)
size_t inverse_bytes(const Layout& L);
// Fixed device scratch of the entry point that allocates nothing (one copy
// per device, shared by every call on it): its size, and this device's copy
// (NULL if the address lookup fails).
size_t fixed_scratch_bytes();
uint8_t* fixed_scratch();
// cap on the record steps that later lifts on the calling thread use per
// launch (0: none); the layout keeps room for its default count either way
void set_lift_record_cap(int steps);
// record steps per launch for a lift with layout L on the calling thread
int lift_record_steps(const Layout& L);

// ---------------------------------------------------------------- launchers
// Each enqueues on `st` and returns the launch status.

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t st);
hipError_t launch_stats(const int64_t* A, const int64_t* b, const Layout& L, uint8_t* ws,
                        hipStream_t st);
// also writes the int32 copy of A (meaningful only when every |A_ij| < 2^31)
hipError_t launch_residues(const int64_t* A, const Layout& L, uint8_t* ws, hipStream_t st,
                           bool balanced_out = false);
hipError_t launch_gj_step(const Layout& L, uint8_t* ws, int k, hipStream_t st);
// blocked form of the same elimination: 32 steps per panel launch, then one
// MFMA update launch (residues must be balanced: launch_residues(..., true))
constexpr int kPanel = 32;
// rows of the blocked elimination's queue counters (one per lookahead launch)
inline int work_queue_rows(int n) { return n / kPanel + 2; }
int device_cu_count();
bool blocked_inverse_fits(const Layout& L);
hipError_t launch_gj_panel(const Layout& L, uint8_t* ws, int K, hipStream_t st);
hipError_t launch_gj_update(const Layout& L, uint8_t* ws, int K, hipStream_t st);
// lookahead form: panel K together with the update of panel K - 32 outside
// the columns [K - 32, K + 32) (K = 0: the panel alone; K >= n: the update
// alone), and after each panel its pivot rows to GT with the update of the
// next panel's columns
hipError_t launch_gj_panel_rest(const Layout& L, uint8_t* ws, int K, hipStream_t st);
hipError_t launch_gj_gather_next(const Layout& L, uint8_t* ws, int K, hipStream_t st);
hipError_t launch_export_inverse(const Layout& L, const uint8_t* ws, int8_t* B, hipStream_t st);
// r = b and its residues (natural: in natural row order, the MFMA residual's path)
hipError_t launch_split_b(const int64_t* b, const Layout& L, uint8_t* ws, int E, bool natural, hipStream_t st);
// one lift step = contraction, then the CRT (digit into chunk slot `slot`),
// then the residual update with the split of the new residual
hipError_t launch_lift_contract(const Layout& L, uint8_t* ws, int E, hipStream_t st);
hipError_t launch_lift_crt(const Layout& L, uint8_t* ws, int slot, bool planes, hipStream_t st);
// one right-hand side: the contraction and the CRT in one launch (after
// launch_lift_rows once per lift, which copies the live primes' B_j rows
// into component order); false when the layout does not take it
bool lift_fused_fits(const Layout& L);
// digits of records [0, nrec) of the record buffer into digit slots
// slot0 .. slot0 + nrec - 1 of the current chunk
hipError_t launch_lift_crt_records(const Layout& L, uint8_t* ws, int nrec, int slot0, hipStream_t st);
// The residual as int8 MFMA products of byte planes (c > 1, |A| < 2^30):
// A's planes once per lift, then per step the CRT also writes x_low's planes.
bool residual_mfma_fits(const Layout& L, bool a32, uint64_t maxabs);
hipError_t launch_a_planes(const Layout& L, uint8_t* ws, hipStream_t st);
// S's live-prime rows in natural column order (the MFMA residual's path;
// the lift's residues are then in natural order too)
hipError_t launch_natural_cols(const Layout& L, uint8_t* ws, int E, hipStream_t st);
// the residual's position table (c = 1), once per lift
hipError_t launch_lift_positions(const Layout& L, uint8_t* ws, hipStream_t st);
hipError_t launch_lift_rows(const Layout& L, uint8_t* ws, int E, hipStream_t st);
hipError_t launch_lift_contract_crt(const Layout& L, uint8_t* ws, int E, int slot, hipStream_t st);
hipError_t launch_lift_residual(const Layout& L, uint8_t* ws, bool a32, const int64_t* A64, bool mfma,
                                hipStream_t st);

// reconstruction on the GPU (recon.hip); see the kernels for layouts
hipError_t launch_digit_bytes(const uint64_t* digits, int dstride, int m, int j0, int valid_rows, int rows_pad,
                              int Kpad, int8_t* S, int* rowsum, hipStream_t st);
hipError_t launch_wchain(const uint32_t* T, const uint32_t* Mw, int m, int TM, double Md, int Ncolsp, uint8_t* W,
                         hipStream_t st);
int wchain_words_per_lane(int NW);  // 0 when NW words do not fit one wave
hipError_t launch_transpose_offset(const uint8_t* W, int Kpad, int Ncolsp, int8_t* WT, hipStream_t st);
hipError_t launch_recon_gemm(const int8_t* S, const int8_t* WT, int Kpad, int NCcp, int Ncolsp, int* VT,
                             hipStream_t st);
int gcd_words_per_lane(int words);  // 0 when the numbers do not fit one wave
// group: components per block, 0 to choose it from valid_rows
hipError_t launch_gcd(const uint32_t* Y, int nw, const int* status, int valid_rows, const uint32_t* Dw, int nwd,
                      uint64_t* G, int* gstat, int group, hipStream_t st);
// Components of the first of two gcd launches over valid_rows components
// (valid_rows when one launch should serve them all) and, in *group, the
// components per block both launches use.  The split falls on a whole round
// of the CUs' resident blocks and leaves about a fifth of the rounds to the
// second launch, so that the host can finish the first launch's components
// while the second runs; only launches of four rounds or more are split.
int gcd_split(int valid_rows, int nw, int nwd, int* group);
int numer_words_per_lane(int NW);  // 0 when a numerator pass does not fit one wave
hipError_t launch_numer(const int* V, int Ncolsp, const int* rowsum, int valid_rows, const uint32_t* Mw, int TM,
                        double Mtop, int nbits, uint32_t* Y, int* status, hipStream_t st);

}  // namespace es
