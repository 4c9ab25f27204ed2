// Reconstruction on the GPU: plan, device scratch and the host driver
// (recon_host.cpp; kernels in recon.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "bignum.h"
#include "host.h"

namespace es {

// Sizes and scratch layout for one solve.  ok is false when the GPU
// path does not apply (too few words in M, rows wider than one wave can
// hold, more than 1365 lift steps, or more than 16 GiB of scratch); the
// host path then reconstructs from digits copied to the host.
struct GpuReconPlan {
    bool ok = false;
    int n = 0, c = 0, m = 0;
    size_t NC = 0;
    int TM = 0, NW = 0;       // top word index of M, words per weight row
    int nw = 0;               // words kept per numerator (nbits / 32 + 1)
    int Ncolsp = 0, Kpad = 0; // GEMM columns (bytes of a weight row, padded), contraction bytes
    int NCc = 0, NCcp = 0;    // components per GEMM chunk, padded to 128
    size_t off_digits = 0;    // uint64 [NC][m][6]  lift digits (written by the CRT kernel)
    size_t off_S = 0;         // int8 [NCcp][Kpad]  balanced digit bytes of a chunk
    size_t off_rowsum = 0;    // int32 [NCcp]
    size_t off_T = 0;         // uint32 [m][NW]     P^i d mod M
    size_t off_Mw = 0;        // uint32 [NW]        M
    size_t off_W = 0;         // uint8 [Kpad][Ncolsp] weight rows
    size_t off_WT = 0;        // int8 [Ncolsp][Kpad]  transposed, offset by -128
    size_t off_VT = 0;        // int32 [NCcp][Ncolsp] GEMM column sums, one row per component
    size_t off_Y = 0;         // uint32 [NCcp][nw]  numerators
    size_t off_status = 0;    // int32 [NCcp]
    size_t off_Dw = 0;        // uint32 [NW]        the common denominator d
    size_t off_G = 0;         // uint64 [NCcp]      gcd(|y|, d) when it fits 64 bits
    size_t off_gstat = 0;     // int32 [NCcp]       0: G valid, 1: the host computes the gcd
    size_t total = 0;
};

// Event timing hooks for the hot kernels (no-ops unless profiling is on).
struct KernelTimer {
    virtual long start(int cls) = 0;
    // the same for a bracket that holds exactly one kernel launch, timed by
    // that kernel's own dispatch
    virtual long start_one(int cls) { return start(cls); }
    virtual void stop(long idx) = 0;
    virtual ~KernelTimer() = default;
};
enum { KC_RECON_GEMM = 5, KC_RECON_OTHER = 6, KC_RECON_GCD = 7 };

struct GpuReconTimes {
    double sample_ms = 0, seeds_ms = 0, gpu_ms = 0, finish_ms = 0;
    size_t failed = 0;       // components reconstructed alone (outside the numerator bound)
    size_t host_gcds = 0;    // gcds the GPU handed back
};

// The host reconstruction is used when es_set_gpu_reconstruction(0) was
// called on this thread, or (without such a call) when ES_RECON=host.
bool gpu_recon_disabled();
void set_gpu_recon(bool on);

GpuReconPlan plan_gpu_recon(int n, int c, int m, size_t mbits, int nbits);  // mbits: bit length of M = P^m

// Scratch bytes that the workspace of an n x n system with c right-hand
// sides reserves for the GPU reconstruction (0 when the path never applies
// to that shape): the largest plan over every input within the range limit
// n max|A| < 2^63 for which at most kReserveDrops primes divide det A,
// capped at the widest modulus the GPU path takes.  The plan's sizes grow
// with m, the bit length of M and the numerator bound, so every such input's
// plan fits; any other input takes the host reconstruction (same result).
constexpr int kReserveDrops = 5;
size_t gpu_recon_reserve(int n, int c);

// Reconstruction from the digits at scr + pl.off_digits (scr: pl.total bytes
// of device memory, part of the caller's workspace).  pw holds P^0 .. P^m,
// so M = pw[m].  Returns ES_OK, ES_EHIP, ES_ENOMEM or ES_EINTERNAL.
int reconstruct_gpu(const GpuReconPlan& pl, uint8_t* scr, const BigInt& P, const std::vector<BigInt>& pw,
                    int nbits, int dbits, int nthreads, hipStream_t st, SolutionData* out, GpuReconTimes* tm,
                    KernelTimer* kt);

}  // namespace es
