// HIP kernels for CDNA4 (gfx950): the hot path of multi-prime Dixon lifting.
//
// Method: exact-solve card (phanerozoic/exact-solve), section "Method":
//   * batched modular inverse: Gauss-Jordan on [A | I] mod every odd prime
//     q_j < 256 at once, one launch per elimination step across all primes,
//     Barrett reduction instead of a hardware modulo;
//   * lift step: per-prime balanced-residue int8 contraction with int32
//     accumulation, a balanced CRT into the wide base-P digit, and the
//     one-limb residual update (r_i - A x_i) P^-1 mod 2^64 (P odd);
//   * range limits (card, "Method"/"Requirements"): n * max|A_ij| < 2^63 so
//     the residual is one signed 64-bit limb; n <= 2^17 so int8 x int8
//     products accumulate in int32 without overflow.
//
// Layout (see es_internal.h, Layout): the residue matrices are u8/int8
// [53][n][pitch] with a power-of-two (n <= 1024) or 64-aligned row pitch so
// that one lane always moves 16 aligned bytes.  The Gauss-Jordan inverse runs
// in place without physical row swaps: the row chosen as pivot of column k
// (piv[j][k]) keeps its place, and slot k of every row then holds column
// piv[j][k] of the inverse.  rowpos[j][i] records the step at which row i
// became the pivot.  Hence A^-1 mod q_j = S_j with rows gathered by piv and
// columns scattered by rowpos, and the lift uses S_j as is: its input vector
// is stored permuted by rowpos and its outputs are scattered by rowpos.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "es_internal.h"

namespace es {

__constant__ PrimeTable c_pt = kPrimeTable;
__constant__ InverseTable c_inv = kInverseTable;

// ---------------------------------------------------------------- arithmetic

// x mod q for x < 2^16 (Barrett with mu16 = floor(2^16/q)): the estimate
// floor(x mu16 / 2^16) is floor(x/q) or one less, so one conditional
// subtraction finishes; min(r, r - q) is that subtraction in unsigned form.
__device__ __forceinline__ uint32_t red16(uint32_t x, uint32_t q, uint32_t mu16) {
    uint32_t t = __umul24(x, mu16) >> 16;
    uint32_t r = x - __umul24(t, q);
    return min(r, r - q);
}

// x mod q for x < 2^32 (Barrett with mu32 = floor(2^32/q)).
__device__ __forceinline__ uint32_t red32(uint32_t x, uint32_t q, uint32_t mu32) {
    uint32_t t = __umulhi(x, mu32);
    uint32_t r = x - t * q;
    return min(r, r - q);
}

// u mod q for u < 2^64: fold the high word with r32 = 2^32 mod q.
__device__ __forceinline__ uint32_t red64(uint64_t u, uint32_t q, uint32_t mu16, uint32_t mu32,
                                          uint32_t r32) {
    uint32_t h = red32((uint32_t)(u >> 32), q, mu32);
    uint32_t l = red32((uint32_t)u, q, mu32);
    return red16(h * r32 + l, q, mu16);  // <= (q-1)^2 + (q-1) < 2^16
}

// signed 64-bit value mod q in [0, q)
__device__ __forceinline__ uint32_t mod_i64(int64_t a, uint32_t q, uint32_t mu16, uint32_t mu32,
                                            uint32_t r32) {
    uint64_t u = a < 0 ? (uint64_t)0 - (uint64_t)a : (uint64_t)a;
    uint32_t r = red64(u, q, mu16, mu32, r32);
    return (a < 0 && r) ? q - r : r;
}

// signed 32-bit value mod q in [0, q)
__device__ __forceinline__ uint32_t mod_i32(int32_t a, uint32_t q, uint32_t mu32) {
    uint32_t u = a < 0 ? (uint32_t)0 - (uint32_t)a : (uint32_t)a;
    uint32_t r = red32(u, q, mu32);
    return (a < 0 && r) ? q - r : r;
}

// balanced representative in [-(q-1)/2, (q-1)/2] of r in [0, q), q odd
__device__ __forceinline__ int balanced(uint32_t r, uint32_t q) {
    return r > (q >> 1) ? (int)r - (int)q : (int)r;
}

// a^-1 mod q by Fermat (a != 0 mod q, q prime)
__device__ __forceinline__ uint32_t inv_mod(uint32_t a, uint32_t q, uint32_t mu16) {
    uint32_t r = 1, b = a, e = q - 2;
    while (e) {
        if (e & 1) r = red16(r * b, q, mu16);
        b = red16(b * b, q, mu16);
        e >>= 1;
    }
    return r;
}

__device__ __forceinline__ void unpack16(const uint4 w, uint32_t (&x)[16]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int b = 0; b < 4; b++) x[4 * i + b] = (ws[i] >> (8 * b)) & 0xffu;
    }
}

__device__ __forceinline__ uint4 pack16(const uint32_t (&x)[16]) {
    uint32_t ws[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        ws[i] = (x[4 * i] & 0xffu) | ((x[4 * i + 1] & 0xffu) << 8) | ((x[4 * i + 2] & 0xffu) << 16) |
                ((x[4 * i + 3] & 0xffu) << 24);
    return make_uint4(ws[0], ws[1], ws[2], ws[3]);
}

// ---------------------------------------------------------------- utility

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t count, uint32_t value) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < count; i += stride) p[i] = value;
}

hipError_t launch_fill_u32(uint32_t* p, size_t count, uint32_t value, hipStream_t st) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    es_launch(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, count, value);
    return hipGetLastError();
}

// ---------------------------------------------------------------- range check and norms
// Feeds the range check n * max|A| < 2^63 (card, "Method") and the Hadamard
// bounds that fix the step count.  Reductions run in a fixed order, so the
// fp64 sums (and hence the step count) are reproducible.

__global__ __launch_bounds__(256) void row_stats_kernel(const int64_t* __restrict__ A, int n,
                                                        uint64_t* __restrict__ rowmax,
                                                        double* __restrict__ rownorm) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    uint64_t mx = 0;
    double s = 0.0;
    const int64_t* a = A + (size_t)row * n;
    for (int j = lane; j < n; j += 64) {
        int64_t v = a[j];
        uint64_t u = v < 0 ? (uint64_t)0 - (uint64_t)v : (uint64_t)v;
        mx = u > mx ? u : mx;
        double f = (double)v;
        s += f * f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint64_t o = __shfl_xor(mx, off);
        mx = o > mx ? o : mx;
        s += __shfl_xor(s, off);
    }
    if (lane == 0) {
        rowmax[row] = mx;
        rownorm[row] = s;
    }
}

// partial column sums of squares over a 64-row block
__global__ __launch_bounds__(256) void col_part_kernel(const int64_t* __restrict__ M, int rows,
                                                       int cols, double* __restrict__ part) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    const int rb = blockIdx.y;
    if (col >= cols) return;
    const int r0 = rb * 64, r1 = min(rows, r0 + 64);
    double s = 0.0;
    for (int r = r0; r < r1; r++) {
        double f = (double)M[(size_t)r * cols + col];
        s += f * f;
    }
    part[(size_t)rb * cols + col] = s;
}

__global__ __launch_bounds__(256) void col_final_kernel(const double* __restrict__ part, int nrb,
                                                        int cols, double* __restrict__ out) {
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= cols) return;
    double s = 0.0;
    for (int rb = 0; rb < nrb; rb++) s += part[(size_t)rb * cols + col];
    out[col] = s;
}

hipError_t launch_stats(const int64_t* A, const int64_t* b, const Layout& L, uint8_t* ws,
                        hipStream_t st) {
    const int n = L.n, c = L.c, nrb = (n + 63) / 64;
    es_launch(row_stats_kernel, dim3((n + 3) / 4), dim3(256), 0, st, A, n,
                       (uint64_t*)(ws + L.off_rowmax), (double*)(ws + L.off_rownorm));
    es_launch(col_part_kernel, dim3((n + 255) / 256, nrb), dim3(256), 0, st, A, n, n,
                       (double*)(ws + L.off_colpart));
    es_launch(col_final_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                       (const double*)(ws + L.off_colpart), nrb, n, (double*)(ws + L.off_colnorm));
    es_launch(col_part_kernel, dim3((c + 255) / 256, nrb), dim3(256), 0, st, b, n, c,
                       (double*)(ws + L.off_bpart));
    es_launch(col_final_kernel, dim3((c + 255) / 256), dim3(256), 0, st,
                       (const double*)(ws + L.off_bpart), nrb, c, (double*)(ws + L.off_bnorm));
    return hipGetLastError();
}

// ---------------------------------------------------------------- residues of A
// The 53 residue bytes of four entries (magnitudes mag, signs neg) of row i
// from column col: BIG reduces 64-bit magnitudes, else 32-bit ones.
template <bool BIG>
__device__ __forceinline__ void residue_bytes(const uint64_t* mag, const bool* neg, int n, int pitch, int i,
                                              int col, uint8_t* __restrict__ S, int bal) {
    for (int j = 0; j < kNumPrimes; j++) {
        const uint32_t q = c_pt.q[j], mu16 = c_pt.mu16[j], mu32 = c_pt.mu32[j], r32 = c_pt.r32[j];
        uint32_t w = 0;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            uint32_t r = BIG ? red64(mag[u], q, mu16, mu32, r32) : red32((uint32_t)mag[u], q, mu32);
            if (neg[u] && r) r = q - r;
            if (bal && r > (q >> 1)) r = (r - q) & 0xffu;  // balanced residue as a two's-complement byte
            w |= r << (8 * u);
        }
        *(uint32_t*)(S + ((size_t)j * n + i) * pitch + col) = w;
    }
}

// S[j][i][col] = A[i][col] mod q_j for all 53 primes (zero in the pitch
// padding), reduced from 32 bits where a thread's four magnitudes fit them;
// and an int32 copy of A for the residual update (used only when every
// entry fits, which the host learns from the range statistics meanwhile).
__global__ __launch_bounds__(256) void residue_kernel(const int64_t* __restrict__ A, int n, int pitch,
                                                      uint8_t* __restrict__ S,
                                                      int32_t* __restrict__ A32, int bal) {
    const int i = blockIdx.x;
    const int col = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (col >= pitch) return;
    uint64_t mag[4];
    bool neg[4];
    uint64_t any = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        int64_t a = (col + u < n) ? A[(size_t)i * n + col + u] : 0;
        if (col + u < n) A32[(size_t)i * n + col + u] = (int32_t)a;
        neg[u] = a < 0;
        mag[u] = a < 0 ? (uint64_t)0 - (uint64_t)a : (uint64_t)a;
        any |= mag[u];
    }
    if (any >> 32)
        residue_bytes<true>(mag, neg, n, pitch, i, col, S, bal);
    else
        residue_bytes<false>(mag, neg, n, pitch, i, col, S, bal);
}

// first pivot (step 0) per prime: the lowest row with a nonzero residue in column 0
__global__ __launch_bounds__(256) void pivot0_kernel(const uint8_t* __restrict__ S, int n, int pitch,
                                                     int* __restrict__ piv) {
    const int j = blockIdx.x;
    __shared__ int smin;
    if (threadIdx.x == 0) smin = INT_MAX;
    __syncthreads();
    int cand = INT_MAX;
    for (int i = threadIdx.x; i < n; i += 256)
        if (S[((size_t)j * n + i) * pitch] != 0) {
            cand = i;
            break;
        }
    if (cand != INT_MAX) atomicMin(&smin, cand);
    __syncthreads();
    if (threadIdx.x == 0) piv[(size_t)j * (n + 1)] = smin;
}

// compute units of the current device (queried once per device)
int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        cache[dev] = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0
                         ? cus
                         : 256;
    }
    return cache[dev];
}

hipError_t launch_residues(const int64_t* A, const Layout& L, uint8_t* ws, hipStream_t st, bool balanced_out) {
    dim3 grid(L.n, (L.pitch / 4 + 255) / 256);
    es_launch(residue_kernel, grid, dim3(256), 0, st, A, L.n, L.pitch, ws + L.off_S, (int32_t*)(ws + L.off_A32),
              balanced_out ? 1 : 0);
    if (balanced_out) {  // the blocked elimination's update queues start empty
        const hipError_t e = launch_fill_u32((uint32_t*)(ws + L.off_wq), (size_t)work_queue_rows(L.n) * 8, 0u, st);
        if (e != hipSuccess) return e;
    }
    if (!balanced_out)  // the step-wise elimination takes its first pivot from here
        es_launch(pivot0_kernel, dim3(kNumPrimes), dim3(256), 0, st,
                           (const uint8_t*)(ws + L.off_S), L.n, L.pitch, (int*)(ws + L.off_piv));
    return hipGetLastError();
}

// ---------------------------------------------------------------- Gauss-Jordan step
// One launch per elimination step k, grid (row tiles, 53 primes).  With the
// pivot row p = piv[j][k] (chosen by the previous launch) scaled to
// v = S[p] * inv(S[p][k]) and v[k] = inv(S[p][k]), every other row becomes
// S[i] <- S[i] with slot k cleared, plus (q - S[i][k]) * v, mod q.  The
// pivot row itself is not written back here (other blocks are still reading
// it): its scaled form goes to a side buffer, and its owner folds it back
// into S as an ordinary row in the next launch.  While updating, each block
// records the lowest not-yet-pivoted row with a nonzero entry in column
// k + 1, which becomes the next pivot (atomicMin), so no separate pivot
// search is launched.  A prime with no pivot is singular mod q_j: its flag
// is set and all of its later launches exit at once.  The last step writes
// balanced int8 residues, the operand format of the lift.
//
// Arithmetic runs "one byte up": each residue s sits in bits 8..15 of a
// 32-bit lane value and x' = 256 (s + f v) < 2^24.  With mq24 = ceil(2^24/q)
// the high word of the 24 x 24-bit product x' mq24 (v_mul_hi_u32_u24) is the
// exact quotient floor(x / q), and x' - 256 q floor(x/q) (one signed 24-bit
// multiply-add) is 256 (x mod q) with no correction step.  Bytes move in and
// out of that position with byte permutes, so an element costs about five
// VALU operations.

// byte b of w placed in bits 8..15 (other bits zero)
__device__ __forceinline__ uint32_t byte_up(uint32_t w, int b) {
    return __builtin_amdgcn_perm(0u, w, 0x0c0c000cu | ((uint32_t)b << 8));
}

__device__ __forceinline__ uint32_t mulhi_u24(uint32_t a, uint32_t b) {
    return (uint32_t)(((uint64_t)(a & 0xffffffu) * (uint64_t)(b & 0xffffffu)) >> 32);
}

// a * b + c on signed 24-bit operands, b uniform across the wave.  Written as
// an instruction because the compiler otherwise widens t * q to the
// quarter-rate 32-bit multiply.
__device__ __forceinline__ uint32_t mad_i24(uint32_t a, int32_t b, uint32_t c) {
    uint32_t r;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
    return r;
}

// Balanced x mod q for odd q < 256 and |x| < 2^19, in full-rate operations:
// t = x / q rounded to nearest in single precision is the nearest integer to
// x / q, because the float product (x exact, 1 / q and the product each
// rounded once) lies within 2^-23 2^19 / q = 2^-4 / q of x / q, while x / q,
// q odd, lies at least 1 / (2q) from every half-integer; x - t q is then the
// residue in [-(q - 1) / 2, (q - 1) / 2].  rq = 1 / q rounded, nq = -q.
__device__ __forceinline__ int bal_mod_19(int x, float rq, int32_t nq) {
    const int t = (int)__builtin_rintf((float)x * rq);
    return (int)mad_i24((uint32_t)t, nq, (uint32_t)x);
}

// 256 (x mod q) from xs = 256 x, x < 2^16 (exact quotient, no correction)
__device__ __forceinline__ uint32_t red_up(uint32_t xs, uint32_t mq24, int32_t nq8) {
    return mad_i24(mulhi_u24(xs, mq24), nq8, xs);
}

// four values held in bits 8..15 -> one packed word (byte b from e[b])
__device__ __forceinline__ uint32_t pack_up(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3) {
    const uint32_t lo = __builtin_amdgcn_perm(e1, e0, 0x0c0c0501u);
    const uint32_t hi = __builtin_amdgcn_perm(e3, e2, 0x0c0c0501u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

template <int LPR, int RI, bool LAST>
__global__ __launch_bounds__(256) void gj_step_kernel(uint8_t* __restrict__ S, int n, int pitch,
                                                      int k, int* __restrict__ piv,
                                                      int* __restrict__ rowpos,
                                                      uint8_t* __restrict__ pend,
                                                      int* __restrict__ flags) {
    constexpr int RPW = 64 / LPR;           // rows per wave and pass
    constexpr int ROWS = 4 * RPW * RI;      // rows per block
    const int j = blockIdx.y;
    int* pj = piv + (size_t)j * (n + 1);
    uint8_t* Sj = S + (size_t)j * n * pitch;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, cl = lane % LPR;
    const int npass = (LPR == 64) ? (pitch + 1023) >> 10 : 1;
    const int row0 = blockIdx.x * ROWS;

    // Issue this thread's first-pass row loads and column-k bytes before the
    // pivot index arrives: they depend only on the row index (the previous
    // step's pivot row is re-read from the side buffer below).
    uint4 s[RI];
    uint32_t f[RI];
#pragma unroll
    for (int r = 0; r < RI; r++) {
        const int i = row0 + wave * RPW + g + r * 4 * RPW;
        const bool ok = i < n && cl * 16 < pitch;
        s[r] = ok ? *(const uint4*)(Sj + (size_t)i * pitch + cl * 16) : make_uint4(0, 0, 0, 0);
        f[r] = i < n ? Sj[(size_t)i * pitch + k] : 0u;
    }
    const int p = pj[k];
    const int pprev = k > 0 ? pj[k - 1] : -1;
    if (p == INT_MAX) {
        if (blockIdx.x == 0 && threadIdx.x == 0) flags[j] = 1;
        return;
    }
    const uint32_t q = c_pt.q[j], mq = c_pt.mq24[j];
    const uint32_t q8 = q << 8, half8 = (q >> 1) << 8;
    const int32_t nq8 = -(int32_t)q8;
    int* rpj = rowpos + (size_t)j * n;
    const uint8_t* pend_prev = pend + ((size_t)((k + 1) & 1) * kNumPrimes + j) * pitch;
    uint8_t* pend_cur = pend + ((size_t)(k & 1) * kNumPrimes + j) * pitch;
    const uint32_t pinv = c_inv.inv[j][Sj[(size_t)p * pitch + k]];
    int cand = INT_MAX;

    // live[r]: row r is updated here (it exists and is not the pivot row);
    // the previous pivot row's current content is in the side buffer
    bool live[RI];
    uint32_t fneg[RI];
#pragma unroll
    for (int r = 0; r < RI; r++) {
        const int i = row0 + wave * RPW + g + r * 4 * RPW;
        live[r] = i < n && i != p;
        fneg[r] = 0;
        if (live[r]) {
            if (i == pprev) {
                f[r] = pend_prev[k];
                if (cl * 16 < pitch) s[r] = *(const uint4*)(pend_prev + cl * 16);
            }
            fneg[r] = f[r] ? q - f[r] : 0;
        }
    }
    const bool own_p = (p >= row0 && p < row0 + ROWS) && ((p - row0) % (4 * RPW)) == wave * RPW + g;

    for (int pass = 0; pass < npass; ++pass) {
        const int col0 = pass * 1024 + cl * 16;
        if (col0 >= pitch) continue;
        if (pass > 0) {
#pragma unroll
            for (int r = 0; r < RI; r++) {
                const int i = row0 + wave * RPW + g + r * 4 * RPW;
                const uint8_t* src = (i == pprev) ? pend_prev : Sj + (size_t)i * pitch;
                s[r] = live[r] ? *(const uint4*)(src + col0) : make_uint4(0, 0, 0, 0);
            }
        }
        // scaled pivot row, one byte up; slot k holds pinv
        uint32_t vs[16];
        {
            const uint4 raw = *(const uint4*)(Sj + (size_t)p * pitch + col0);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int b = 0; b < 16; b++) {
                const uint32_t xs = __umul24(byte_up(w[b >> 2], b & 3), pinv);  // 256 x pinv < 2^24
                vs[b] = (col0 + b == k) ? (pinv << 8) : red_up(xs, mq, nq8);
            }
        }
        if (own_p) {  // the pivot row's new content goes to the side buffer
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t e[4];
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    uint32_t y = vs[4 * i + b];
                    if (LAST) y = (y > half8 ? y - q8 : y) & 0xff00u;  // balanced, two's complement byte
                    e[b] = y;
                }
                o[i] = pack_up(e[0], e[1], e[2], e[3]);
            }
            *(uint4*)(pend_cur + col0) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        // slot k of every other row is cleared before the update: a per-lane word mask
        const int kk = k - col0, kk1 = k + 1 - col0;
        uint32_t kmask[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            kmask[i] = (kk >= 0 && kk < 16 && (kk >> 2) == i) ? ~(0xffu << (8 * (kk & 3))) : 0xffffffffu;
#pragma unroll
        for (int r = 0; r < RI; r++) {
            if (!live[r]) continue;
            const uint32_t w[4] = {s[r].x & kmask[0], s[r].y & kmask[1], s[r].z & kmask[2], s[r].w & kmask[3]};
            const uint32_t fr = fneg[r];
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t e[4];
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    const uint32_t xs = byte_up(w[i], b) + __umul24(fr, vs[4 * i + b]);  // 256 (s + f v)
                    uint32_t y = red_up(xs, mq, nq8);
                    if (LAST) y = (y > half8 ? y - q8 : y) & 0xff00u;
                    e[b] = y;
                }
                o[i] = pack_up(e[0], e[1], e[2], e[3]);
            }
            const int i = row0 + wave * RPW + g + r * 4 * RPW;
            if (!LAST && kk1 >= 0 && kk1 < 16) {
                const uint32_t word = (kk1 >> 2) == 0 ? o[0] : (kk1 >> 2) == 1 ? o[1] : (kk1 >> 2) == 2 ? o[2] : o[3];
                if (((word >> (8 * (kk1 & 3))) & 0xffu) != 0 && rpj[i] < 0) cand = min(cand, i);
            }
            *(uint4*)(Sj + (size_t)i * pitch + col0) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    if (threadIdx.x == 0 && p >= row0 && p < row0 + ROWS) rpj[p] = k;
    if (!LAST) {
        __shared__ int smin;
        if (threadIdx.x == 0) smin = INT_MAX;
        __syncthreads();
        if (cand != INT_MAX) atomicMin(&smin, cand);
        __syncthreads();
        if (threadIdx.x == 0 && smin != INT_MAX) atomicMin(&pj[k + 1], smin);
    }
}

// After the last step: fold each prime's final pivot row back into S.
__global__ __launch_bounds__(256) void gj_finalize_kernel(uint8_t* __restrict__ S, int n, int pitch,
                                                          const int* __restrict__ piv,
                                                          const uint8_t* __restrict__ pend) {
    const int j = blockIdx.x;
    const int p = piv[(size_t)j * (n + 1) + n - 1];
    if (p == INT_MAX) return;
    const uint8_t* src = pend + ((size_t)((n - 1) & 1) * kNumPrimes + j) * pitch;
    uint8_t* dst = S + ((size_t)j * n + p) * pitch;
    for (int col = threadIdx.x * 4; col < pitch; col += 1024)
        *(uint32_t*)(dst + col) = *(const uint32_t*)(src + col);
}

// Rows per thread for the wide-row Gauss-Jordan kernel (4 unless ES_GJ_RI=8):
// a tuning knob, both variants compute the same result.
static int gj_rows_per_thread() {
    static const int v = [] {
        const char* e = getenv("ES_GJ_RI");
        return (e && e[0] == '8') ? 8 : 4;
    }();
    return v;
}

template <int LPR, int RI>
static void launch_gj_t(const Layout& L, uint8_t* ws, int k, hipStream_t st) {
    constexpr int ROWS = 4 * (64 / LPR) * RI;
    dim3 grid((L.n + ROWS - 1) / ROWS, kNumPrimes);
    if (k == L.n - 1)
        es_launch((gj_step_kernel<LPR, RI, true>), grid, dim3(256), 0, st, ws + L.off_S, L.n, L.pitch,
                           k, (int*)(ws + L.off_piv), (int*)(ws + L.off_rowpos), ws + L.off_pend,
                           (int*)(ws + L.off_flags));
    else
        es_launch((gj_step_kernel<LPR, RI, false>), grid, dim3(256), 0, st, ws + L.off_S, L.n,
                           L.pitch, k, (int*)(ws + L.off_piv), (int*)(ws + L.off_rowpos), ws + L.off_pend,
                           (int*)(ws + L.off_flags));
}

hipError_t launch_gj_step(const Layout& L, uint8_t* ws, int k, hipStream_t st) {
    switch (L.lpr) {
        case 4: launch_gj_t<4, 1>(L, ws, k, st); break;
        case 8: launch_gj_t<8, 1>(L, ws, k, st); break;
        case 16: launch_gj_t<16, 2>(L, ws, k, st); break;
        case 32: launch_gj_t<32, 4>(L, ws, k, st); break;
        default:
            if (gj_rows_per_thread() == 8) launch_gj_t<64, 8>(L, ws, k, st);
            else launch_gj_t<64, 4>(L, ws, k, st);
            break;
    }
    if (k == L.n - 1)
        es_launch(gj_finalize_kernel, dim3(kNumPrimes), dim3(256), 0, st, ws + L.off_S, L.n,
                           L.pitch, (const int*)(ws + L.off_piv), (const uint8_t*)(ws + L.off_pend));
    return hipGetLastError();
}

// ---------------------------------------------------------------- blocked elimination
// The same in-place Gauss-Jordan (each step k exchanges row piv[k] with
// column k: the pivot row is scaled by the inverse pivot, slot k keeps the
// inverse-matrix entry, every other row loses its column-k multiple), run 32
// steps at a time.  Exchanging b pivot pairs (rows p_c, columns K + c) at
// once is the block form of that step: with the panel columns Kc and the
// rest r, the panel after its own b steps holds S'[Pi, Kc] = S[Pi, Kc]^-1 and
// S'[i, Kc] = -S[i, Kc] S[Pi, Kc]^-1 for the other rows, and every other
// column follows as
//     S'[i, r] = [i not a pivot of the panel] S[i, r] + sum_c S'[i, K + c] S[p_c, r],
// a rank-32 update of the whole matrix by the old pivot rows: one int8 GEMM
// per prime on the matrix cores.  Pivots are the same as the step-wise
// kernel's (lowest unused row with a nonzero entry), so piv, rowpos and the
// final S are identical.  Residues are kept balanced, as int8 operands need.

// (x mod q) balanced, for |x| < 2^15 - 2^9 (every product of two residues
// plus one): with off = q ceil(2^15 / q), x' = x + off lies in (0, 2^16), so
// the round-up reciprocal mq24 gives the exact quotient
__device__ __forceinline__ int bal_red16(int x, uint32_t q, uint32_t mq, int off) {
    const uint32_t xs = (uint32_t)(x + off) << 8;  // 256 x', x' < 2^16
    const uint32_t r = mad_i24(mulhi_u24(xs, mq), -(int)(q << 8), xs) >> 8;
    return (int)r > (int)(q >> 1) ? (int)r - (int)q : (int)r;
}

typedef int v4i_t __attribute__((ext_vector_type(4)));

// Panel pieces shared by both panel kernels.  Rows that pivoted in earlier
// panels (clist[nc .. n)) get S'[i, Kc] = -S[i, Kc] Z, 16 rows per product;
// first operand Z^T (16 output columns c' per product, k = c), second the
// rows' panel bytes; each output lane holds one row and four consecutive
// columns c'.
__device__ __forceinline__ void panel_old_rows(int8_t* __restrict__ Sj, int n, int pitch, int K, int nc,
                                               const int* clist, const int8_t (*Zt)[64], uint32_t q, int lane,
                                               int wave) {
    const int lr = lane & 15, lg = lane >> 4;
    // |S Z| <= 32 * 125^2 < 2^19
    const float rq = 1.0f / (float)q;
    const int32_t nq = -(int32_t)q;
    v4i_t za[2];
#pragma unroll
    for (int a = 0; a < 2; a++) za[a] = lg < 2 ? *(const v4i_t*)(&Zt[16 * a + lr][16 * lg]) : v4i_t{0, 0, 0, 0};
    const int nother = n - nc;
    for (int tile = wave; 16 * tile < nother; tile += 16) {
        const int k = nc + 16 * tile + lr;
        const int i = k < n ? clist[k] : -1;
        const v4i_t sb =
            (lg < 2 && i >= 0) ? *(const v4i_t*)(Sj + (size_t)i * pitch + K + 16 * lg) : v4i_t{0, 0, 0, 0};
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const v4i_t acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(za[a], sb, v4i_t{0, 0, 0, 0}, 0, 0, 0);
            uint32_t outw = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) outw |= ((uint32_t)bal_mod_19(-acc[e], rq, nq) & 0xffu) << (8 * e);
            if (i >= 0) *(uint32_t*)(Sj + (size_t)i * pitch + K + 16 * a + 4 * lg) = outw;
        }
    }
}

// Columns col .. col + 3 of pivot rows r0 .. r0 + 7 (of the panel's bw,
// rows plist[c]) into GT transposed ([col][c], 32 bytes a column): eight
// word loads, the 8 x 4 bytes regrouped in registers, and one 8-byte slice
// of each of the four columns' GT rows.  col + 3 < pitch.
__device__ __forceinline__ void gt_slice(const int8_t* __restrict__ Sj, int pitch, int bw,
                                         const int* __restrict__ plist, int8_t* __restrict__ GTj, int col, int r0) {
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 8; r++)
        w[r] = r0 + r < bw ? *(const uint32_t*)(Sj + (size_t)plist[r0 + r] * pitch + col) : 0u;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            lo |= ((w[r] >> (8 * b)) & 0xffu) << (8 * r);
            hi |= ((w[r + 4] >> (8 * b)) & 0xffu) << (8 * r);
        }
        *(uint2*)(GTj + (size_t)(col + b) * kPanel + r0) = make_uint2(lo, hi);
    }
}

// The panel's pivot rows (all columns) to GT, by a 1024-thread block:
// thread t takes columns 4 (t mod 256) + 1024 i .. + 3 of the pivot rows
// 8 (t / 256) .. + 7 (each wave's loads cover 256 contiguous bytes of a
// row; the pitch is a multiple of 64).
__device__ __forceinline__ void panel_gather_gt(const int8_t* __restrict__ Sj, int pitch, int bw,
                                                const int* __restrict__ plist, int8_t* __restrict__ GTj, int t) {
    const int r0 = 8 * (t >> 8);
    for (int col = 4 * (t & 255); col < pitch; col += 1024) gt_slice(Sj, pitch, bw, plist, GTj, col, r0);
}

// The candidate rows (no pivot step yet, rowpos < 0) in row order at
// clist[0 .. nc), the other rows after them; returns nc.  Every thread of the
// block takes part (barriers inside).
__device__ __forceinline__ int panel_list_rows(const int* __restrict__ rpj, int n, int* clist, int* wsum, int t,
                                               int lane, int wave) {
    int nc = 0;
    for (int base = 0; base < n; base += 1024) {
        const int i = base + t;
        const bool cand = i < n && rpj[i] < 0;
        const uint64_t m = __ballot(cand);
        if (lane == 0) wsum[wave] = __popcll(m);
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < 16; w++) {
            const int v = wsum[w];
            before += w < wave ? v : 0;
            tot += v;
        }
        const int pos = nc + before + __popcll(m & ((1ull << lane) - 1));
        if (cand) clist[pos] = i;
        else if (i < n) clist[n - 1 - (i - pos)] = i;  // the (i - pos)-th other row, listed from the end
        nc += tot;
        __syncthreads();
    }
    return nc;
}

// Panel: one block of 1024 threads per prime.  Only the rows that can still
// become pivots (no pivot step yet, rowpos < 0) take part in the steps: a
// block-wide prefix sum lists them in row order, and thread t keeps
// candidates t, t + 1024, ... (RPT of them), each as the 32 panel bytes in
// eight registers, held as residues in [0, q).  Each step: every wave finds
// its lowest candidate with a nonzero byte kk and the owner publishes that
// row in the wave's LDS slot; after one barrier every thread takes the lowest
// of the sixteen and reads the row from its slot.  Every listed row then
// updates itself as base + factor * prow' (mod q), where prow' is the raw
// pivot row with a 1 in slot kk, base is the row with slot kk cleared (zero
// for the pivot row itself) and factor is -f pinv (pinv for the pivot row):
// the scaled-pivot-row update with the scaling folded into one factor per
// row, in the byte-up arithmetic of the step kernel.  After the steps the
// panel's pivot rows hold Z = S[Pi, Kc]^-1 (row c for the pivot of step c),
// and every row that pivoted in an earlier panel takes the block form of the
// same steps, S'[i, Kc] = -S[i, Kc] Z: one int8 product per 16 rows on the
// matrix cores.  The panel goes back to S (balanced) and the old pivot rows
// (all columns) go to GT transposed, [col][c] with 32 bytes per column, the
// update's operand layout.
// (The bodies below run the panel of prime j in the calling block and return
// false when the prime is, or turns out to be, singular.)
template <int RPT>
__device__ __forceinline__ bool panel_packed_body(int8_t* __restrict__ S, int n, int pitch, int K,
                                                  int* __restrict__ piv, int* __restrict__ rowpos,
                                                  int* __restrict__ flags, int j) {
    if (flags[j]) return false;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint32_t q = c_pt.q[j], mq = c_pt.mq24[j];
    const int32_t nq8 = -(int32_t)(q << 8);
    const int bw = min(kPanel, n - K);
    int8_t* Sj = S + (size_t)j * n * pitch;
    int* rpj = rowpos + (size_t)j * n;
    int* pj = piv + (size_t)j * (n + 1);
    __shared__ int clist[1024 * RPT];      // candidate rows in row order, then the other rows
    __shared__ int wsum[16];
    __shared__ __attribute__((aligned(16))) uint32_t slot[2][16][8];  // per wave: its best candidate's row
    __shared__ __attribute__((aligned(16))) int sidx[2][16];          // and that candidate's index
    __shared__ int plist[kPanel];
    __shared__ __attribute__((aligned(16))) int8_t Zt[kPanel][64];  // Zt[c'][c] = Z[c][c'], zero-padded
    __shared__ uint8_t inv[256];  // inverses mod q_j

    ((int16_t*)&Zt[0][0])[t] = 0;  // 1024 threads x 2 bytes
    if (t < 256) inv[t] = c_inv.inv[j][t];
    const int nc = panel_list_rows(rpj, n, clist, wsum, t, lane, wave);

    uint32_t pw[RPT][8];
    bool live[RPT];
    int pc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const int k = t + 1024 * r;
        live[r] = k < nc;
        pc[r] = -1;
        if (live[r]) {
            const int i = clist[k];
            const uint4 a = *(const uint4*)(Sj + (size_t)i * pitch + K);
            const uint4 b = *(const uint4*)(Sj + (size_t)i * pitch + K + 16);
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {  // balanced bytes -> residues in [0, q)
                uint32_t o = 0;
#pragma unroll
                for (int bb = 0; bb < 4; bb++) {
                    const int x = (int)(int8_t)(w[e] >> (8 * bb));
                    o |= (uint32_t)(x < 0 ? x + (int)q : x) << (8 * bb);
                }
                pw[r][e] = o;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++) pw[r][e] = 0;
        }
    }
    for (int kk = 0; kk < bw; kk++) {
        const int kw = kk >> 2, ks = 8 * (kk & 3), buf = kk & 1;
        uint32_t fk[RPT];  // byte kk of each row
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            uint32_t w = pw[r][0];
#pragma unroll
            for (int e = 1; e < 8; e++) w = kw == e ? pw[r][e] : w;
            fk[r] = (w >> ks) & 0xffu;
        }
        // this wave's lowest candidate with a nonzero byte kk: candidates
        // t + 1024 r come in order of r, then of lane
        int best = INT_MAX;
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            const uint64_t m = __ballot(live[r] && fk[r] != 0u);
            if (best == INT_MAX && m != 0) {
                const int wl = __builtin_ctzll(m);
                best = 64 * wave + wl + 1024 * r;
                if (lane == wl) {
                    uint4* dst = (uint4*)&slot[buf][wave][0];
                    dst[0] = make_uint4(pw[r][0], pw[r][1], pw[r][2], pw[r][3]);
                    dst[1] = make_uint4(pw[r][4], pw[r][5], pw[r][6], pw[r][7]);
                }
            }
        }
        if (lane == 0) sidx[buf][wave] = best;
        __syncthreads();
        int p = INT_MAX;
        {
            const int4* si = (const int4*)&sidx[buf][0];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int4 v = si[g];
                p = min(min(p, v.x), min(v.y, min(v.z, v.w)));
            }
        }
        const int pwv = (p >> 6) & 15;  // candidate t + 1024 r is in wave t / 64
        if (p == INT_MAX) {  // no pivot: singular modulo q_j
            if (t == 0) flags[j] = 1;
            return false;
        }
        if (t == (p & 1023)) {
            const int pr = p >> 10;
#pragma unroll
            for (int r = 0; r < RPT; r++) {
                if (r != pr) continue;
                live[r] = false;
                pc[r] = kk;
            }
            const int prow_i = clist[p];
            pj[K + kk] = prow_i;
            rpj[prow_i] = K + kk;
            plist[kk] = prow_i;
        }
        // prow' one byte up, with 1 in slot kk
        uint32_t vs[32];
        uint32_t prw[8];
        {
            const uint4* src = (const uint4*)&slot[buf][pwv][0];
            const uint4 a = src[0], b = src[1];
            prw[0] = a.x, prw[1] = a.y, prw[2] = a.z, prw[3] = a.w;
            prw[4] = b.x, prw[5] = b.y, prw[6] = b.z, prw[7] = b.w;
        }
        uint32_t pkw = prw[0];
#pragma unroll
        for (int e = 1; e < 8; e++) pkw = kw == e ? prw[e] : pkw;
        const uint32_t pinv = inv[(pkw >> ks) & 0xffu];
        pkw = (pkw & ~(0xffu << ks)) | (1u << ks);  // the 1 in slot kk
#pragma unroll
        for (int e = 0; e < 8; e++) prw[e] = kw == e ? pkw : prw[e];
#pragma unroll
        for (int e = 0; e < 8; e++)
#pragma unroll
            for (int bb = 0; bb < 4; bb++) vs[4 * e + bb] = byte_up(prw[e], bb);
        // a wave whose slots all lie past the candidate list has nothing to update
        if (64 * wave >= nc) continue;
        uint32_t kmask[8];
#pragma unroll
        for (int e = 0; e < 8; e++) kmask[e] = e == kw ? ~(0xffu << ks) : 0xffffffffu;
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            const int k = t + 1024 * r;
            if (k >= nc) continue;
            const bool isp = k == p;
            if (!isp && fk[r] == 0u) continue;  // nothing to eliminate in this row
            // factor: -f pinv for other rows, pinv for the pivot row
            const uint32_t g = red_up(__umul24(fk[r], pinv) << 8, mq, nq8) >> 8;
            const uint32_t fac = isp ? pinv : (g ? q - g : 0u);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t w = isp ? 0u : (pw[r][e] & kmask[e]);
                uint32_t o[4];
#pragma unroll
                for (int bb = 0; bb < 4; bb++) o[bb] = red_up(byte_up(w, bb) + __umul24(fac, vs[4 * e + bb]), mq, nq8);
                pw[r][e] = pack_up(o[0], o[1], o[2], o[3]);
            }
        }
    }
    // listed rows back to S, balanced; the pivot rows' bytes also form Z
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const int k = t + 1024 * r;
        if (k >= nc) continue;
        const int i = clist[k];
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            uint32_t o = 0;
#pragma unroll
            for (int bb = 0; bb < 4; bb++) {
                const uint32_t x = (pw[r][e] >> (8 * bb)) & 0xffu;
                o |= ((x > (q >> 1) ? x - q : x) & 0xffu) << (8 * bb);
            }
            w[e] = o;
        }
        *(uint4*)(Sj + (size_t)i * pitch + K) = make_uint4(w[0], w[1], w[2], w[3]);
        *(uint4*)(Sj + (size_t)i * pitch + K + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        if (pc[r] >= 0) {
#pragma unroll
            for (int cc = 0; cc < kPanel; cc++) Zt[cc][pc[r]] = (int8_t)(w[cc >> 2] >> (8 * (cc & 3)));
        }
    }
    __syncthreads();
    panel_old_rows(Sj, n, pitch, K, nc, clist, Zt, q, lane, wave);
    return true;
}

// The panel's 32 steps on the first candidates only.  The pivot of step kk
// is the lowest listed candidate with a nonzero entry in column kk after the
// earlier steps, so when the first T = min(nc, 64) candidates hold one for
// every step, the pivots found among them are those of the whole list, and
// every other row (candidate or earlier pivot) leaves the panel as
// S'[i, Kc] = -S[i, Kc] Z, the block form the earlier pivot rows take.  One
// wave runs the steps with no barrier: lane l holds candidate l's panel
// bytes (byte-up residues, as in the panel below), the pivot is the lowest
// lane of a ballot, and its row reaches every lane through readlane.
// Nothing is written unless all 32 steps find their pivot among the T rows:
// then the T rows go back to S (balanced), Z to Zt, and the pivots to piv,
// rowpos and plist, and the function returns T; otherwise it returns 0 and
// the caller runs the panel over the whole list.  Called by wave 0 only.
__device__ __forceinline__ int panel_top_steps(int8_t* __restrict__ Sj, int pitch, int K, int nc,
                                               const int* clist, int* __restrict__ pj, int* __restrict__ rpj,
                                               int* plist, int8_t (*Zt)[64], const uint8_t* inv, uint32_t q,
                                               uint32_t mq, int32_t nq8, int lane) {
    const int T = min(nc, 64);
    const bool mine = lane < T;
    uint32_t W[kPanel];
    {
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (mine) {
            const int i = clist[lane];
            const uint4 a = *(const uint4*)(Sj + (size_t)i * pitch + K);
            const uint4 b = *(const uint4*)(Sj + (size_t)i * pitch + K + 16);
            w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w, w[4] = b.x, w[5] = b.y, w[6] = b.z, w[7] = b.w;
        }
#pragma unroll
        for (int c = 0; c < kPanel; c++) {
            const int x = (int)(int8_t)(w[c >> 2] >> (8 * (c & 3)));
            W[c] = (uint32_t)(x < 0 ? x + (int)q : x) << 8;
        }
    }
    bool live = mine;
    int pcol = -1;
    int pl[kPanel];  // the candidate index (lane) of each step's pivot
#pragma clang loop unroll(full)
    for (int kk = 0; kk < kPanel; kk++) {
        const uint32_t fk = W[kk] >> 8;
        const uint64_t m = __ballot(live && fk != 0u);
        if (m == 0) return 0;  // no pivot among the first T candidates
        const int p = __builtin_ctzll(m);
        pl[kk] = p;
        uint32_t vs[kPanel];
#pragma unroll
        for (int c = 0; c < kPanel; c++) vs[c] = (uint32_t)__builtin_amdgcn_readlane((int)W[c], p);
        const uint32_t pinv = inv[vs[kk] >> 8];
        vs[kk] = 256u;
        const bool isp = lane == p;
        if (isp) {
            live = false;
            pcol = kk;
        }
        // as in the panel below: base (slot kk cleared) + fac prow'
        const uint32_t g = red_up(__umul24(fk, pinv) << 8, mq, nq8) >> 8;
        const uint32_t fac = isp ? pinv - 1u : (g ? q - g : 0u);
        W[kk] = 0u;
#pragma unroll
        for (int c = 0; c < kPanel; c++) W[c] = red_up(__umul24(fac, vs[c]) + W[c], mq, nq8);
        W[kk] = isp ? pinv << 8 : W[kk];
    }
    // every step found its pivot: the T rows back to S, Z, the pivots
    if (mine) {
        const int i = clist[lane];
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            uint32_t o = 0;
#pragma unroll
            for (int bb = 0; bb < 4; bb++) {
                const uint32_t x = W[4 * e + bb] >> 8;
                o |= ((x > (q >> 1) ? x - q : x) & 0xffu) << (8 * bb);
            }
            w[e] = o;
        }
        *(uint4*)(Sj + (size_t)i * pitch + K) = make_uint4(w[0], w[1], w[2], w[3]);
        *(uint4*)(Sj + (size_t)i * pitch + K + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        if (pcol >= 0) {
#pragma unroll
            for (int cc = 0; cc < kPanel; cc++) Zt[cc][pcol] = (int8_t)(w[cc >> 2] >> (8 * (cc & 3)));
            pj[K + pcol] = i;
            rpj[i] = K + pcol;
            plist[pcol] = i;
        }
    }
    (void)pl;
    return T;
}

// The same panel with every candidate row held unpacked: one register per
// panel byte, in byte-up form (256 x, x in [0, q)), so a step costs three
// instructions per element (x' = 256 base + fac 256 v, then the exact
// round-up reduction); the steps are unrolled, so the byte of column kk is a
// fixed register.  For up to 1024 rows (one row per thread: 32 registers);
// the byte-packed kernel above covers larger systems.  Same pivots, same
// results.
template <int RPT>
__device__ __forceinline__ bool panel_up_body(int8_t* __restrict__ S, int n, int pitch, int K,
                                              int* __restrict__ piv, int* __restrict__ rowpos,
                                              int* __restrict__ flags, int j) {
    if (flags[j]) return false;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint32_t q = c_pt.q[j], mq = c_pt.mq24[j];
    const int32_t nq8 = -(int32_t)(q << 8);
    const int bw = kPanel;
    int8_t* Sj = S + (size_t)j * n * pitch;
    int* rpj = rowpos + (size_t)j * n;
    int* pj = piv + (size_t)j * (n + 1);
    __shared__ int clist[1024 * RPT];
    __shared__ int wsum[16];
    __shared__ __attribute__((aligned(16))) uint32_t slot[2][16][kPanel];  // per wave: its best candidate's row (byte-up)
    __shared__ __attribute__((aligned(16))) int sidx[2][16];          // and that candidate's index
    __shared__ int plist[kPanel];
    __shared__ __attribute__((aligned(16))) int8_t Zt[kPanel][64];  // Zt[c'][c] = Z[c][c'], zero-padded
    __shared__ uint8_t inv[256];

    ((int16_t*)&Zt[0][0])[t] = 0;
    if (t < 256) inv[t] = c_inv.inv[j][t];
    const int nc = panel_list_rows(rpj, n, clist, wsum, t, lane, wave);
    {
        // the steps on the first candidates alone (almost always enough);
        // then every other row by the block formula
        __shared__ int topT;
        if (wave == 0) {
            const int T = panel_top_steps(Sj, pitch, K, nc, clist, pj, rpj, plist, Zt, inv, q, mq, nq8, lane);
            if (lane == 0) topT = T;
        }
        __syncthreads();
        const int T = topT;
        if (T > 0) {
            panel_old_rows(Sj, n, pitch, K, T, clist, Zt, q, lane, wave);
            return true;
        }
    }

    uint32_t W[RPT][kPanel];  // 256 x residue
    bool live[RPT];
    int pc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const int k = t + 1024 * r;
        live[r] = k < nc;
        pc[r] = -1;
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (live[r]) {
            const int i = clist[k];
            const uint4 a = *(const uint4*)(Sj + (size_t)i * pitch + K);
            const uint4 b = *(const uint4*)(Sj + (size_t)i * pitch + K + 16);
            w[0] = a.x, w[1] = a.y, w[2] = a.z, w[3] = a.w, w[4] = b.x, w[5] = b.y, w[6] = b.z, w[7] = b.w;
        }
#pragma unroll
        for (int c = 0; c < kPanel; c++) {
            const int x = (int)(int8_t)(w[c >> 2] >> (8 * (c & 3)));
            W[r][c] = (uint32_t)(x < 0 ? x + (int)q : x) << 8;
        }
    }
    // fully unrolled (a full panel: bw = 32), so that column kk is a fixed
    // register in every step; a prime found singular runs the remaining steps
    // without effect and leaves after them
    bool dead = false;
#pragma clang loop unroll(full)
    for (int kk = 0; kk < kPanel; kk++) {
        const int buf = kk & 1;
        uint32_t fk[RPT];
#pragma unroll
        for (int r = 0; r < RPT; r++) fk[r] = W[r][kk] >> 8;
        int best = INT_MAX;
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            const uint64_t m = __ballot(live[r] && fk[r] != 0u);
            if (best == INT_MAX && m != 0) {
                const int wl = __builtin_ctzll(m);
                best = 64 * wave + wl + 1024 * r;
                if (lane == wl) {
                    // published as held (one byte up), so no lane unpacks it
                    uint4* dst = (uint4*)&slot[buf][wave][0];
#pragma unroll
                    for (int e = 0; e < kPanel / 4; e++)
                        dst[e] = make_uint4(W[r][4 * e], W[r][4 * e + 1], W[r][4 * e + 2], W[r][4 * e + 3]);
                }
            }
        }
        if (lane == 0) sidx[buf][wave] = best;
        __syncthreads();
        int p = INT_MAX;
        {
            const int4* si = (const int4*)&sidx[buf][0];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int4 v = si[g];
                p = min(min(p, v.x), min(v.y, min(v.z, v.w)));
            }
        }
        const int pwv = (p >> 6) & 15;  // candidate t + 1024 r is in wave t / 64
        if (p == INT_MAX) {  // no pivot: singular modulo q_j
            if (t == 0 && !dead) flags[j] = 1;
            dead = true;
        }
        if (!dead && t == (p & 1023)) {
            const int pr = p >> 10;
#pragma unroll
            for (int r = 0; r < RPT; r++) {
                if (r != pr) continue;
                live[r] = false;
                pc[r] = kk;
            }
            const int prow_i = clist[p];
            pj[K + kk] = prow_i;
            rpj[prow_i] = K + kk;
            plist[kk] = prow_i;
        }
        // prow' one byte up, with 1 in slot kk
        uint32_t vs[kPanel];
        {
            const uint4* src = (const uint4*)&slot[buf][pwv][0];
#pragma unroll
            for (int e = 0; e < kPanel / 4; e++) {
                const uint4 v = src[e];
                vs[4 * e] = v.x, vs[4 * e + 1] = v.y, vs[4 * e + 2] = v.z, vs[4 * e + 3] = v.w;
            }
        }
        const uint32_t pinv = dead ? 0u : inv[vs[kk] >> 8];
        vs[kk] = 256u;
        // a wave whose slots lie past the candidate list holds only zeros,
        // which the update leaves as they are: it skips the update (the list
        // shrinks by 64 rows a wave as the panels advance)
        if (64 * wave >= nc) continue;
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            // every row without a branch: base (slot kk cleared) + fac prow'
            // with fac = -f pinv, which leaves a row with f = 0 as it is; the
            // pivot row equals prow' outside slot kk, so fac = pinv - 1 scales
            // it by pinv there, and its slot kk is set to pinv
            const bool isp = t + 1024 * r == p;
            const uint32_t g = red_up(__umul24(fk[r], pinv) << 8, mq, nq8) >> 8;
            const uint32_t fac = isp ? pinv - 1u : (g ? q - g : 0u);
            W[r][kk] = 0u;
#pragma unroll
            for (int c = 0; c < kPanel; c++) W[r][c] = red_up(__umul24(fac, vs[c]) + W[r][c], mq, nq8);
            W[r][kk] = isp ? pinv << 8 : W[r][kk];
        }
    }
    if (dead) return false;
    // listed rows back to S, balanced; the pivot rows' bytes also form Z
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const int k = t + 1024 * r;
        if (k >= nc) continue;
        const int i = clist[k];
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            uint32_t o = 0;
#pragma unroll
            for (int bb = 0; bb < 4; bb++) {
                const uint32_t x = W[r][4 * e + bb] >> 8;
                o |= ((x > (q >> 1) ? x - q : x) & 0xffu) << (8 * bb);
            }
            w[e] = o;
        }
        *(uint4*)(Sj + (size_t)i * pitch + K) = make_uint4(w[0], w[1], w[2], w[3]);
        *(uint4*)(Sj + (size_t)i * pitch + K + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        if (pc[r] >= 0) {
#pragma unroll
            for (int cc = 0; cc < kPanel; cc++) Zt[cc][pc[r]] = (int8_t)(w[cc >> 2] >> (8 * (cc & 3)));
        }
    }
    __syncthreads();
    panel_old_rows(Sj, n, pitch, K, nc, clist, Zt, q, lane, wave);
    return true;
}

// Rank-32 update of the columns outside the panel, all rows, one tile of
// 128 columns x 128 rows per four waves.  v_mfma_i32_16x16x64_i8 with the
// old pivot rows (GT, [col][c]) as the first operand and the new panel
// (S[i][K .. K + 32), zero beyond 32) as the second, so each output lane
// holds four consecutive columns of one row:
// C[i][col] = sum_c S'[i][K + c] S[p_c][col]; then
// S'[i][col] = [i not pivot] S[i][col] + C, reduced balanced.  The columns
// in [skip0, skip1) (both ends multiples of 32, holding the panel) are neither
// changed nor written.

// Orders this wave's LDS writes before its later LDS reads (no cross-wave sync).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kUpdLS = 144;  // LDS row stride of the update staging: a 128-byte row plus 16
                             // (16-byte aligned, at most 2-way conflicts for 4-byte access)

// One wave's 32 x 128 part (w4 = 0..3 within the four waves of the tile):
// rows row0 .. row0 + 31 across all of the tile's 128 columns, so that each
// row's 128-byte line is read and written whole, 32 bytes by each of four
// lanes (a line written in halves by two waves cost a line read each).
// The row pitch is a multiple of 64, so the tile's upper 64 columns may lie
// past it: their operands are zero and their lanes write nothing.
__device__ __forceinline__ void update_tile(int8_t* __restrict__ S, int n, int pitch, int K,
                                            const int* __restrict__ rowpos, const int8_t* __restrict__ GT,
                                            int j, int tx, int ty, int w4, int lane, uint8_t* st, int skip0,
                                            int skip1) {
    const int lr = lane & 15, lg = lane >> 4;
    const int col0 = tx * 128;                // the tile's 128 columns
    const int row0 = ty * 128 + 32 * w4;      // this wave's 32 rows
    const int colend = min(col0 + 128, pitch);
    if (col0 >= pitch || row0 >= n || (col0 >= skip0 && colend <= skip1)) return;  // wave-uniform
    const uint32_t q = c_pt.q[j];
    // |x| <= 32 * 125^2 + 125 < 2^19
    const float rq = 1.0f / (float)q;
    const int32_t nq = -(int32_t)q;
    int8_t* Sj = S + (size_t)j * n * pitch;
    const int* rpj = rowpos + (size_t)j * n;
    const int8_t* GTj = GT + (size_t)j * pitch * kPanel;
    // operands: lanes of group lg supply k in [16 lg, 16 lg + 16); only k < 32 is nonzero
    v4i_t ga[8], pb[2];
#pragma unroll
    for (int a = 0; a < 8; a++) {
        const int col = col0 + 16 * a + lr;
        ga[a] = (lg < 2 && col < pitch) ? *(const v4i_t*)(GTj + (size_t)col * kPanel + 16 * lg) : v4i_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int b = 0; b < 2; b++) {
        const int i = row0 + 16 * b + lr;
        pb[b] = (lg < 2 && i < n) ? *(const v4i_t*)(Sj + (size_t)i * pitch + K + 16 * lg) : v4i_t{0, 0, 0, 0};
    }
    // this lane's 32 columns col0 + 32 lg .. are written when they lie below
    // the pitch and outside the skipped range (both ends multiples of 32)
    const int mycol = col0 + 32 * lg;
    const bool wr = mycol < pitch && !(mycol >= skip0 && mycol < skip1);
    // old S for rows row0 + 16 b + lr, 32 columns per lane, and the rows'
    // pivot steps: every load of the tile is issued before the first use
    uint4 old32[2][2];
    int rp[2];
#pragma unroll
    for (int b = 0; b < 2; b++) {
        const int i = row0 + 16 * b + lr;
        const bool in = i < n && mycol < pitch;
        old32[b][0] = in ? *(const uint4*)(Sj + (size_t)i * pitch + mycol) : make_uint4(0, 0, 0, 0);
        old32[b][1] = in ? *(const uint4*)(Sj + (size_t)i * pitch + mycol + 16) : make_uint4(0, 0, 0, 0);
        rp[b] = i < n ? rpj[i] : 0;
    }
#pragma unroll
    for (int b = 0; b < 2; b++) {
        // through LDS into the accumulator layout
        const int i = row0 + 16 * b + lr;
        const bool rowok = i < n;
        *(uint4*)(st + lr * kUpdLS + 32 * lg) = old32[b][0];
        *(uint4*)(st + lr * kUpdLS + 32 * lg + 16) = old32[b][1];
        const bool pivot_row = rp[b] >= K && rp[b] < K + kPanel;
        wave_lds_sync();
        // accumulator layout: lane holds row lr, columns 16 a + 4 lg + 0..3
#pragma unroll
        for (int a = 0; a < 8; a++) {
            const v4i_t acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ga[a], pb[b], v4i_t{0, 0, 0, 0}, 0, 0, 0);
            const uint32_t old = *(const uint32_t*)(st + lr * kUpdLS + 16 * a + 4 * lg);
            uint32_t outw = 0;
            const uint32_t oldw = pivot_row ? 0u : old;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int x = (int)(int8_t)(oldw >> (8 * e)) + acc[e];
                outw |= ((uint32_t)bal_mod_19(x, rq, nq) & 0xffu) << (8 * e);
            }
            *(uint32_t*)(st + lr * kUpdLS + 16 * a + 4 * lg) = outw;
        }
        wave_lds_sync();
        if (rowok && wr) {
            *(uint4*)(Sj + (size_t)i * pitch + mycol) = *(const uint4*)(st + lr * kUpdLS + 32 * lg);
            *(uint4*)(Sj + (size_t)i * pitch + mycol + 16) = *(const uint4*)(st + lr * kUpdLS + 32 * lg + 16);
        }
        wave_lds_sync();
    }
}

// Which 128 x 128 tile the u-th update unit on XCD x takes.  Blocks are
// dealt to the eight XCDs round-robin by their index, and each XCD has its
// own L2; every column tile of a row tile reads the rows' panel bytes (32
// bytes of each row's 128-byte line), so all column tiles of a row tile go
// to one XCD: XCD x takes the row tiles x, x + 8, ... (a row tile is one
// prime's 128 rows), and only the transposed pivot rows GT (32 dense bytes a
// column) are read on every XCD.  Returns false past the last row tile.
__device__ __forceinline__ bool update_unit(int x, int u, int ntx, int nty, int* j, int* tx, int* ty) {
    const int r = x + 8 * (u / ntx);
    if (r >= nty * kNumPrimes) return false;
    *tx = u % ntx;
    *j = r / nty;
    *ty = r % nty;
    return true;
}

// Every column but the panel's [K, K + 32) (or the wider skipped range):
// one 128 x 128 tile per block, 8 ntx ceil(nty 53 / 8) blocks in a row,
// mapped to tiles by update_unit.
__global__ __launch_bounds__(256) void gj_update_kernel(int8_t* __restrict__ S, int n, int pitch, int K,
                                                        const int* __restrict__ rowpos,
                                                        const int* __restrict__ flags,
                                                        const int8_t* __restrict__ GT, int skip1, int ntx,
                                                        int nty) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][16 * kUpdLS];
    int j, tx, ty;
    if (!update_unit(blockIdx.x & 7, blockIdx.x >> 3, ntx, nty, &j, &tx, &ty) || flags[j]) return;
    const int wave = threadIdx.x >> 6;
    update_tile(S, n, pitch, K, rowpos, GT, j, tx, ty, wave, threadIdx.x & 63, stage[wave], K, skip1);
}

// Panel K on its own (no other work in flight), then its pivot rows to GT.
template <int RPT, bool UP>
__global__ __launch_bounds__(1024) void gj_panel_kernel(int8_t* __restrict__ S, int n, int pitch, int K,
                                                        int* __restrict__ piv, int* __restrict__ rowpos,
                                                        int* __restrict__ flags, int8_t* __restrict__ GT) {
    const int j = blockIdx.x;
    const bool ok = UP ? panel_up_body<RPT>(S, n, pitch, K, piv, rowpos, flags, j)
                       : panel_packed_body<RPT>(S, n, pitch, K, piv, rowpos, flags, j);
    if (!ok) return;  // the whole block
    __syncthreads();  // the pivot rows the panel wrote are visible to the block
    panel_gather_gt(S + (size_t)j * n * pitch, pitch, min(kPanel, n - K), piv + (size_t)j * (n + 1) + K,
                    GT + (size_t)j * pitch * kPanel, threadIdx.x);
}

// Start of panel K's block (lookahead form, K >= 32): the pivot rows of
// panel K - 32 in panel K's columns, which the gather-next launch left:
// S[p][K + col] = sum_c S[p][K - 32 + c] S[piv[K - 32 + c]][K + col] (mod q),
// the same sum the other rows got there.  The old 32 x 32 blocks are read
// into LDS before any is written.
__device__ __forceinline__ void finish_pivot_rows(int8_t* __restrict__ S, int n, int pitch, int K,
                                                  const int* __restrict__ piv, int j) {
    const int t = threadIdx.x;
    int8_t* Sj = S + (size_t)j * n * pitch;
    const int* pl = piv + (size_t)j * (n + 1) + K - kPanel;
    __shared__ __attribute__((aligned(16))) int8_t oldb[kPanel][kPanel];  // oldb[c][col] = S[pl[c]][K + col]
    __shared__ __attribute__((aligned(16))) int8_t mul[kPanel][kPanel];   // mul[r][c] = S[pl[r]][K - 32 + c]
    if (t < 2 * kPanel) {
        const int c = t >> 1, h = t & 1;
        *(uint4*)&oldb[c][16 * h] = *(const uint4*)(Sj + (size_t)pl[c] * pitch + K + 16 * h);
    } else if (t < 4 * kPanel) {
        const int r = (t - 2 * kPanel) >> 1, h = t & 1;
        *(uint4*)&mul[r][16 * h] = *(const uint4*)(Sj + (size_t)pl[r] * pitch + K - kPanel + 16 * h);
    }
    __syncthreads();
    if (t < kPanel * kPanel) {
        const int r = t >> 5, col = t & 31;
        int acc = 0;
#pragma unroll
        for (int c = 0; c < kPanel; c++) acc += (int)mul[r][c] * (int)oldb[c][col];
        const uint32_t q = c_pt.q[j];  // |acc| <= 32 * 125^2 < 2^19
        Sj[(size_t)pl[r] * pitch + K + col] = (int8_t)bal_mod_19(acc, 1.0f / (float)q, -(int32_t)q);
    }
    __syncthreads();
}

// Lookahead form: panel K (blocks 0 .. 52, one per prime) and, in the same
// launch, the update of panel K - 32 on every column outside
// [K - 32, K + 32) (the blocks after them, four 128 x 128 tiles each).  The
// two touch disjoint columns; panel K's columns were updated beforehand by
// gj_gather_next_kernel.  The panel blocks come first, so they are placed
// first.  K >= n: the update part only.
template <int RPT, bool UP>
__global__ __launch_bounds__(1024) void gj_panel_rest_kernel(int8_t* __restrict__ S, int n, int pitch, int K,
                                                             int* __restrict__ piv, int* __restrict__ rowpos,
                                                             int* __restrict__ flags, const int8_t* __restrict__ GT,
                                                             int ntx, int nty, int* __restrict__ wq) {
    const int np = K < n ? kNumPrimes : 0;
    if ((int)blockIdx.x < np) {
        if (K >= kPanel && !flags[blockIdx.x]) finish_pivot_rows(S, n, pitch, K, piv, blockIdx.x);
        if (UP) (void)panel_up_body<RPT>(S, n, pitch, K, piv, rowpos, flags, blockIdx.x);
        else (void)panel_packed_body<RPT>(S, n, pitch, K, piv, rowpos, flags, blockIdx.x);
        // then the panel's block joins the update below
    }
    if (K < kPanel) return;  // no earlier panel to update
    // The update of panel K - 32: each block takes four units at a time
    // from its XCD's queue (blocks are dealt to the eight XCDs round-robin by
    // index, and update_unit gives each XCD whole row tiles) until the queue
    // is empty, so the CUs that ran a panel take the update's tail too.  The
    // counters start at zero (set before the elimination); every round takes
    // four more, so the loop ends.
    __shared__ __attribute__((aligned(16))) uint8_t stage[16][16 * kUpdLS];
    __shared__ int s_base;
    const int wave = threadIdx.x >> 6;
    const int x = (int)blockIdx.x & 7;
    const int units = ntx * ((nty * kNumPrimes - x + 7) / 8);  // this XCD's units
    int* qx = wq + (size_t)(K / kPanel) * 8 + x;
    const int Kr = K - kPanel;
    for (;;) {
        __syncthreads();  // everyone has read the previous round's base
        if (threadIdx.x == 0) s_base = atomicAdd(qx, 4);
        __syncthreads();
        const int base = s_base;
        if (base >= units) break;
        int j, tx, ty;
        if (update_unit(x, base + (wave >> 2), ntx, nty, &j, &tx, &ty) && !flags[j])
            update_tile(S, n, pitch, Kr, rowpos, GT, j, tx, ty, wave & 3, threadIdx.x & 63, stage[wave], Kr,
                        Kr + 2 * kPanel);
    }
}

// After panel K: its pivot rows to GT, 256 columns per block (grid
// (column chunks, primes)), with no LDS: thread t takes columns
// c0 + 4 (t mod 64) .. + 3 of the pivot rows 8 (t / 64) .. + 7 (each wave's
// loads cover 256 contiguous bytes of a row); the block's four waves fill
// the 32-byte GT rows of its columns.
__device__ __forceinline__ void gather_gt_block(const int8_t* __restrict__ S, int n, int pitch, int K,
                                                const int* __restrict__ piv, int8_t* __restrict__ GT, int j,
                                                int bx) {
    const int t = threadIdx.x;
    const int col = bx * 256 + 4 * (t & 63);
    if (col >= pitch) return;  // the pitch is a multiple of 64: col + 3 < pitch otherwise
    gt_slice(S + (size_t)j * n * pitch, pitch, min(kPanel, n - K), piv + (size_t)j * (n + 1) + K,
             GT + (size_t)j * pitch * kPanel, col, 8 * (t >> 6));
}

// Then, when K + 32 < n, the update of the next panel's columns
// [K + 32, K + 64) on every row: 64 rows per block, one 16-row tile per
// wave, two 16-column halves.  The panel's pivot rows in those columns (a
// 32 x 32 byte block) come straight from S through LDS, so this part does
// not wait for GT and shares a launch with the gather.
__device__ __forceinline__ void next_cols_block(int8_t* __restrict__ S, int n, int pitch, int K,
                                                const int* __restrict__ piv, const int* __restrict__ rowpos,
                                                int j, int bx) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    int8_t* Sj = S + (size_t)j * n * pitch;
    const uint32_t q = c_pt.q[j];  // |x| <= 32 * 125^2 + 125 < 2^19 below
    const float rq = 1.0f / (float)q;
    const int32_t nq = -(int32_t)q;
    const int* rpj = rowpos + (size_t)j * n;
    const int c0 = K + kPanel;
    __shared__ __attribute__((aligned(16))) int8_t prs[kPanel][kPanel];  // prs[c][col] = S[piv[K + c]][c0 + col]
    if (t < 2 * kPanel) {
        const int c = t >> 1, h = t & 1;
        const int pr = piv[(size_t)j * (n + 1) + K + c];
        *(uint4*)&prs[c][16 * h] = *(const uint4*)(Sj + (size_t)pr * pitch + c0 + 16 * h);
    }
    __syncthreads();
    v4i_t ga[2];
#pragma unroll
    for (int a = 0; a < 2; a++) {
        uint32_t w[4] = {0, 0, 0, 0};
        if (lg < 2) {
#pragma unroll
            for (int e = 0; e < 16; e++) w[e >> 2] |= (uint32_t)(uint8_t)prs[16 * lg + e][16 * a + lr] << (8 * (e & 3));
        }
        ga[a] = v4i_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
    const int i = bx * 64 + 16 * wave + lr;
    const bool rowok = i < n;
    const v4i_t pb = (lg < 2 && rowok) ? *(const v4i_t*)(Sj + (size_t)i * pitch + K + 16 * lg) : v4i_t{0, 0, 0, 0};
    const int rp = rowok ? rpj[i] : 0;
    const bool pivot_row = rp >= K && rp < K + kPanel;
#pragma unroll
    for (int a = 0; a < 2; a++) {
        const v4i_t acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ga[a], pb, v4i_t{0, 0, 0, 0}, 0, 0, 0);
        const int col = c0 + 16 * a + 4 * lg;
        const uint32_t old = rowok ? *(const uint32_t*)(Sj + (size_t)i * pitch + col) : 0u;
        uint32_t outw = 0;
        const uint32_t oldw = pivot_row ? 0u : old;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int x = (int)(int8_t)(oldw >> (8 * e)) + acc[e];
            outw |= ((uint32_t)bal_mod_19(x, rq, nq) & 0xffu) << (8 * e);
        }
        // the panel's own pivot rows are read by every block of this launch
        // (prs): the next panel's block updates them (finish_pivot_rows)
        if (rowok && !pivot_row) *(uint32_t*)(Sj + (size_t)i * pitch + col) = outw;
    }
}

// After panel K: blocks [0, G) gather its pivot rows into GT (for the next
// update), blocks [G, G + N) update the next panel's columns (N = 0 on the
// last panel); grid (G + N, primes).
__global__ __launch_bounds__(256) void gj_gather_next_kernel(int8_t* __restrict__ S, int n, int pitch, int K,
                                                             const int* __restrict__ piv,
                                                             const int* __restrict__ rowpos,
                                                             const int* __restrict__ flags, int8_t* __restrict__ GT,
                                                             int G) {
    const int j = blockIdx.y;
    if (flags[j]) return;
    if ((int)blockIdx.x < G) gather_gt_block(S, n, pitch, K, piv, GT, j, blockIdx.x);
    else next_cols_block(S, n, pitch, K, piv, rowpos, j, blockIdx.x - G);
}

bool blocked_inverse_fits(const Layout& L) { return L.n <= 4096 && (L.pitch % 64) == 0; }

// the panel variant for panel K: unpacked for full panels of up to 2048 rows
// (one or two rows a thread), byte-packed otherwise
static int panel_kind(const Layout& L, int K) {
    const bool full = L.n - K >= kPanel;
    if (L.n <= 1024) return full ? 0 : 1;
    if (L.n <= 2048) return full ? 5 : 2;
    return 4;
}

hipError_t launch_gj_panel(const Layout& L, uint8_t* ws, int K, hipStream_t st) {
    int8_t* S = (int8_t*)(ws + L.off_S);
    int* piv = (int*)(ws + L.off_piv);
    int* rowpos = (int*)(ws + L.off_rowpos);
    int* flags = (int*)(ws + L.off_flags);
    int8_t* GT = (int8_t*)(ws + L.off_GT);
    const dim3 g(kNumPrimes), b(1024);
    switch (panel_kind(L, K)) {
        case 0: es_launch((gj_panel_kernel<1, true>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT); break;
        case 1: es_launch((gj_panel_kernel<1, false>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT); break;
        case 2: es_launch((gj_panel_kernel<2, false>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT); break;
        case 5: es_launch((gj_panel_kernel<2, true>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT); break;
        default: es_launch((gj_panel_kernel<4, false>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT); break;
    }
    return hipGetLastError();
}

hipError_t launch_gj_update(const Layout& L, uint8_t* ws, int K, hipStream_t st) {
    const int ntx = (L.pitch + 127) / 128, nty = (L.n + 127) / 128;
    const int per_xcd = ntx * ((nty * kNumPrimes + 7) / 8);  // units (tiles) per XCD
    es_launch(gj_update_kernel, dim3(8 * per_xcd), dim3(256), 0, st, (int8_t*)(ws + L.off_S), L.n, L.pitch, K,
              (const int*)(ws + L.off_rowpos), (const int*)(ws + L.off_flags), (const int8_t*)(ws + L.off_GT),
              K + kPanel, ntx, nty);
    return hipGetLastError();
}

hipError_t launch_gj_panel_rest(const Layout& L, uint8_t* ws, int K, hipStream_t st) {
    int8_t* S = (int8_t*)(ws + L.off_S);
    int* piv = (int*)(ws + L.off_piv);
    int* rowpos = (int*)(ws + L.off_rowpos);
    int* flags = (int*)(ws + L.off_flags);
    const int8_t* GT = (const int8_t*)(ws + L.off_GT);
    const int ntx = (L.pitch + 127) / 128, nty = (L.n + 127) / 128;
    int* wq = (int*)(ws + L.off_wq);
    if (K / kPanel >= work_queue_rows(L.n)) return hipErrorInvalidValue;
    // one 1024-thread block per CU: the update blocks fill the CUs the panel
    // blocks leave (a multiple of 8, so every XCD gets its share); they and
    // the panel blocks drain the per-XCD queues
    const int np = K < L.n ? kNumPrimes : 0;
    const int nupd = K >= kPanel ? std::max(8, (device_cu_count() - np + 7) / 8 * 8) : 0;
    const dim3 g(np + nupd), b(1024);
    if (np + nupd == 0) return hipSuccess;
    switch (K < L.n ? panel_kind(L, K) : 1) {
        case 0: es_launch((gj_panel_rest_kernel<1, true>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT, ntx, nty, wq); break;
        case 1: es_launch((gj_panel_rest_kernel<1, false>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT, ntx, nty, wq); break;
        case 2: es_launch((gj_panel_rest_kernel<2, false>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT, ntx, nty, wq); break;
        case 5: es_launch((gj_panel_rest_kernel<2, true>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT, ntx, nty, wq); break;
        default: es_launch((gj_panel_rest_kernel<4, false>), g, b, 0, st, S, L.n, L.pitch, K, piv, rowpos, flags, GT, ntx, nty, wq); break;
    }
    return hipGetLastError();
}

hipError_t launch_gj_gather_next(const Layout& L, uint8_t* ws, int K, hipStream_t st) {
    const int G = (L.pitch + 255) / 256, N = K + kPanel < L.n ? (L.n + 63) / 64 : 0;
    es_launch(gj_gather_next_kernel, dim3(G + N, kNumPrimes), dim3(256), 0, st, (int8_t*)(ws + L.off_S), L.n,
              L.pitch, K, (const int*)(ws + L.off_piv), (const int*)(ws + L.off_rowpos),
              (const int*)(ws + L.off_flags), (int8_t*)(ws + L.off_GT), G);
    return hipGetLastError();
}

// B[j][k][col] = A^-1 mod q_j (balanced int8): row piv[j][k] of S, slot rowpos[j][col]
__global__ __launch_bounds__(256) void export_inverse_kernel(const int8_t* __restrict__ S, int n, int pitch,
                                                             const int* __restrict__ piv,
                                                             const int* __restrict__ rowpos,
                                                             const int* __restrict__ flags,
                                                             int8_t* __restrict__ B) {
    const int k = blockIdx.x, j = blockIdx.y;
    if (flags[j]) return;
    const int p = piv[(size_t)j * (n + 1) + k];
    const int8_t* src = S + ((size_t)j * n + p) * pitch;
    const int* rp = rowpos + (size_t)j * n;
    int8_t* dst = B + ((size_t)j * n + k) * n;
    for (int col = threadIdx.x; col < n; col += 256) dst[col] = src[rp[col]];
}

hipError_t launch_export_inverse(const Layout& L, const uint8_t* ws, int8_t* B, hipStream_t st) {
    es_launch(export_inverse_kernel, dim3(L.n, kNumPrimes), dim3(256), 0, st,
                       (const int8_t*)(ws + L.off_S), L.n, L.pitch, (const int*)(ws + L.off_piv),
                       (const int*)(ws + L.off_rowpos), (const int*)(ws + L.off_flags), B);
    return hipGetLastError();
}

// ---------------------------------------------------------------- lift: contraction
// y_j = B_j rho_j for every live prime, int8 x int8 -> int32 with the 4-way
// dot product (v_dot4_i32_i8); u_j = y_j mod q_j is scattered to component
// order through rowpos.  Grid (row tiles, live primes); a lane covers 16
// columns of a row and CT right-hand sides at once.
template <int LPR, int RI, int CT>
__global__ __launch_bounds__(256) void lift_gemv_kernel(const int8_t* __restrict__ S, int n, int pitch,
                                                        int c, const int8_t* __restrict__ rho,
                                                        const LiftParams* __restrict__ prm,
                                                        const int* __restrict__ rowpos,
                                                        uint8_t* __restrict__ U) {
    constexpr int RPW = 64 / LPR;
    constexpr int ROWS = 4 * RPW * RI;
    const int jl = blockIdx.y;
    const int J = prm->qidx[jl];
    const uint32_t q = prm->q[jl], mu32 = prm->mu32[jl];
    const int8_t* Sj = S + (size_t)J * n * pitch;
    const int8_t* rj = rho + (size_t)jl * c * pitch;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, cl = lane % LPR;
    const int npass = (LPR == 64) ? (pitch + 1023) >> 10 : 1;
    const int row0 = blockIdx.x * ROWS;
    const size_t NC = (size_t)n * c;

    for (int t0 = 0; t0 < c; t0 += CT) {
        int acc[RI][CT];
#pragma unroll
        for (int r = 0; r < RI; r++)
#pragma unroll
            for (int t = 0; t < CT; t++) acc[r][t] = 0;
        for (int pass = 0; pass < npass; ++pass) {
            const int col0 = pass * 1024 + cl * 16;
            const bool active = col0 < pitch;
            uint4 rv[CT];
#pragma unroll
            for (int t = 0; t < CT; t++)
                rv[t] = (active && t0 + t < c) ? *(const uint4*)(rj + (size_t)(t0 + t) * pitch + col0)
                                               : make_uint4(0, 0, 0, 0);
            uint4 s[RI];
#pragma unroll
            for (int r = 0; r < RI; r++) {
                const int i = row0 + wave * RPW + g + r * 4 * RPW;
                s[r] = (active && i < n) ? *(const uint4*)(Sj + (size_t)i * pitch + col0)
                                         : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < RI; r++)
#pragma unroll
                for (int t = 0; t < CT; t++) {
                    int a = acc[r][t];
                    a = __builtin_amdgcn_sdot4((int)s[r].x, (int)rv[t].x, a, false);
                    a = __builtin_amdgcn_sdot4((int)s[r].y, (int)rv[t].y, a, false);
                    a = __builtin_amdgcn_sdot4((int)s[r].z, (int)rv[t].z, a, false);
                    a = __builtin_amdgcn_sdot4((int)s[r].w, (int)rv[t].w, a, false);
                    acc[r][t] = a;
                }
        }
        {
#pragma unroll
            for (int r = 0; r < RI; r++)
#pragma unroll
                for (int t = 0; t < CT; t++)
#pragma unroll
                    for (int off = LPR / 2; off > 0; off >>= 1) acc[r][t] += __shfl_xor(acc[r][t], off);
            if (cl == 0) {
#pragma unroll
                for (int r = 0; r < RI; r++) {
                    const int i = row0 + wave * RPW + g + r * 4 * RPW;
                    if (i >= n) continue;
                    const size_t kdst = (size_t)rowpos[(size_t)J * n + i] * c;
#pragma unroll
                    for (int t = 0; t < CT; t++)
                        if (t0 + t < c)
                            U[(size_t)jl * NC + kdst + t0 + t] = (uint8_t)mod_i32(acc[r][t], q, mu32);
                }
            }
        }
    }
}

// Exchange with a partner lane whose bit BIT differs (a fixed permutation of
// the wave): data-parallel-primitive moves within a row of 16 lanes, LDS
// permutes across rows.  Any such pairing serves a butterfly sum.
template <int BIT>
__device__ __forceinline__ int xchg_bit(int v, int lane) {
    if constexpr (BIT >= 16) return __builtin_amdgcn_ds_bpermute((lane ^ BIT) << 2, v);
    else if constexpr (BIT == 8) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);  // row_mirror
    else if constexpr (BIT == 4) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);  // row_half_mirror
    else if constexpr (BIT == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false);   // quad [2,3,0,1]
    else return __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false);                            // quad [1,0,3,2]
}

// One butterfly level at lane bit BIT over the first 2 * HALF entries of v:
// keep the half picked by this lane's bit, add the partner's matching half.
template <int BIT, int HALF, int N>
__device__ __forceinline__ void split_level(int (&v)[N], int lane) {
    const bool hi = (lane & BIT) != 0;
#pragma unroll
    for (int u = 0; u < HALF; u++) {
        const int send = hi ? v[u] : v[u + HALF];
        const int keep = hi ? v[u + HALF] : v[u];
        v[u] = keep + xchg_bit<BIT>(send, lane);
    }
}

// Transposed butterfly sum of RI per-lane row sums (RI in {8, 16}) over the
// 64 lanes: the first log2(RI) levels split the rows between partner lanes,
// the rest are plain sums.  Afterwards v[0] of every lane holds the total of
// row (lane >> (6 - log2 RI)) & (RI - 1); 6 + RI - 1 - log2(RI) exchanges
// replace 6 RI.
template <int RI>
__device__ __forceinline__ void wave_sum_rows(int (&v)[RI], int lane) {
    static_assert(RI == 8 || RI == 16, "row count");
    split_level<32, RI / 2>(v, lane);
    split_level<16, RI / 4>(v, lane);
    split_level<8, RI / 8>(v, lane);
    if constexpr (RI == 16) split_level<4, 1>(v, lane);
    else v[0] += xchg_bit<4>(v[0], lane);
    v[0] += xchg_bit<2>(v[0], lane);
    v[0] += xchg_bit<1>(v[0], lane);
}

// y_j = B_j rho_j for one right-hand side when rows span at least 1 KB
// (pitch >= 1024): each load instruction of a wave covers 1 KB of one row,
// a wave owns RI consecutive rows, and the sums meet in a transposed
// butterfly.  Loads are unconditional: rows past n re-read row n - 1 and
// lanes past the pitch re-read the pass's first column, and both results
// are discarded, so the loop has no branches.
template <int RI>
__global__ __launch_bounds__(256) void lift_gemv1_kernel(const int8_t* __restrict__ S, int n, int pitch,
                                                         const int8_t* __restrict__ rho,
                                                         const LiftParams* __restrict__ prm,
                                                         const int* __restrict__ rowpos,
                                                         uint8_t* __restrict__ U) {
    const int jl = blockIdx.y;
    const int J = prm->qidx[jl];
    const uint32_t q = prm->q[jl], mu32 = prm->mu32[jl];
    const int8_t* Sj = S + (size_t)J * n * pitch;
    const int8_t* rj = rho + (size_t)jl * pitch;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = (blockIdx.x * 4 + wave) * RI;
    const int8_t* rowp[RI];
#pragma unroll
    for (int r = 0; r < RI; r++) rowp[r] = Sj + (size_t)min(rbase + r, n - 1) * pitch;
    int acc[RI];
#pragma unroll
    for (int r = 0; r < RI; r++) acc[r] = 0;
    for (int col0 = 0; col0 < pitch; col0 += 1024) {
        const int col = col0 + lane * 16;
        const bool cin = col < pitch;
        const int colc = cin ? col : col0;
        uint4 rv = *(const uint4*)(rj + colc);
        if (!cin) rv = make_uint4(0, 0, 0, 0);
        uint4 s[RI];
#pragma unroll
        for (int r = 0; r < RI; r++) s[r] = *(const uint4*)(rowp[r] + colc);
#pragma unroll
        for (int r = 0; r < RI; r++) {
            int a = acc[r];
            a = __builtin_amdgcn_sdot4((int)s[r].x, (int)rv.x, a, false);
            a = __builtin_amdgcn_sdot4((int)s[r].y, (int)rv.y, a, false);
            a = __builtin_amdgcn_sdot4((int)s[r].z, (int)rv.z, a, false);
            a = __builtin_amdgcn_sdot4((int)s[r].w, (int)rv.w, a, false);
            acc[r] = a;
        }
    }
    wave_sum_rows<RI>(acc, lane);
    constexpr int LOG_RI = RI == 16 ? 4 : 3;
    if ((lane & ((64 / RI) - 1)) == 0) {
        const int i = rbase + ((lane >> (6 - LOG_RI)) & (RI - 1));
        if (i < n) U[(size_t)jl * n + (size_t)rowpos[(size_t)J * n + i]] = (uint8_t)mod_i32(acc[0], q, mu32);
    }
}

// ---------------------------------------------------------------- lift: MFMA contraction (c > 1)
// For several right-hand sides the per-prime product Y_j = B_j R_j is a real
// int8 GEMM (n x n by n x c), run on v_mfma_i32_16x16x64_i8.  A wave owns 32
// storage rows (two 16-row tiles) and 16 right-hand sides; B_j streams from
// HBM once, the block's 16 residue columns (R_j transposed, [t][k]) sit in
// LDS for the whole K range.  Operand lanes: lane l feeds row (or column)
// l % 16 with 16 bytes of k; lane group g = l / 16 and register quad u cover
// k in [kc + 64 u + 16 g, +16), the same for both operands, so every k of a
// 256-byte block is summed exactly once.  Output lane l holds column l % 16,
// rows 4 (l / 16) + 0..3 of each 16 x 16 tile.
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMfmaRowsPerWave = 32;
constexpr int kMfmaKSeg = 2048;          // k bytes staged in LDS at a time
constexpr int kMfmaLdsStride = kMfmaKSeg + 16;

__global__ __launch_bounds__(256) void lift_mfma_kernel(const int8_t* __restrict__ S, int n, int pitch, int c,
                                                        const int8_t* __restrict__ rho,
                                                        const LiftParams* __restrict__ prm,
                                                        const int* __restrict__ rowpos,
                                                        uint8_t* __restrict__ U) {
    __shared__ __attribute__((aligned(16))) int8_t Bs[16 * kMfmaLdsStride];
    const int jl = blockIdx.y;
    const int t0 = blockIdx.z * 16;
    const int J = prm->qidx[jl];
    const uint32_t q = prm->q[jl], mu32 = prm->mu32[jl];
    const int8_t* Sj = S + (size_t)J * n * pitch;
    const int8_t* rj = rho + (size_t)jl * c * pitch;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int wrow0 = blockIdx.x * (4 * kMfmaRowsPerWave) + wave * kMfmaRowsPerWave;
    const int ra = wrow0 + lr, rb = wrow0 + 16 + lr;     // this lane's A rows
    const bool okA = ra < n, okB = rb < n;
    v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};

    for (int seg = 0; seg < pitch; seg += kMfmaKSeg) {
        const int seglen = min(kMfmaKSeg, pitch - seg);
        __syncthreads();  // previous segment's readers are done
        // stage R^T[t0 .. t0+15][seg .. seg+seglen) (zero beyond c)
        for (int idx = threadIdx.x; idx < 16 * (seglen / 16); idx += 256) {
            const int t = idx / (seglen / 16), off = (idx % (seglen / 16)) * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t0 + t < c) v = *(const uint4*)(rj + (size_t)(t0 + t) * pitch + seg + off);
            *(uint4*)(Bs + t * kMfmaLdsStride + off) = v;
        }
        __syncthreads();
        for (int kc = 0; kc < seglen; kc += 256) {
            v4i a0[4], a1[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int ko = kc + 64 * u + 16 * lg;
                const bool in = ko < seglen;
                a0[u] = (okA && in) ? *(const v4i*)(Sj + (size_t)ra * pitch + seg + ko) : v4i{0, 0, 0, 0};
                a1[u] = (okB && in) ? *(const v4i*)(Sj + (size_t)rb * pitch + seg + ko) : v4i{0, 0, 0, 0};
                b[u] = in ? *(const v4i*)(Bs + lr * kMfmaLdsStride + ko) : v4i{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                if (kc + 64 * u < seglen) {
                    acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[u], b[u], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[u], b[u], acc1, 0, 0, 0);
                }
            }
        }
    }
    // epilogue: lane holds column t0 + lr, rows 4 lg + 0..3 of each tile
    const int t = t0 + lr;
    if (t >= c) return;
    const size_t NC = (size_t)n * c;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int i0 = wrow0 + 4 * lg + r, i1 = wrow0 + 16 + 4 * lg + r;
        if (i0 < n)
            U[(size_t)jl * NC + (size_t)rowpos[(size_t)J * n + i0] * c + t] = (uint8_t)mod_i32(acc0[r], q, mu32);
        if (i1 < n)
            U[(size_t)jl * NC + (size_t)rowpos[(size_t)J * n + i1] * c + t] = (uint8_t)mod_i32(acc1[r], q, mu32);
    }
}

// ---------------------------------------------------------------- lift: CRT
// The balanced digit x (|x| <= (P - 1) / 2, x = r_l mod q_l for every live
// prime) by the Chinese remainder formula with balanced coefficients:
//   X = sum_l u_l W_l,  W_l = P / q_l,  u_l = (r_l c_l mod q_l) in (-q_l/2, q_l/2),
//   c_l = W_l^-1 mod q_l,  so X = x (mod P) and |X| < E P / 2;
//   x = X - k P with k = round(X / P) = round(sum_l u_l / q_l).
// Sixteen lanes per component, lane s taking the primes l = s mod 16; word w
// of X accumulates sum_l u_l W_l[w] in double precision, exact (each term is
// below 2^39 in magnitude, every partial sum below 2^45), and the sixteen
// partial sums are added across the lanes.  k comes from the double sum
// of u_l / q_l, whose error (about E 2^-54) can only matter when X / P is
// within it of a half-integer; there an exact comparison with (P - 1) / 2
// settles the representative.  x mod 2^64 is kept for the residual.

// v + (v from a partner lane), for a double: X = 1, 2 pair lanes l ^ 1,
// l ^ 2 in each quad; X = 4 pairs l with 7 - l in each eight lanes and
// X = 8 pairs l with 15 - l in each sixteen.  After the levels below X every
// lane holds the sum of its aligned group of X, so each level doubles it.
template <int X>
__device__ __forceinline__ double quad_add(double v) {
    // quad_perm [1,0,3,2] / [2,3,0,1] / row_half_mirror / row_mirror
    constexpr int ctrl = X == 1 ? 0xb1 : X == 2 ? 0x4e : X == 4 ? 0x141 : 0x140;
    const uint64_t b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, ctrl, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), ctrl, 0xf, 0xf, false);
    return v + __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// the CRT constants of the live primes, staged in LDS
struct CrtTables {
    double Wd[kNumPrimes][kDigitWords];
    double qrec[kNumPrimes];
    uint32_t qc[kNumPrimes][4];  // q, mu16, c, mu32
};

__device__ __forceinline__ void load_crt_tables(CrtTables& T, const LiftParams* __restrict__ prm, int tid,
                                                int nthreads) {
    for (int i = tid; i < kNumPrimes * kDigitWords; i += nthreads) (&T.Wd[0][0])[i] = (&prm->Wd[0][0])[i];
    for (int l = tid; l < kNumPrimes; l += nthreads) {
        T.qrec[l] = prm->qrec[l];
        T.qc[l][0] = prm->q[l];
        T.qc[l][1] = prm->mu16[l];
        T.qc[l][2] = prm->cinv[l];
        T.qc[l][3] = prm->mu32[l];
    }
}

// x = X - k P as twelve 32-bit words (two's complement), X given by its
// exact word sums acc[w] (X = sum_w acc[w] 2^(32 w))
__device__ __forceinline__ void crt_sub_kP(const double (&acc)[kDigitWords], int64_t ki,
                                           const LiftParams* __restrict__ prm, uint32_t (&x)[kDigitWords]) {
    int64_t carry = 0;
#pragma unroll
    for (int w = 0; w < kDigitWords; w++) {
        const int64_t v = (int64_t)acc[w] - ki * (int64_t)prm->Pw[w] + carry;
        x[w] = (uint32_t)v;
        carry = v >> 32;
    }
}

// k = round(X / P) from f = sum_l u_l / q_l, and x = X - k P.  When f lies
// within 2^-30 of a half-integer the representative is settled by an exact
// comparison of x with (P - 1) / 2, and k moves by one with it.
__device__ __forceinline__ int64_t crt_finish(const double (&acc)[kDigitWords], double f,
                                              const LiftParams* __restrict__ prm, uint32_t (&x)[kDigitWords]) {
    int64_t ki = (int64_t)rint(f);
    crt_sub_kP(acc, ki, prm, x);
    if (fabs(f - (double)ki) > 0.5 - 0x1p-30) {
        // neg: is x + (P - 1) / 2 negative?  else: is x - (P - 1) / 2 positive?
        const bool neg = (int32_t)x[kDigitWords - 1] < 0;
        int64_t c = 0;
        uint32_t y[kDigitWords];
#pragma unroll
        for (int w = 0; w < kDigitWords; w++) {
            const int64_t v = (int64_t)x[w] + (neg ? (int64_t)prm->Phw[w] : -(int64_t)prm->Phw[w]) + c;
            y[w] = (uint32_t)v;
            c = v >> 32;
        }
        bool nz = false;
#pragma unroll
        for (int w = 0; w < kDigitWords; w++) nz |= y[w] != 0u;
        const bool out = neg ? (int32_t)y[kDigitWords - 1] < 0 : ((int32_t)y[kDigitWords - 1] >= 0 && nz);
        if (out) {
            ki += neg ? -1 : 1;
            c = 0;
#pragma unroll
            for (int w = 0; w < kDigitWords; w++) {
                const int64_t v = (int64_t)x[w] + (neg ? (int64_t)prm->Pw[w] : -(int64_t)prm->Pw[w]) + c;
                x[w] = (uint32_t)v;
                c = v >> 32;
            }
        }
    }
    return ki;
}

constexpr int kCrtLanes = 16;                                          // lanes per component
constexpr int kCrtPrimesPerLane = (kNumPrimes + kCrtLanes - 1) / kCrtLanes;

// The digit of one component from its residues: lane s of the component's
// sixteen holds res[i] = r_l for l = s + 16 i (l < E).  Writes the digit
// (twelve words) into slot `slot` of the component's chunk and x mod 2^64.
__device__ __forceinline__ uint64_t crt_digit(const CrtTables& T, const LiftParams* __restrict__ prm, int E, int s,
                                          const uint32_t (&res)[kCrtPrimesPerLane], int comp,
                                          uint64_t* __restrict__ digits, int kchunk, int slot,
                                          uint64_t* __restrict__ xlow) {
    double acc[kDigitWords];
#pragma unroll
    for (int w = 0; w < kDigitWords; w++) acc[w] = 0.0;
    double f = 0.0;
#pragma unroll
    for (int i = 0; i < kCrtPrimesPerLane; i++) {
        const int l = s + kCrtLanes * i;
        if (l >= E) continue;
        const uint32_t q = T.qc[l][0];
        const uint32_t u = red16(res[i] * T.qc[l][2], q, T.qc[l][1]);
        const double ud = (double)(u > (q >> 1) ? (int)u - (int)q : (int)u);
        f = fma(ud, T.qrec[l], f);
#pragma unroll
        for (int w = 0; w < kDigitWords; w++) acc[w] = fma(ud, T.Wd[l][w], acc[w]);
    }
    f = quad_add<8>(quad_add<4>(quad_add<2>(quad_add<1>(f))));
#pragma unroll
    for (int w = 0; w < kDigitWords; w++) acc[w] = quad_add<8>(quad_add<4>(quad_add<2>(quad_add<1>(acc[w]))));
    if (s != 0) return 0;
    uint32_t x[kDigitWords];
    (void)crt_finish(acc, f, prm, x);
    uint4* dst = (uint4*)(digits + ((size_t)comp * kchunk + slot) * kDigitLimbs);
    dst[0] = make_uint4(x[0], x[1], x[2], x[3]);
    dst[1] = make_uint4(x[4], x[5], x[6], x[7]);
    dst[2] = make_uint4(x[8], x[9], x[10], x[11]);
    const uint64_t xl = ((uint64_t)x[1] << 32) | x[0];
    xlow[comp] = xl;
    return xl;
}

// With xp set (c right-hand sides, rows of `pitch` bytes), x mod 2^64 of
// component k c + t also goes out as eight balanced bytes, byte b to
// xp[(b c + t) pitch + k] (x = sum_b byte_b 256^b mod 2^64), the operand of
// the MFMA residual.
__global__ __launch_bounds__(256) void crt_kernel(const LiftParams* __restrict__ prm, const uint8_t* __restrict__ U,
                                                  int NC, uint64_t* __restrict__ digits, int kchunk, int slot,
                                                  uint64_t* __restrict__ xlow, int8_t* __restrict__ xp, int c,
                                                  int pitch) {
    __shared__ CrtTables T;
    const int E = prm->E;
    load_crt_tables(T, prm, threadIdx.x, 256);
    __syncthreads();
    const int s = threadIdx.x & (kCrtLanes - 1);
    const int comp = blockIdx.x * (256 / kCrtLanes) + threadIdx.x / kCrtLanes;
    if (comp >= NC) return;  // the component's sixteen lanes leave together
    uint32_t res[kCrtPrimesPerLane];
#pragma unroll
    for (int i = 0; i < kCrtPrimesPerLane; i++) {
        const int l = s + kCrtLanes * i;
        res[i] = l < E ? U[(size_t)l * NC + comp] : 0u;
    }
    uint64_t v = crt_digit(T, prm, E, s, res, comp, digits, kchunk, slot, xlow);
    if (xp == nullptr || s != 0) return;
    const int k = comp / c, t = comp % c;
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const int8_t d = (int8_t)(v & 0xffu);  // balanced: the low byte read as signed
        xp[(size_t)(b * c + t) * pitch + k] = d;
        v = (v - (uint64_t)(int64_t)d) >> 8;
    }
}

// ---------------------------------------------------------------- lift: contraction + CRT, one right-hand side
// For one right-hand side with rows of at least 1 KB, the contraction and
// the step's share of the CRT share a launch: a block owns kFusedComps
// consecutive components and forms every live prime's residue for them, so
// the residues stay in LDS and the CRT's step share (k and x mod 2^64, the
// only part the next step needs) follows in the same block; the digits are
// formed later from the stored (u_l, k) records.  The live primes' B_j rows
// are copied once per lift into component order (row k of Sperm_j is the
// row of S_j that pivoted at step k), so a block reads 4 KB runs and the
// grid sweeps every matrix front to back.  The block's rows (prime,
// component) go eight to a wave as in the plain contraction (the sums meet
// in the same transposed butterfly).

// Sperm[jl][rowpos[J][i]] = S[J][i]: one wave per row, 1 KB per load
__global__ __launch_bounds__(256) void lift_rows_kernel(const int8_t* __restrict__ S, const int* __restrict__ rowpos,
                                                        const LiftParams* __restrict__ prm, int n, int pitch,
                                                        int8_t* __restrict__ Sperm) {
    const int jl = blockIdx.y;
    const int J = prm->qidx[jl];
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (i >= n) return;
    const int k = min((unsigned)rowpos[(size_t)J * n + i], (unsigned)(n - 1));  // a permutation; clamped all the same
    const int8_t* src = S + ((size_t)J * n + i) * pitch;
    int8_t* dst = Sperm + ((size_t)jl * n + k) * pitch;
    for (int col = lane * 16; col < pitch; col += 1024) *(uint4*)(dst + col) = *(const uint4*)(src + col);
}

// The block has ceil(batches / 2) waves (batch: eight rows), each holding
// two batches' loads in flight at once; at least kFusedMinThreads threads so
// that every CRT constant has a thread to fetch it.
constexpr int kFusedComps = 4, kFusedBatches = 2;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
// buffer resource word 3 for raw byte-addressed loads (32-bit data format),
// and the cache-policy operand of a non-temporal load
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCacheNT = 2;
// L2 bytes per XCD that the fused lift's cached row batches may take: at
// n = 1024 that is 8 of a block's 26 batches (2 MB of an XCD's 6.7 MB
// share; 6 to 9 batches measured alike, 2.41 -> 2.35 ms for the lift; 15
// or more thrash the 4 MB L2)
constexpr size_t kLiftCachedBytes = (size_t)2 << 20;
constexpr int kFusedMinThreads = kNumPrimes * (kDigitWords + 1);

// The step's share of the CRT for a block's kFusedComps components (one wave:
// sixteen lanes per component): the balanced u_l = y_l (P / q_l)^-1 mod q_l,
// k = round(X / P) and x mod 2^64 = (acc_0 + acc_1 2^32 - k P) mod 2^64,
// which need only the two low words of X.  The record (u_l, k) goes to
// urec (64 bytes a component) and x mod 2^64 to xlow; the full digit is
// formed later from the record.
__device__ __forceinline__ void fused_crt_share(const CrtTables& T, const int (&sY)[kNumPrimes][kFusedComps],
                                                const LiftParams* __restrict__ prm, int E, int c0, int n, int lane,
                                                uint8_t* __restrict__ urec, uint64_t* __restrict__ xlow) {
    static_assert(kFusedComps * kCrtLanes == 64, "one wave of CRT lanes");
    const int s = lane & (kCrtLanes - 1), cl = lane / kCrtLanes;
    const int comp = c0 + cl;
    if (comp >= n) return;  // the component's sixteen lanes leave together
    int ub[kCrtPrimesPerLane];
    double f = 0.0, a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int i = 0; i < kCrtPrimesPerLane; i++) {
        const int l = s + kCrtLanes * i;
        ub[i] = 0;
        if (l >= E) continue;
        const uint32_t q = T.qc[l][0];
        const uint32_t u = red16(mod_i32(sY[l][cl], q, T.qc[l][3]) * T.qc[l][2], q, T.qc[l][1]);
        ub[i] = balanced(u, q);
        f = fma((double)ub[i], T.qrec[l], f);
        a0 = fma((double)ub[i], T.Wd[l][0], a0);
        a1 = fma((double)ub[i], T.Wd[l][1], a1);
    }
    f = quad_add<8>(quad_add<4>(quad_add<2>(quad_add<1>(f))));
    a0 = quad_add<8>(quad_add<4>(quad_add<2>(quad_add<1>(a0))));
    a1 = quad_add<8>(quad_add<4>(quad_add<2>(quad_add<1>(a1))));
    int64_t ki = (int64_t)rint(f);
    const bool near = fabs(f - (double)ki) > 0.5 - 0x1p-30;
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
        // rare: some component's X / P lies near a half-integer, so its k
        // needs every word of X (the lanes still here take this branch)
        double acc[kDigitWords];
#pragma unroll
        for (int w = 0; w < kDigitWords; w++) acc[w] = 0.0;
#pragma unroll
        for (int i = 0; i < kCrtPrimesPerLane; i++) {
            const int l = min(s + kCrtLanes * i, kNumPrimes - 1);  // ub = 0 past E
#pragma unroll
            for (int w = 0; w < kDigitWords; w++) acc[w] = fma((double)ub[i], T.Wd[l][w], acc[w]);
        }
#pragma unroll
        for (int w = 0; w < kDigitWords; w++) acc[w] = quad_add<8>(quad_add<4>(quad_add<2>(quad_add<1>(acc[w]))));
        uint32_t x[kDigitWords];
        ki = crt_finish(acc, f, prm, x);
    }
    uint8_t* rec = urec + (size_t)comp * 64;
#pragma unroll
    for (int i = 0; i < kCrtPrimesPerLane; i++) {
        const int l = s + kCrtLanes * i;
        if (l < E) rec[l] = (uint8_t)ub[i];
    }
    if (s == 0) {
        rec[63] = (uint8_t)ki;
        const uint64_t P64 = ((uint64_t)prm->Pw[1] << 32) | prm->Pw[0];
        xlow[comp] = (uint64_t)(int64_t)a0 + ((uint64_t)(int64_t)a1 << 32) - (uint64_t)ki * P64;
    }
}

__global__ __launch_bounds__(1024) void lift_gemv_crt_kernel(const int8_t* __restrict__ Sperm, int n, int pitch,
                                                            int E, const int8_t* __restrict__ rho,
                                                            const LiftParams* __restrict__ prm,
                                                            uint8_t* __restrict__ urec,
                                                            uint64_t* __restrict__ xlow, int cached) {
    constexpr int C = kFusedComps, KB = kFusedBatches;
    constexpr int kTabD = kNumPrimes * (kDigitWords + 1), kTabU = kNumPrimes * 4;
    constexpr int NP = 8 / C;  // primes per batch
    static_assert(kTabU <= kTabD && kTabD == kFusedMinThreads, "table fetch");
    __shared__ CrtTables T;
    __shared__ int sY[kNumPrimes][C];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: row addresses stay scalar
    const int nw = blockDim.x >> 6;
    const int c0 = blockIdx.x * C;
    // The CRT constants are fetched now and stored to LDS after the
    // contraction, so the fetch overlaps the row loads instead of preceding them.
    const double tabd = tid < kNumPrimes * kDigitWords ? (&prm->Wd[0][0])[tid]
                        : tid < kTabD                ? prm->qrec[tid - kNumPrimes * kDigitWords]
                                                     : 0.0;
    uint32_t tabu = 0;
    if (tid < kTabU) {
        const int l = tid >> 2, f = tid & 3;
        tabu = f == 0 ? prm->q[l] : f == 1 ? prm->mu16[l] : f == 2 ? prm->cinv[l] : prm->mu32[l];
    }
    // rows (prime r / C, component r mod C); batch b holds rows 8 b .. 8 b + 7
    // and wave w the batches w and w + nw.  Batches past the last re-read it
    // and rows past the last re-read it too; their sums are dropped.
    const int nrows = E * C, nb = (nrows + 7) >> 3;
    // the rows are read through one buffer resource over the live primes'
    // matrices (at most 53 n pitch < 2^32 bytes), each at a scalar offset
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Sperm, 0, (int)((size_t)E * n * pitch), kBufferWord3);
    uint32_t rowo[KB][8];
    const int8_t* rvp[KB][NP];
#pragma unroll
    for (int kb = 0; kb < KB; kb++) {
        const int rb = 8 * min(wave + nw * kb, nb - 1);
#pragma unroll
        for (int r = 0; r < 8; r++) {
            const int rr = min(rb + r, nrows - 1);
            const int jl = rr / C, comp = min(c0 + rr % C, n - 1);
            rowo[kb][r] = (uint32_t)(((size_t)jl * n + comp) * pitch);
        }
#pragma unroll
        for (int p = 0; p < NP; p++) rvp[kb][p] = rho + (size_t)min(rb / C + p, E - 1) * pitch;
    }
    int acc[KB][8];
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int r = 0; r < 8; r++) acc[kb][r] = 0;
    for (int col0 = 0; col0 < pitch; col0 += 1024) {
        const int col = col0 + lane * 16;
        const bool cin = col < pitch;
        const uint32_t colc = cin ? col : col0;
        // every load is issued before any is used; lanes past the pitch
        // re-read the pass's first column and take rho as zero
        uint4 sv[KB][8], rvs[KB][NP];
#pragma unroll
        for (int kb = 0; kb < KB; kb++) {
#pragma unroll
            for (int p = 0; p < NP; p++) rvs[kb][p] = *(const uint4*)(rvp[kb][p] + colc);
            // the block's first `cached` batches with plain loads, the rest
            // non-temporal: each XCD's blocks read the same rows every step,
            // and those then stay in its L2 from step to step
            const bool keep = wave + nw * kb < cached;
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const v4u t = keep ? __builtin_amdgcn_raw_buffer_load_b128(srs, colc, rowo[kb][r], 0)
                                   : __builtin_amdgcn_raw_buffer_load_b128(srs, colc, rowo[kb][r], kCacheNT);
                sv[kb][r] = make_uint4(t.x, t.y, t.z, t.w);
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
#pragma unroll
            for (int p = 0; p < NP; p++) {
                rvs[kb][p].x = cin ? rvs[kb][p].x : 0u;
                rvs[kb][p].y = cin ? rvs[kb][p].y : 0u;
                rvs[kb][p].z = cin ? rvs[kb][p].z : 0u;
                rvs[kb][p].w = cin ? rvs[kb][p].w : 0u;
            }
#pragma unroll
        for (int kb = 0; kb < KB; kb++) {
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const uint4 rv = rvs[kb][r / C];
                int a = acc[kb][r];
                a = __builtin_amdgcn_sdot4((int)sv[kb][r].x, (int)rv.x, a, false);
                a = __builtin_amdgcn_sdot4((int)sv[kb][r].y, (int)rv.y, a, false);
                a = __builtin_amdgcn_sdot4((int)sv[kb][r].z, (int)rv.z, a, false);
                a = __builtin_amdgcn_sdot4((int)sv[kb][r].w, (int)rv.w, a, false);
                acc[kb][r] = a;
            }
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; kb++) {
        const int b = wave + nw * kb;
        if (b >= nb) continue;
        wave_sum_rows<8>(acc[kb], lane);
        const int rr = 8 * b + ((lane >> 3) & 7);
        if ((lane & 7) == 0 && rr < nrows) sY[rr / C][rr % C] = acc[kb][0];
    }
    if (tid < kTabD) {
        if (tid < kNumPrimes * kDigitWords) (&T.Wd[0][0])[tid] = tabd;
        else T.qrec[tid - kNumPrimes * kDigitWords] = tabd;
    }
    if (tid < kTabU) (&T.qc[0][0])[tid] = tabu;
    __syncthreads();
    if (wave == 0) fused_crt_share(T, sY, prm, E, c0, n, lane, urec, xlow);
}

// The digits of a run of steps from their records: one thread per (step,
// component) forms X = sum_l u_l (P / q_l) word by word (exact in double, as
// above) and subtracts the recorded k P.
__global__ __launch_bounds__(256) void crt_records_kernel(const uint8_t* __restrict__ urec, int nrec, int n,
                                                          const LiftParams* __restrict__ prm,
                                                          uint64_t* __restrict__ digits, int dstride, int slot0) {
    __shared__ double sW[kNumPrimes][kDigitWords];
    for (int i = threadIdx.x; i < kNumPrimes * kDigitWords; i += 256) (&sW[0][0])[i] = (&prm->Wd[0][0])[i];
    __syncthreads();
    const int E = prm->E;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)nrec * n) return;
    const int rs = (int)(idx / n), comp = (int)(idx % n);
    const uint4* rp = (const uint4*)(urec + idx * 64);
    uint32_t wv[16];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const uint4 t = rp[v];
        wv[4 * v] = t.x, wv[4 * v + 1] = t.y, wv[4 * v + 2] = t.z, wv[4 * v + 3] = t.w;
    }
    double acc[kDigitWords];
#pragma unroll
    for (int w = 0; w < kDigitWords; w++) acc[w] = 0.0;
#pragma unroll
    for (int l = 0; l < kNumPrimes; l++) {
        if (l >= E) break;
        const double u = (double)(int8_t)(wv[l >> 2] >> (8 * (l & 3)));
#pragma unroll
        for (int w = 0; w < kDigitWords; w++) acc[w] = fma(u, sW[l][w], acc[w]);
    }
    uint32_t x[kDigitWords];
    crt_sub_kP(acc, (int64_t)(int8_t)(wv[15] >> 24), prm, x);
    uint4* dst = (uint4*)(digits + ((size_t)comp * dstride + slot0 + rs) * kDigitLimbs);
    dst[0] = make_uint4(x[0], x[1], x[2], x[3]);
    dst[1] = make_uint4(x[4], x[5], x[6], x[7]);
    dst[2] = make_uint4(x[8], x[9], x[10], x[11]);
}

// ---------------------------------------------------------------- lift: residual
// r <- (r - A x_low) P^-1 mod 2^64, one wave per row.  The true quotient lies
// in (-2^63, 2^63) (card, "Method": the residual stays one signed 64-bit limb
// when n max|A| < 2^63), so the wrapped product read as int64 is exact.
// The new residual is split at once into the next step's balanced residues,
// stored permuted by rowpos.  With first != 0 only the split of r = b runs.
template <typename AT, int CT>
__global__ __launch_bounds__(256) void residual_kernel(const AT* __restrict__ A, int n, int c,
                                                       int64_t* __restrict__ R,
                                                       const uint64_t* __restrict__ xlow,
                                                       const LiftParams* __restrict__ prm,
                                                       const int* __restrict__ rowpos,
                                                       int8_t* __restrict__ rho, int pitch, int first) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n) return;
    const int E = prm->E;
    const uint64_t Pinv = prm->Pinv;
    uint32_t q = 1, mu16 = 0, mu32 = 0, r32 = 0;
    int pos = 0;
    if (lane < E) {
        q = prm->q[lane];
        mu16 = prm->mu16[lane];
        mu32 = prm->mu32[lane];
        r32 = prm->r32[lane];
        pos = rowpos ? rowpos[(size_t)prm->qidx[lane] * n + r] : r;  // null: natural order
    }
    for (int t0 = 0; t0 < c; t0 += CT) {
        uint64_t acc[CT];
#pragma unroll
        for (int t = 0; t < CT; t++) acc[t] = 0;
        if (!first) {
            const AT* a = A + (size_t)r * n;
            for (int jc = lane; jc < n; jc += 64) {
                const uint64_t av = (uint64_t)(int64_t)a[jc];
                const uint64_t* xr = xlow + (size_t)jc * c + t0;
#pragma unroll
                for (int t = 0; t < CT; t++)
                    if (t0 + t < c) acc[t] += av * xr[t];
            }
#pragma unroll
            for (int t = 0; t < CT; t++)
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) acc[t] += __shfl_xor(acc[t], off);
        }
#pragma unroll
        for (int t = 0; t < CT; t++) {
            if (t0 + t >= c) continue;
            int64_t* rp = R + (size_t)r * c + t0 + t;
            const uint64_t old = (uint64_t)*rp;
            const uint64_t val = first ? old : (old - acc[t]) * Pinv;
            if (!first && lane == 0) *rp = (int64_t)val;
            if (lane < E) {
                const uint32_t res = mod_i64((int64_t)val, q, mu16, mu32, r32);
                rho[((size_t)lane * c + t0 + t) * pitch + pos] = (int8_t)balanced(res, q);
            }
        }
    }
}

// 64-bit sum over the wave, in every lane (the butterfly of the GEMV's row sums)
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v, int lane) {
    auto level = [&](auto bit) {
        constexpr int B = decltype(bit)::value;
        const int lo = xchg_bit<B>((int)(uint32_t)v, lane);
        const int hi = xchg_bit<B>((int)(uint32_t)(v >> 32), lane);
        v += ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
    };
    level(std::integral_constant<int, 32>{});
    level(std::integral_constant<int, 16>{});
    level(std::integral_constant<int, 8>{});
    level(std::integral_constant<int, 4>{});
    level(std::integral_constant<int, 2>{});
    level(std::integral_constant<int, 1>{});
    return v;
}

// The same update for one right-hand side (int32 A): one wave per row, 16-byte
// loads of A and x_low, the 64-bit sums meet in a wave butterfly, and lanes
// below E write the balanced residues of r_{i+1}.  Everything the tail needs
// (the prime constants, the row's position in each prime's order, r_i) is
// fetched first, and a row's loads of A and x_low go out four passes at a
// time, so the wave waits on memory about once.
// rpos[i][l] = rowpos[qidx[l]][i] for the live primes l < E: where row i's
// residue goes in each prime's order (one wave per row)
__global__ __launch_bounds__(256) void lift_positions_kernel(const int* __restrict__ rowpos,
                                                             const LiftParams* __restrict__ prm, int n,
                                                             int* __restrict__ rpos) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n || lane >= prm->E) return;
    rpos[(size_t)r * 64 + lane] = rowpos[(size_t)prm->qidx[lane] * n + r];
}

template <bool kAligned>  // n % 4 == 0: rows start 16-byte aligned
__global__ __launch_bounds__(256) void residual1_kernel(const int32_t* __restrict__ A, int n,
                                                        int64_t* __restrict__ R,
                                                        const uint64_t* __restrict__ xlow,
                                                        const LiftParams* __restrict__ prm,
                                                        const int* __restrict__ rpos,
                                                        int8_t* __restrict__ rho, int pitch) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n) return;
    const int E = prm->E;
    const bool split = lane < E;
    const int pl = split ? lane : 0;
    // independent loads only: the tail's operands, then the row
    const uint32_t q = prm->q[pl], mu16 = prm->mu16[pl], mu32 = prm->mu32[pl], r32 = prm->r32[pl];
    const int pos = rpos[(size_t)r * 64 + pl];
    const uint64_t Rr = (uint64_t)R[r];
    const int32_t* a = A + (size_t)r * n;
    uint64_t acc = 0;
    if constexpr (kAligned) {
        int j0 = lane * 4;
        int4 av[4];
        ulonglong2 x01[4], x23[4];
        // the first four passes (n >= 1024 covers them all at n = 1024)
#pragma unroll
        for (int u = 0; u < 4; u++) {
            // lanes past the row re-read its start; their terms are dropped below
            const int jc = j0 + 256 * u < n ? j0 + 256 * u : 0;
            av[u] = *(const int4*)(a + jc);
            x01[u] = *(const ulonglong2*)(xlow + jc);
            x23[u] = *(const ulonglong2*)(xlow + jc + 2);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first use
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const uint64_t t = (uint64_t)(int64_t)av[u].x * x01[u].x + (uint64_t)(int64_t)av[u].y * x01[u].y +
                               (uint64_t)(int64_t)av[u].z * x23[u].x + (uint64_t)(int64_t)av[u].w * x23[u].y;
            acc += j0 + 256 * u < n ? t : 0;
        }
        for (j0 += 1024; j0 < n; j0 += 256) {
            const int4 v = *(const int4*)(a + j0);
            const ulonglong2 y01 = *(const ulonglong2*)(xlow + j0);
            const ulonglong2 y23 = *(const ulonglong2*)(xlow + j0 + 2);
            acc += (uint64_t)(int64_t)v.x * y01.x + (uint64_t)(int64_t)v.y * y01.y +
                   (uint64_t)(int64_t)v.z * y23.x + (uint64_t)(int64_t)v.w * y23.y;
        }
    } else {
        for (int jc = lane; jc < n; jc += 64) acc += (uint64_t)(int64_t)a[jc] * xlow[jc];
    }
    acc = wave_sum_u64(acc, lane);
    const uint64_t val = (Rr - acc) * prm->Pinv;
    if (lane == 0) R[r] = (int64_t)val;
    if (split) {
        const uint32_t res = mod_i64((int64_t)val, q, mu16, mu32, r32);
        rho[(size_t)lane * pitch + pos] = (int8_t)balanced(res, q);
    }
}

// ---------------------------------------------------------------- lift: residual on MFMA
// For c right-hand sides the product A x_low (mod 2^64) is a sum of int8
// matrix products: A = sum_a A_a 256^a with balanced byte planes A_a (four
// planes cover |A| < 2^30), x_low = sum_b X_b 256^b (mod 2^64) with eight
// balanced byte planes, and modulo 2^64 only the 26 pairs a + b < 8 matter:
//   A x_low = sum_{a + b < 8} 256^(a + b) (A_a X_b)  (mod 2^64),
// each A_a X_b exact in int32 (|entry| <= n 128^2 < 2^31 for n < 2^17).

// A_a[i][k] for k < pitch (zero past n), four columns a thread
__global__ __launch_bounds__(256) void a_planes_kernel(const int32_t* __restrict__ A, int n, int pitch,
                                                       int8_t* __restrict__ Ab) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int q4 = pitch / 4;
    if (idx >= (size_t)n * q4) return;
    const int i = (int)(idx / q4), k0 = (int)(idx % q4) * 4;
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; e++) {
        int32_t v = k0 + e < n ? A[(size_t)i * n + k0 + e] : 0;
#pragma unroll
        for (int a = 0; a < 4; a++) {
            const int8_t d = (int8_t)(v & 0xff);
            w[a] |= (uint32_t)(uint8_t)d << (8 * e);
            v = (v - d) >> 8;
        }
    }
    const size_t plane = (size_t)n * pitch;
#pragma unroll
    for (int a = 0; a < 4; a++) *(uint32_t*)(Ab + a * plane + (size_t)i * pitch + k0) = w[a];
}

constexpr int kResWaves = 8;  // waves of a block, splitting the contraction

// Block: rows i0 .. i0 + 15 and columns t0 .. t0 + 15; wave w takes the
// 64-byte chunks w, w + 8, ... of the contraction.  Then r <- (r - A x_low)
// P^-1 and the next step's balanced residues, in natural row order.
__global__ __launch_bounds__(kResWaves * 64) void residual_mfma_kernel(
    const int8_t* __restrict__ Ab, const int8_t* __restrict__ xp, int n, int c, int pitch,
    int64_t* __restrict__ R, const LiftParams* __restrict__ prm, int8_t* __restrict__ rho) {
    typedef int v4i_r __attribute__((ext_vector_type(4)));
    __shared__ uint64_t part[kResWaves][4][64];
    __shared__ uint64_t sval[16][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int i0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
    // planes through buffer resources: one 32-bit lane offset per operand,
    // each plane at a scalar offset (both arrays below 2^31 bytes)
    const uint32_t plane = (uint32_t)n * pitch, bstride = (uint32_t)c * pitch;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)Ab, 0, (int)(4 * plane), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc((void*)xp, 0, (int)(8 * bstride), kBufferWord3);
    const uint32_t arow = (uint32_t)min(i0 + lr, n - 1) * pitch;  // rows past n: dropped below
    const int tb = t0 + lr;
    const bool okB = tb < c;
    const uint32_t xcol = (uint32_t)(okB ? tb : 0) * pitch;
    v4i_r acc[26];
#pragma unroll
    for (int p = 0; p < 26; p++) acc[p] = v4i_r{0, 0, 0, 0};
    const int nch = pitch / 64;
    // A (from HBM) in two buffers taken in turn: the next chunk's A loads are
    // in flight while the current chunk's x planes (from L2) arrive and its
    // 26 products run; past the end a buffer re-reads its own chunk, unused
    v4i_r a0[4], a1[4], bv[8];
    auto loadA = [&](int ch, v4i_r (&A4)[4]) {
        const uint32_t k = ch * 64 + 16 * lg;
#pragma unroll
        for (int a = 0; a < 4; a++) A4[a] = (v4i_r)__builtin_amdgcn_raw_buffer_load_b128(rsA, arow + k, a * plane, 0);
    };
    auto loadB = [&](int ch) {
        const uint32_t k = ch * 64 + 16 * lg;
#pragma unroll
        for (int b = 0; b < 8; b++) bv[b] = (v4i_r)__builtin_amdgcn_raw_buffer_load_b128(rsB, xcol + k, b * bstride, 0);
    };
    auto products = [&](v4i_r (&A4)[4]) {
        if (!okB) {
#pragma unroll
            for (int b = 0; b < 8; b++) bv[b] = v4i_r{0, 0, 0, 0};
        }
        int p = 0;
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
            for (int b = 0; b + a < 8; b++, p++) acc[p] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A4[a], bv[b], acc[p], 0, 0, 0);
    };
    if (wave < nch) loadA(wave, a0);
    for (int ch = wave; ch < nch; ch += 2 * kResWaves) {
        const int c1 = ch + kResWaves, c2 = ch + 2 * kResWaves;
        loadB(ch);
        loadA(c1 < nch ? c1 : ch, a1);
        __builtin_amdgcn_sched_barrier(0);
        products(a0);
        __builtin_amdgcn_sched_barrier(0);
        if (c1 >= nch) break;
        loadB(c1);
        loadA(c2 < nch ? c2 : c1, a0);
        __builtin_amdgcn_sched_barrier(0);
        products(a1);
        __builtin_amdgcn_sched_barrier(0);
    }
    // lane: column t0 + lr, rows i0 + 4 lg + 0..3; fold the pairs into 64 bits
#pragma unroll
    for (int r = 0; r < 4; r++) {
        uint64_t v = 0;
        int p = 0;
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
            for (int b = 0; b + a < 8; b++, p++) v += (uint64_t)(int64_t)acc[p][r] << (8 * (a + b));
        part[wave][r][lane] = v;
    }
    __syncthreads();
    const uint64_t Pinv = prm->Pinv;
    if (tid < 256) {
        const int rho_ = tid >> 4, tt = tid & 15;  // element (row i0 + rho_, column t0 + tt)
        const int ln = 16 * (rho_ >> 2) + tt, r = rho_ & 3;
        uint64_t sum = 0;
#pragma unroll
        for (int w = 0; w < kResWaves; w++) sum += part[w][r][ln];
        const int i = i0 + rho_, t = t0 + tt;
        uint64_t val = 0;
        if (i < n && t < c) {
            int64_t* rp = R + (size_t)i * c + t;
            val = ((uint64_t)*rp - sum) * Pinv;
            *rp = (int64_t)val;
        }
        sval[rho_][tt] = val;
    }
    __syncthreads();
    // next residues in natural row order (the lift reads B_j with its
    // columns in that order): wave w takes the live primes w, w + 8, ...;
    // lane (t, g) the column t0 + t and rows 4 g .. 4 g + 3, one word a store
    const int E = prm->E;
    const int t = lane >> 2, g = lane & 3;
    const bool colok = t0 + t < c;
    const int r0 = i0 + 4 * g;
    for (int jl = wave; jl < E; jl += kResWaves) {
        const uint32_t q = prm->q[jl], mu16 = prm->mu16[jl], mu32 = prm->mu32[jl], r32 = prm->r32[jl];
        if (!colok) continue;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t res = mod_i64((int64_t)sval[4 * g + e][t], q, mu16, mu32, r32);
            w |= ((uint32_t)balanced(res, q) & 0xffu) << (8 * e);
        }
        int8_t* dst = rho + ((size_t)jl * c + t0 + t) * pitch + r0;
        if (r0 + 4 <= n) {
            *(uint32_t*)dst = w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++)
                if (r0 + e < n) dst[e] = (int8_t)(w >> (8 * e));
        }
    }
}

// Once per lift on the MFMA residual's path: every live prime's row of S
// rewritten in natural column order, S[J][i][r] <- S[J][i][rowpos[J][r]]
// (zero past n), so the contraction takes its residues in natural order.
// One block per (row, prime); the row goes through LDS.
__global__ __launch_bounds__(256) void natural_cols_kernel(int8_t* __restrict__ S, const int* __restrict__ rowpos,
                                                           const LiftParams* __restrict__ prm, int n, int pitch) {
    extern __shared__ __attribute__((aligned(16))) int8_t rowbuf[];
    const int J = prm->qidx[blockIdx.y];
    const int i = blockIdx.x;
    int8_t* row = S + ((size_t)J * n + i) * pitch;
    for (int k = threadIdx.x * 16; k < pitch; k += 256 * 16) *(uint4*)(rowbuf + k) = *(const uint4*)(row + k);
    __syncthreads();
    const int* rp = rowpos + (size_t)J * n;
    for (int r = threadIdx.x; r < pitch; r += 256) {
        const int k = r < n ? rp[r] : -1;
        row[r] = (k >= 0 && k < pitch) ? rowbuf[k] : (int8_t)0;
    }
}

bool residual_mfma_fits(const Layout& L, bool a32, uint64_t maxabs) {
    static const bool off = [] {
        const char* e = std::getenv("ES_RESIDUAL_VALU");
        return e && e[0] == '1';
    }();
    return !off && L.c > 1 && a32 && maxabs < ((uint64_t)1 << 30) && L.pitch % 64 == 0 && L.pitch <= 48 * 1024 &&
           4 * (size_t)L.n * L.pitch <= (size_t)0x7fffffff && 8 * (size_t)L.c * L.pitch <= (size_t)0x7fffffff;
}

hipError_t launch_natural_cols(const Layout& L, uint8_t* ws, int E, hipStream_t st) {
    if (E < 1 || E > kNumPrimes || L.pitch > 48 * 1024) return hipErrorInvalidValue;
    es_launch(natural_cols_kernel, dim3(L.n, E), dim3(256), (uint32_t)L.pitch, st, (int8_t*)(ws + L.off_S),
              (const int*)(ws + L.off_rowpos), (const LiftParams*)(ws + L.off_params), L.n, L.pitch);
    return hipGetLastError();
}

hipError_t launch_a_planes(const Layout& L, uint8_t* ws, hipStream_t st) {
    const size_t threads = (size_t)L.n * (L.pitch / 4);
    es_launch(a_planes_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
              (const int32_t*)(ws + L.off_A32), L.n, L.pitch, (int8_t*)(ws + L.off_Ab));
    return hipGetLastError();
}

hipError_t launch_split_b(const int64_t* b, const Layout& L, uint8_t* ws, int E, bool natural, hipStream_t st) {
    (void)E;
    hipError_t e = hipMemcpyAsync(ws + L.off_R, b, (size_t)L.n * L.c * sizeof(int64_t),
                                  hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
    const dim3 grid((L.n + 3) / 4);
    if (L.c == 1)
        es_launch((residual_kernel<int64_t, 1>), grid, dim3(256), 0, st, (const int64_t*)nullptr,
                           L.n, L.c, (int64_t*)(ws + L.off_R), (const uint64_t*)(ws + L.off_xlow),
                           (const LiftParams*)(ws + L.off_params), (const int*)(ws + L.off_rowpos),
                           (int8_t*)(ws + L.off_rho), L.pitch, 1);
    else
        es_launch((residual_kernel<int64_t, 16>), grid, dim3(256), 0, st, (const int64_t*)nullptr,
                           L.n, L.c, (int64_t*)(ws + L.off_R), (const uint64_t*)(ws + L.off_xlow),
                           (const LiftParams*)(ws + L.off_params),
                           natural ? (const int*)nullptr : (const int*)(ws + L.off_rowpos),
                           (int8_t*)(ws + L.off_rho), L.pitch, 1);
    return hipGetLastError();
}

template <int LPR, int RI, int CT>
static void launch_gemv_t(const Layout& L, uint8_t* ws, int E, hipStream_t st) {
    constexpr int ROWS = 4 * (64 / LPR) * RI;
    dim3 grid((L.n + ROWS - 1) / ROWS, E);
    es_launch((lift_gemv_kernel<LPR, RI, CT>), grid, dim3(256), 0, st,
                       (const int8_t*)(ws + L.off_S), L.n, L.pitch, L.c, (const int8_t*)(ws + L.off_rho),
                       (const LiftParams*)(ws + L.off_params), (const int*)(ws + L.off_rowpos),
                       ws + L.off_U);
}

template <int CT>
static void launch_gemv_c(const Layout& L, uint8_t* ws, int E, hipStream_t st) {
    switch (L.lpr) {
        case 4: launch_gemv_t<4, 1, CT>(L, ws, E, st); break;
        case 8: launch_gemv_t<8, 1, CT>(L, ws, E, st); break;
        case 16: launch_gemv_t<16, 2, CT>(L, ws, E, st); break;
        case 32: launch_gemv_t<32, 4, CT>(L, ws, E, st); break;
        default: launch_gemv_t<64, (CT == 1 ? 8 : 4), CT>(L, ws, E, st); break;
    }
}

// Contraction path: the v_dot4 GEMV for one right-hand side, MFMA for more
// (ES_LIFT_VALU=1 keeps the VALU kernel for c > 1, for comparison).
static bool lift_use_valu() {
    static const bool v = [] {
        const char* e = getenv("ES_LIFT_VALU");
        return e && e[0] == '1';
    }();
    return v;
}

// Rows per wave of the wide-row c = 1 contraction (8 unless ES_GEMV_RI=16):
// a tuning knob, both compute the same result.
static int gemv_rows_per_wave() {
    static const int v = [] {
        const char* e = getenv("ES_GEMV_RI");
        return (e && e[0] == '1') ? 16 : 8;
    }();
    return v;
}

template <int RI>
static void launch_gemv1_t(const Layout& L, uint8_t* ws, int E, hipStream_t st) {
    dim3 grid((L.n + 4 * RI - 1) / (4 * RI), E);
    es_launch(lift_gemv1_kernel<RI>, grid, dim3(256), 0, st, (const int8_t*)(ws + L.off_S), L.n, L.pitch,
                       (const int8_t*)(ws + L.off_rho), (const LiftParams*)(ws + L.off_params),
                       (const int*)(ws + L.off_rowpos), ws + L.off_U);
}

hipError_t launch_lift_contract(const Layout& L, uint8_t* ws, int E, hipStream_t st) {
    if (L.c == 1 && L.pitch >= 1024) {
        if (gemv_rows_per_wave() == 16) launch_gemv1_t<16>(L, ws, E, st);
        else launch_gemv1_t<8>(L, ws, E, st);
    } else if (L.c == 1) {
        launch_gemv_c<1>(L, ws, E, st);
    } else if (lift_use_valu()) {
        launch_gemv_c<16>(L, ws, E, st);
    } else {
        dim3 grid((L.n + 4 * kMfmaRowsPerWave - 1) / (4 * kMfmaRowsPerWave), E, (L.c + 15) / 16);
        es_launch(lift_mfma_kernel, grid, dim3(256), 0, st, (const int8_t*)(ws + L.off_S), L.n, L.pitch,
                           L.c, (const int8_t*)(ws + L.off_rho), (const LiftParams*)(ws + L.off_params),
                           (const int*)(ws + L.off_rowpos), ws + L.off_U);
    }
    return hipGetLastError();
}

bool lift_fused_fits(const Layout& L) {
    static const bool off = [] {
        const char* e = std::getenv("ES_FUSED_CRT");
        return e && e[0] == '0';
    }();
    return !off && fused_lift_shape(L.n, L.c, L.pitch);
}

hipError_t launch_lift_positions(const Layout& L, uint8_t* ws, hipStream_t st) {
    if (L.c != 1) return hipSuccess;
    es_launch(lift_positions_kernel, dim3((L.n + 3) / 4), dim3(256), 0, st, (const int*)(ws + L.off_rowpos),
              (const LiftParams*)(ws + L.off_params), L.n, (int*)(ws + L.off_rpos));
    return hipGetLastError();
}

hipError_t launch_lift_rows(const Layout& L, uint8_t* ws, int E, hipStream_t st) {
    es_launch(lift_rows_kernel, dim3((L.n + 3) / 4, E), dim3(256), 0, st, (const int8_t*)(ws + L.off_S),
                       (const int*)(ws + L.off_rowpos), (const LiftParams*)(ws + L.off_params), L.n, L.pitch,
                       (int8_t*)(ws + L.off_Sperm));
    return hipGetLastError();
}

hipError_t launch_lift_contract_crt(const Layout& L, uint8_t* ws, int E, int slot, hipStream_t st) {
    if (E < 1 || E > kNumPrimes) return hipErrorInvalidValue;
    if (!fused_lift_shape(L.n, L.c, L.pitch)) return hipErrorInvalidValue;
    // four components per block (two and eight measured slower at n = 1024)
    const int nb = (E * kFusedComps + 7) / 8;
    const int waves = max((nb + kFusedBatches - 1) / kFusedBatches, (kFusedMinThreads + 63) / 64);
    if (slot < 0 || slot >= L.krec) return hipErrorInvalidValue;
    const int blocks = (L.n + kFusedComps - 1) / kFusedComps;
    // cached batches a block: kLiftCachedBytes over the XCD's blocks (dealt
    // round-robin to the eight XCDs) at 8 rows of `pitch` bytes a batch
    const int cached = (int)std::min<size_t>((size_t)nb, kLiftCachedBytes / ((size_t)((blocks + 7) / 8) * 8 * L.pitch));
    es_launch(lift_gemv_crt_kernel, dim3(blocks), dim3(waves * 64), 0, st,
                       (const int8_t*)(ws + L.off_Sperm), L.n, L.pitch, E, (const int8_t*)(ws + L.off_rho),
                       (const LiftParams*)(ws + L.off_params), ws + L.off_urec + (size_t)slot * L.n * 64,
                       (uint64_t*)(ws + L.off_xlow), cached);
    return hipGetLastError();
}

hipError_t launch_lift_crt_records(const Layout& L, uint8_t* ws, int nrec, int slot0, hipStream_t st) {
    if (nrec < 1 || nrec > L.krec || slot0 < 0 || slot0 + nrec > L.kchunk) return hipErrorInvalidValue;
    const size_t threads = (size_t)nrec * L.n;
    es_launch(crt_records_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                       (const uint8_t*)(ws + L.off_urec), nrec, L.n, (const LiftParams*)(ws + L.off_params),
                       L.dig_dev ? L.dig_dev : (uint64_t*)(ws + L.off_digits), L.kchunk, slot0);
    return hipGetLastError();
}

hipError_t launch_lift_crt(const Layout& L, uint8_t* ws, int slot, bool planes, hipStream_t st) {
    if (planes && L.c < 2) return hipErrorInvalidValue;
    const int NC = L.n * L.c;
    es_launch(crt_kernel, dim3((NC + 15) / 16), dim3(256), 0, st,
                       (const LiftParams*)(ws + L.off_params), (const uint8_t*)(ws + L.off_U), NC,
                       L.dig_dev ? L.dig_dev : (uint64_t*)(ws + L.off_digits), L.kchunk, slot,
                       (uint64_t*)(ws + L.off_xlow), planes ? (int8_t*)(ws + L.off_xp) : (int8_t*)nullptr, L.c,
                       L.pitch);
    return hipGetLastError();
}

hipError_t launch_lift_residual(const Layout& L, uint8_t* ws, bool a32, const int64_t* A64, bool mfma,
                                hipStream_t st) {
    if (mfma) {
        if (!a32 || L.c < 2 || L.pitch % 64 != 0) return hipErrorInvalidValue;
        es_launch(residual_mfma_kernel, dim3((L.n + 15) / 16, (L.c + 15) / 16), dim3(kResWaves * 64), 0, st,
                  (const int8_t*)(ws + L.off_Ab), (const int8_t*)(ws + L.off_xp), L.n, L.c, L.pitch,
                  (int64_t*)(ws + L.off_R), (const LiftParams*)(ws + L.off_params), (int8_t*)(ws + L.off_rho));
        return hipGetLastError();
    }
    const dim3 grid((L.n + 3) / 4);
    const LiftParams* prm = (const LiftParams*)(ws + L.off_params);
    int64_t* R = (int64_t*)(ws + L.off_R);
    const uint64_t* xl = (const uint64_t*)(ws + L.off_xlow);
    const int* rp = (const int*)(ws + L.off_rowpos);
    int8_t* rho = (int8_t*)(ws + L.off_rho);
    if (a32) {
        const int32_t* A = (const int32_t*)(ws + L.off_A32);
        const int* rpos = (const int*)(ws + L.off_rpos);
        if (L.c == 1 && L.n % 4 == 0)
            es_launch(residual1_kernel<true>, dim3((L.n + 3) / 4), dim3(256), 0, st, A, L.n, R, xl, prm, rpos, rho,
                      L.pitch);
        else if (L.c == 1)
            es_launch(residual1_kernel<false>, dim3((L.n + 3) / 4), dim3(256), 0, st, A, L.n, R, xl, prm, rpos,
                      rho, L.pitch);
        else
            es_launch((residual_kernel<int32_t, 16>), grid, dim3(256), 0, st, A, L.n, L.c, R, xl,
                               prm, rp, rho, L.pitch, 0);
    } else {
        if (L.c == 1)
            es_launch((residual_kernel<int64_t, 1>), grid, dim3(256), 0, st, A64, L.n, L.c, R, xl,
                               prm, rp, rho, L.pitch, 0);
        else
            es_launch((residual_kernel<int64_t, 16>), grid, dim3(256), 0, st, A64, L.n, L.c, R, xl,
                               prm, rp, rho, L.pitch, 0);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- fixed scratch
// Device memory for es_batched_inverse_noalloc, the entry point for callers
// that cannot allocate: a file-scope array, one copy per device, held until
// the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol); the device address of
// this device's copy is looked up once per device, with that device current,
// and kept.
constexpr size_t kFixedScratchBytes = (size_t)24 << 20;
static __device__ __align__(256) uint8_t scratch[kFixedScratchBytes];

size_t fixed_scratch_bytes() { return kFixedScratchBytes; }

uint8_t* fixed_scratch() {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptr[dev] = p;
    }
    return (uint8_t*)ptr[dev];
}

}  // namespace es
