// HIP kernels for the rational-reconstruction stage on CDNA4 (gfx950).
//
// Method (exact-solve card, phanerozoic/exact-solve, section "Method"): the
// lift stops when M = P^m is larger than 2 N D (N, D the Hadamard-type
// bounds on numerators and denominator); the denominator d shared by the
// components is found from a few of them, and each numerator is then a
// single product modulo M, y = d X mods M with X = sum_i x_i P^i, accepted
// when |y| <= N.  Here all numerators are formed at once as one
// int8 GEMM on the matrix cores:
//
//   X_j = sum_{i, b} s_{j,i,b} 256^b P^i, where s_{j,i,b} are the balanced
//   bytes of the balanced base-P digit x_i of component j, so
//   d X_j = sum_{i, b} s_{j,i,b} W_{i,b}  (mod M),  W_{i,b} = 256^b P^i d mod M.
//
// Every weight lies in [0, 2M), so the GEMM's column sums (bytes of V_j)
// carry a value |V_j| < K 256 M, and y_j = V_j - t_j M with a one-word
// quotient t_j = round(V_j / M) that double precision gives exactly whenever
// |y_j| is as small as an accepted numerator must be.
//
// Weight rows W_{i,0} = P^i d mod M come from the host (a chain with known
// quotients); the rows for b = 1..41 are byte shifts reduced again, one wave
// per i (wchain_kernel).  The matrix is transposed so that both GEMM operands
// stream 16 bytes of the contraction index per lane.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "es_internal.h"

namespace es {

// ---------------------------------------------------------------- digit bytes
// One block per component row: 42 balanced bytes (each in [-128, 127]) of
// every 384-bit two's-complement digit x_i, |x_i| < 2^333, then 6 zero
// bytes, so slot i occupies bytes [48 i, 48 i + 48) of the row; slots past m
// and rows past the chunk's valid rows are zero.  rowsum = sum of the row's
// bytes (the GEMM stores weights offset by -128, see recon_gemm_kernel).
__global__ __launch_bounds__(256) void digit_bytes_kernel(const uint64_t* __restrict__ digits, int dstride,
                                                          int m, int j0, int valid_rows, int Kpad,
                                                          int8_t* __restrict__ S, int* __restrict__ rowsum) {
    const int r = blockIdx.x;
    const int nslot = Kpad / 48;
    int sum = 0;
    for (int i = threadIdx.x; i < nslot; i += 256) {
        uint32_t outw[12];
#pragma unroll
        for (int w = 0; w < 12; w++) outw[w] = 0;
        if (r < valid_rows && i < m) {
            const uint64_t* x = digits + ((size_t)(j0 + r) * dstride + i) * kDigitLimbs;
            uint64_t u[kDigitLimbs];
#pragma unroll
            for (int w = 0; w < kDigitLimbs; w++) u[w] = x[w];
            int carry = 0;
#pragma unroll
            for (int b = 0; b < 41; b++) {
                const int v = (int)((u[b >> 3] >> (8 * (b & 7))) & 0xffu) + carry;
                const int s = v >= 128 ? v - 256 : v;
                carry = v >= 128 ? 1 : 0;
                sum += s;
                outw[b >> 2] |= ((uint32_t)s & 0xffu) << (8 * (b & 3));
            }
            // bits 328..335 read as a signed byte are x >> 328 (in [-32, 31])
            const int s41 = (int)(int8_t)((u[5] >> 8) & 0xffu) + carry;
            sum += s41;
            outw[10] |= ((uint32_t)s41 & 0xffu) << 8;
        }
        uint4* dst = (uint4*)(S + (size_t)r * Kpad + (size_t)i * 48);
        dst[0] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
        dst[1] = make_uint4(outw[4], outw[5], outw[6], outw[7]);
        dst[2] = make_uint4(outw[8], outw[9], outw[10], outw[11]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    __shared__ int part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) rowsum[r] = part[0] + part[1] + part[2] + part[3];
}

// ---------------------------------------------------------------- weight chains
// A wave-resident integer of NW = TM + 1 32-bit words (TM = index of the top
// word of 2M, so M's own top word may be zero); lane l holds words
// [l CW, l CW + CW).  One step replaces R in [0, 2M) by s R - t M with
// t = max(0, floor(s R / M - 2^-16)) for s <= 2^24.  The windows of R and M
// (three words from TM down, at least 63 significant bits of M) and the
// double-precision quotient put the estimate within about s 2^-50 <= 2^-26
// of s R / M, so t is the true floor or one less and the result stays in
// [0, 2M) without a comparison.
template <int CW>
__device__ __forceinline__ void wave_mul_reduce(uint32_t (&R)[CW], const uint32_t (&Mr)[CW], int lane, int TM,
                                                double Md, uint32_t s) {
    // top-word approximation of R (same window as Md), summed in lane 0's order
    double loc = 0.0;
#pragma unroll
    for (int c = 0; c < CW; c++) {
        const int w = lane * CW + c;
        const int e = w - TM;
        if (e >= -2 && e <= 0) loc += (double)R[c] * (e == 0 ? 1.0 : e == -1 ? 0x1p-32 : 0x1p-64);
    }
    // at most two lanes hold the window: gather their parts into lane 0's sum
    double tot = 0.0;
    for (int src = (TM - 2) / CW; src <= TM / CW && src < 64; src++)
        tot += __shfl(loc, src);
    double q = (double)s * tot / Md - 0x1p-16;
    int t = q <= 0.0 ? 0 : (int)q;
    t = __builtin_amdgcn_readfirstlane(t);
    // local multiply-subtract with a carry chain
    int64_t carry = 0;
#pragma unroll
    for (int c = 0; c < CW; c++) {
        const int64_t acc = carry + (int64_t)((uint64_t)s * R[c]) - (int64_t)((uint64_t)(uint32_t)t * Mr[c]);
        R[c] = (uint32_t)acc;
        carry = acc >> 32;
    }
    // carries into the next lane, then single-unit ripples until none remain
    int64_t cin = __shfl_up(carry, 1);
    if (lane == 0) cin = 0;
    for (;;) {
#pragma unroll
        for (int c = 0; c < CW; c++) {  // a zero carry leaves the words unchanged
            const int64_t v = (int64_t)R[c] + cin;
            R[c] = (uint32_t)v;
            cin = v >> 32;
        }
        // cin is now the unit carried out of this lane's words (0 or +-1)
        int64_t up = __shfl_up(cin, 1);
        if (lane == 0) up = 0;
        if (__ballot(up != 0) == 0) break;
        cin = up;
    }
}

// Weight rows: block i holds T_i = P^i d mod M (host, words in [0, M)) and
// writes rows 48 i + b, b < 42, of W [Kpad][Ncolsp] (u8, little-endian bytes
// of R_{i,b} = 256^b T_i reduced into [0, 2M)); rows 48 i + 42 .. 48 i + 47
// are zero.  Ncolsp / 4 <= 64 CW words per row are written, zero beyond TM.
// Wave w of the block takes the rows b = w (mod 3): one step by 256^w, then
// steps by 2^24, so the three chains of 14 steps run side by side.  With
// s = 2^24 the quotient estimate's error (about 2^-28) stays far inside the
// 2^-16 margin, so each step still lands in [0, 2M).
template <int CW>
__global__ __launch_bounds__(192) void wchain_kernel(const uint32_t* __restrict__ T, const uint32_t* __restrict__ Mw,
                                                     int TM, double Md, int Ncolsp, uint8_t* __restrict__ W) {
    const int i = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int w0 = threadIdx.x >> 6;
    uint32_t R[CW], Mr[CW];
#pragma unroll
    for (int c = 0; c < CW; c++) {
        const int w = lane * CW + c;
        R[c] = w <= TM ? T[(size_t)i * (TM + 1) + w] : 0u;
        Mr[c] = w <= TM ? Mw[w] : 0u;
    }
    if (w0 > 0) wave_mul_reduce<CW>(R, Mr, lane, TM, Md, 1u << (8 * w0));
    const int rowwords = Ncolsp / 4;
    for (int b = w0; b < 48; b += 3) {
        uint32_t* dst = (uint32_t*)(W + (size_t)(48 * i + b) * Ncolsp);
#pragma unroll
        for (int c = 0; c < CW; c++) {
            const int w = lane * CW + c;
            if (w < rowwords) dst[w] = b < 42 ? R[c] : 0u;
        }
        if (b + 3 < 42) wave_mul_reduce<CW>(R, Mr, lane, TM, Md, 1u << 24);
    }
}

// WT[col][k] = W[k][col] - 128 (as int8): 64 x 64 byte tiles through LDS.
__global__ __launch_bounds__(256) void transpose_offset_kernel(const uint8_t* __restrict__ W, int Kpad, int Ncolsp,
                                                               int8_t* __restrict__ WT) {
    __shared__ uint8_t tile[64][64 + 4];
    const int k0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int t = threadIdx.x;
    {
        const int rr = t >> 2, cc = (t & 3) * 16;
        const uint4 v = *(const uint4*)(W + (size_t)(k0 + rr) * Ncolsp + c0 + cc);
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 16; q++) tile[rr][cc + q] = (uint8_t)(ws[q >> 2] >> (8 * (q & 3)));
    }
    __syncthreads();
    {
        const int cr = t >> 2, kk = (t & 3) * 16;  // output row (column of W), 16 k values
        uint32_t ws[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 16; q++) ws[q >> 2] |= (uint32_t)(tile[kk + q][cr] ^ 0x80u) << (8 * (q & 3));
        *(uint4*)(WT + (size_t)(c0 + cr) * Kpad + k0 + kk) = make_uint4(ws[0], ws[1], ws[2], ws[3]);
    }
}

// ---------------------------------------------------------------- the GEMM
// V[j][col] = sum_k S[j][k] WT[col][k] (int8 x int8 -> int32) on
// v_mfma_i32_16x16x64_i8.  Block tile 128 (rows j) x 128 (columns) staged in
// LDS 64 bytes of k at a time; four waves in a 2 x 2 arrangement, each owning
// a 64 x 64 tile as 4 x 4 MFMA tiles.  Operand lanes: lane l feeds row (or
// column) l % 16 with the 16 bytes k in [16 (l / 16), +16) of the 64-byte
// chunk; output lane l holds column l % 16, rows 4 (l / 16) + 0..3.  Row and
// column counts are multiples of 128 and Kpad of 64 (the caller pads), so
// nothing is bounds-checked.
typedef int v4i __attribute__((ext_vector_type(4)));
static int device_cus();

constexpr int kGemmLds = 64 + 16;  // LDS row stride, bytes

__global__ __launch_bounds__(256) void recon_gemm_kernel(const int8_t* __restrict__ S, const int8_t* __restrict__ WT,
                                                         int Kpad, int Ncolsp, int* __restrict__ V, int nx,
                                                         int tiles) {
    __shared__ __attribute__((aligned(16))) int8_t As[128 * kGemmLds];
    __shared__ __attribute__((aligned(16))) int8_t Bs[128 * kGemmLds];
    // Blocks go to the eight XCDs round-robin by index; tile number
    // (b mod 8) (grid / 8) + b / 8 gives each XCD a run of consecutive
    // tiles (row tiles fastest), so the row tiles that share a weight tile
    // share an L2 instead of each XCD reading every weight tile.  The grid
    // is a multiple of 8; tiles past the last do nothing.
    const int b = blockIdx.x;
    const int tile = (b & 7) * (int)(gridDim.x >> 3) + (b >> 3);
    if (tile >= tiles) return;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int j0 = (tile % nx) * 128, c0 = (tile / nx) * 128;
    const int lr = lane & 15, lg = lane >> 4;
    v4i acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[a][b] = v4i{0, 0, 0, 0};
    // global -> LDS: thread t moves rows t / 4 and t / 4 + 64, 16-byte chunk t % 4
    const int gr = t >> 2, gc = (t & 3) * 16;
    const int8_t* Ag0 = S + (size_t)(j0 + gr) * Kpad + gc;
    const int8_t* Ag1 = S + (size_t)(j0 + gr + 64) * Kpad + gc;
    const int8_t* Bg0 = WT + (size_t)(c0 + gr) * Kpad + gc;
    const int8_t* Bg1 = WT + (size_t)(c0 + gr + 64) * Kpad + gc;
    v4i ra0 = *(const v4i*)Ag0, ra1 = *(const v4i*)Ag1, rb0 = *(const v4i*)Bg0, rb1 = *(const v4i*)Bg1;
    for (int k = 0; k < Kpad; k += 64) {
        __syncthreads();  // previous chunk's fragments are read
        *(v4i*)(As + gr * kGemmLds + gc) = ra0;
        *(v4i*)(As + (gr + 64) * kGemmLds + gc) = ra1;
        *(v4i*)(Bs + gr * kGemmLds + gc) = rb0;
        *(v4i*)(Bs + (gr + 64) * kGemmLds + gc) = rb1;
        __syncthreads();
        if (k + 64 < Kpad) {  // next chunk's loads overlap this chunk's MFMAs
            ra0 = *(const v4i*)(Ag0 + k + 64);
            ra1 = *(const v4i*)(Ag1 + k + 64);
            rb0 = *(const v4i*)(Bg0 + k + 64);
            rb1 = *(const v4i*)(Bg1 + k + 64);
        }
        v4i fa[4], fb[4];
#pragma unroll
        for (int a = 0; a < 4; a++) fa[a] = *(const v4i*)(As + (64 * wr + 16 * a + lr) * kGemmLds + 16 * lg);
#pragma unroll
        for (int b = 0; b < 4; b++) fb[b] = *(const v4i*)(Bs + (64 * wc + 16 * b + lr) * kGemmLds + 16 * lg);
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
            for (int b = 0; b < 4; b++) acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int col = c0 + 64 * wc + 16 * b + lr;
            const int j = j0 + 64 * wr + 16 * a + 4 * lg;
#pragma unroll
            for (int r = 0; r < 4; r++) V[(size_t)(j + r) * Ncolsp + col] = acc[a][b][r];
        }
}

// ---------------------------------------------------------------- lowest terms
// g_j = gcd(|y_j|, d) for every accepted component, two waves per component,
// by Lehmer's method on numbers held as signed radix-2^30 limbs,
// sum_k l_k 2^(30 k) with every |l_k| < 0.58 2^30; limb k sits in lane
// k % 64, slot k / 64, so a number's limbs fill the low slots and the work of
// a round shrinks with the numbers.
//
// A round reads three limbs of each number at the larger one's top (in
// double precision, a leading part with about 52 exact bits of a and the
// bits of b at the same scale), runs Euclidean steps on them while the
// divisor keeps 26 bits and the cofactors stay within 2^26, and applies the
// 2 x 2 cofactor matrix [A B; C D] limb by limb: v = A a_k + B b_k is split
// at once into a low part in [-2^29, 2^29), kept in the limb, and a high part
// added to limb k + 1, so no carry ever ripples.  (With |l| <= L before the
// round, |v| <= 2^27 L and the new limb is within 2^29 + L / 8 + 1/2; the
// bound 0.58 2^30 is kept.)  The sign of a number is the sign of its top
// limb, and a negative number is negated.  Any integer matrix of
// determinant +-1 keeps the gcd, so a round is correct whatever the leading
// bits decide; it only has to make progress, and a round that cannot (a
// quotient of 2^26 or more: lengths more than about 26 bits apart) hands the
// component to the host.  Once both numbers fit in four limbs they are read
// out exactly and finished by the binary gcd.  Results: gstat 0 and G = g
// when g fits 64 bits, else gstat 1 (the host finishes that component).
//
// The two waves of a component overlap the two halves of a round: wave 1
// holds the limbs and applies each round's matrix; wave 0 runs the
// Euclidean steps of the next round meanwhile.  A matrix changes limb k
// using limbs k and k - 1 only, so the six limbs h - 4 .. h + 1 around the
// top h, which wave 1 hands over after every apply, give wave 0 the exact
// limbs h - 3 .. h + 2 after the next matrix (one lane per limb): enough for
// the next leading parts.  (When the top falls too far for that window, or
// the numbers reach the last four limbs, wave 0 issues the identity once and
// reads a fresh window.)  One barrier per round; matrices, commands and
// windows are double-buffered in LDS.

// lane l <- lane l - 1, lane 0 <- lane 63
__device__ __forceinline__ int32_t wave_ror1(int32_t v) {
    return __builtin_amdgcn_mov_dpp(v, 0x13c, 0xf, 0xf, false);
}

// bits [30 k, 30 k + 30) of a little-endian word array (words past n read as ext)
__device__ __forceinline__ int32_t chunk30(const uint32_t* __restrict__ W, int n, uint32_t ext, int k) {
    const int bit = 30 * k, w = bit >> 5, o = bit & 31;
    const uint32_t lo = w < n ? W[w] : ext;
    const uint32_t hi = w + 1 < n ? W[w + 1] : ext;
    return (int32_t)(__builtin_amdgcn_alignbit(hi, lo, o) & 0x3fffffffu);
}

// (a, b) <- (A a + B b, C a + D b) over slots [0, ns); the high parts
// leaving slot ns - 1 are dropped (the limbs above the live ones are zero,
// and the top live limb lies below the last lane of slot ns - 1)
constexpr int kSlotGroup = 4;  // slots a limb pass takes at a time (straight-line code)

// (a, b) <- (A a + B b, C a + D b) over slots [0, ns) rounded up to whole
// groups of kSlotGroup slots (ns wave-uniform); the slots above the live
// ones hold zeros and stay zero, and the high parts leaving the last slot
// taken are dropped (the limbs above the live ones are zero, and the top
// live limb lies below the last lane of slot ns - 1)
template <int CW>
__device__ __forceinline__ void limb_apply(int32_t (&a)[CW], int32_t (&b)[CW], int32_t A, int32_t B, int32_t C,
                                           int32_t D, int ns, bool lane0) {
    int32_t pa = 0, pb = 0;  // high parts of the slot below, rotated one lane up
#pragma unroll
    for (int c0 = 0; c0 < CW; c0 += kSlotGroup) {
        if (c0 >= ns) break;
#pragma unroll
        for (int c = c0; c < c0 + kSlotGroup && c < CW; c++) {
            // w = v + 2^29: high part floor(w / 2^30), low part (w mod 2^30) - 2^29
            const int64_t wa = (int64_t)A * a[c] + ((int64_t)B * b[c] + (1 << 29));
            const int64_t wb = (int64_t)C * a[c] + ((int64_t)D * b[c] + (1 << 29));
            const uint32_t wal = (uint32_t)wa, wah = (uint32_t)((uint64_t)wa >> 32);
            const uint32_t wbl = (uint32_t)wb, wbh = (uint32_t)((uint64_t)wb >> 32);
            const int32_t ra = wave_ror1((int32_t)__builtin_amdgcn_alignbit(wah, wal, 30));
            const int32_t rb = wave_ror1((int32_t)__builtin_amdgcn_alignbit(wbh, wbl, 30));
            a[c] = (int32_t)(wal & 0x3fffffffu) - (1 << 29) + (lane0 ? pa : ra);
            b[c] = (int32_t)(wbl & 0x3fffffffu) - (1 << 29) + (lane0 ? pb : rb);
            pa = ra;
            pb = rb;
        }
    }
}

// highest limb index at or below slot s_hi at which a or b is nonzero (-1
// when both are zero there)
template <int CW>
__device__ __forceinline__ int top_limb(const int32_t (&a)[CW], const int32_t (&b)[CW], int s_hi) {
    for (int s = s_hi; s >= 0; s--) {
        const uint64_t m = __ballot((a[s] | b[s]) != 0);
        if (m != 0) return 64 * s + 63 - __builtin_clzll(m);
    }
    return -1;
}


// One Euclidean step on the leading parts: (x, y) -> (y, x - q y) with the
// cofactor rows (A, B), (C, D) -> (C, D), (A - q C, B - q D).  xs is x
// shrunk by 2^-22 relative (computed a step ahead, as y (1 - 2^-22) for the
// next step); the hardware reciprocal of y is within about 2^-24 relative,
// so floor(xs / y estimate) never exceeds the true quotient, and falls short
// of it only for quotients near 2^21 or above, or when x / y is that close
// above an integer (a short quotient leaves a remainder of at least y, which
// the next steps take up).  The quotient is at least 1 whenever x >= y, so
// x = y cannot repeat.  The chain from one divisor to the next is the
// reciprocal, a product, a floor, a maximum and a fused multiply-add.
__device__ __forceinline__ void euclid_step(double x, double xs, double y, double A, double B, double C, double D,
                                            double& ys, double& ny, double& nC, double& nD) {
    const double r = __builtin_amdgcn_rcp(y);
    ys = y * (1.0 - 0x1p-22);
    const double q = fmax(floor(xs * r), x >= y ? 1.0 : 0.0);
    ny = fma(-q, y, x);
    nC = fma(-q, C, A);
    nD = fma(-q, D, B);
}

// Steps of one run on the leading parts: a fixed count, enough for the
// 26 bits of cofactor growth a run takes on average (about fifteen steps).
constexpr int kEuclidRun = 16;

// Waves of a gcd block.  Waves are dealt round-robin to the four SIMDs, so
// waves 0, 4, 8 and 12 share a SIMD: they run the Euclidean steps (wave 0,
// and wave 4 when the block has more than eight components) or stay idle,
// so that the latency-bound Euclid chains never wait behind limb work; every
// other wave holds one component's limbs.  A thirteenth component's limbs
// go to wave 8, on the Euclid waves' SIMD: with that many components a
// launch is bound by the limb waves on the other three SIMDs (four each),
// and the Euclid waves have room.  Up to thirteen components in a
// 1024-thread block.
constexpr int kGcdMaxGroup = 13;
__host__ __device__ constexpr int gcd_limb_wave(int g) { return g < 12 ? g + 1 + g / 3 : 8; }
__host__ __device__ constexpr int gcd_block_waves(int G) { return G <= 12 ? gcd_limb_wave(G - 1) + 1 : 16; }
static_assert(gcd_block_waves(kGcdMaxGroup) == 16, "gcd block layout");

// A block serves G components.  LPC lanes of a Euclid wave serve one
// component (eight, or thirty-two when a block has at most four), lane e
// holding entry e of its window: limbs base + e of a and b, LPC - 2 of them
// handed over by the limb wave with the top limb at entry LPC - 4 (the
// entries above are zero when a window is read).  A matrix updates the
// window lane-parallel, and the leading parts come from three of its
// entries.  Per round the Euclid waves turn each window into KM matrices of
// the component while the limb waves apply those of the round before; one
// barrier per round for the whole block, and per Euclid wave a flag raised
// once all its components are done, so that all waves leave the loop at
// the same barrier.
template <int CW, int GMAX, int LPC, int KM>
__global__ __launch_bounds__(64 * gcd_block_waves(GMAX)) void gcd_kernel(const uint32_t* __restrict__ Y, int nw,
                                                                          const int* __restrict__ status,
                                                                          int valid_rows,
                                                                          const uint32_t* __restrict__ Dw, int nwd,
                                                                          int G, uint64_t* __restrict__ Gout,
                                                                          int* __restrict__ gstat) {
    static_assert((LPC == 8 || LPC == 32) && KM >= 1, "gcd window layout");
    constexpr int kSeg = LPC - 2;       // limbs handed over: h - (kSeg - 2) .. h + 1
    constexpr int kPerWave = 64 / LPC;  // components per Euclid wave
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool lane0 = lane == 0;
    __shared__ int4 sM[2][GMAX][KM];             // round matrices [A B; C D]; all zero: that component is done
    __shared__ int32_t sSeg[2][GMAX][2][LPC];    // the windows of a and b
    __shared__ int sTop[2][GMAX];                // h
    __shared__ int sDone[2][2];                  // per Euclid wave: all its components are done
    __shared__ double2 sRows[2][kEuclidRun + 2][8];  // per Euclid wave: each component's cofactor rows of a run
    const int max_rounds = ((32 * (nw > nwd ? nw : nwd)) / 8 + 64) / KM + 2;
    const int j0 = blockIdx.x * G;
    if (threadIdx.x == 0 && G <= kPerWave) sDone[0][1] = sDone[1][1] = 1;  // no second Euclid wave

    const bool euclid = wave == 0 || (wave == 4 && G > kPerWave);
    const bool limb12 = wave == gcd_limb_wave(12) && G > 12;  // the thirteenth component's limb wave
    if ((wave & 3) == 0 && !euclid && !limb12) {
        // ---- idle wave: keeps the Euclid waves' SIMD free; joins the barriers
        __syncthreads();
        for (int r = 1;; r++) {
            __syncthreads();
            if (sDone[r & 1][0] & sDone[r & 1][1]) break;
        }
        return;
    }
    if (!euclid) {
        // ---- limb wave of component g: a = d, b = y as 30-bit chunks of
        // the two's-complement words (y's sign extended through every
        // limb), then one split pass makes them signed limbs; the carry
        // dropped off the top limb removes the extension
        const int g = limb12 ? 12 : wave - 1 - wave / 4;
        const int j = j0 + g;
        const bool valid = g < G && j < valid_rows && status[j] < 2;
        const uint32_t ext = valid && status[j] == 1 ? 0xffffffffu : 0u;
        const uint32_t* yj = Y + (size_t)(valid ? j : 0) * nw;
        int32_t a[CW], b[CW];
#pragma unroll
        for (int c = 0; c < CW; c++) {
            a[c] = valid ? chunk30(Dw, nwd, 0u, 64 * c + lane) : 0;
            b[c] = valid ? chunk30(yj, nw, ext, 64 * c + lane) : 0;
        }
        limb_apply<CW>(a, b, 1, 0, 0, 1, CW, lane0);
        int ns = CW, hprev = 64 * CW - 1;
        // the top h (at most one limb above the last one: a matrix entry is
        // below 2^26, and the numbers only shrink) and the limbs
        // h - (kSeg - 2) .. h + 1 (zero below limb 0): the lane holding limb
        // k0 + e writes entry e, from slot k >> 6, which is one of the two
        // slots the window touches.  ns covers limb h + 1 for every matrix
        // until the next hand-over.
        auto hand_over = [&](int buf) {
            const int h = __builtin_amdgcn_readfirstlane(top_limb<CW>(a, b, min(CW - 1, (hprev + 1) >> 6)));
            hprev = h;
            ns = h < 0 ? 1 : min(CW, (h + 1) / 64 + 1);
            const int k0 = h - (kSeg - 2);
            const int e = (lane - k0) & 63;
            const int k = k0 + e;
            const int slo = k0 < 0 ? 0 : k0 >> 6, shi = (h + 1) >> 6;
            const int32_t alo = a[slo], ahi = a[min(shi, CW - 1)], blo = b[slo], bhi = b[min(shi, CW - 1)];
            if (e < kSeg) {
                const bool up = (k >> 6) != slo;
                sSeg[buf][g][0][e] = k < 0 ? 0 : (up ? ahi : alo);
                sSeg[buf][g][1][e] = k < 0 ? 0 : (up ? bhi : blo);
            }
            if (lane0) sTop[buf][g] = h;
        };
        if (valid) hand_over(0);
        __syncthreads();
        bool alive = valid;
        for (int r = 1;; r++) {
            __syncthreads();  // matrices r are ready (and the windows after matrices r - 1 were read)
            if (sDone[r & 1][0] & sDone[r & 1][1]) break;
            if (!alive) continue;
            for (int i = 0; i < KM; i++) {
                const int4 m = sM[r & 1][g][i];
                const int32_t A = __builtin_amdgcn_readfirstlane(m.x), B = __builtin_amdgcn_readfirstlane(m.y);
                const int32_t C = __builtin_amdgcn_readfirstlane(m.z), D = __builtin_amdgcn_readfirstlane(m.w);
                if ((A | B | C | D) == 0) {
                    alive = false;
                    break;
                }
                if (!(A == 1 && B == 0 && C == 0 && D == 1)) limb_apply<CW>(a, b, A, B, C, D, ns, lane0);
            }
            if (alive) hand_over(r & 1);
        }
        return;
    }

    // ---- Euclid wave ew: lane LPC q + e serves component g = kPerWave ew +
    // q, entry e of its window.  Every value below is uniform over a
    // component's lanes.
    __builtin_amdgcn_s_setprio(3);
    const int ew = wave >> 2, q = lane / LPC, e = lane % LPC;
    const int g = kPerWave * ew + q;
    const int j = j0 + g;
    bool stopped = !(g < G && j < valid_rows);
    if (!stopped && status[j] >= 2) {
        if (e == 0) gstat[j] = 1;  // outside the bound: the host reconstructs it
        stopped = true;
    }
    // whether this lane's component is reconstructed here (its result is
    // written when the loop ends)
    const bool live0 = !stopped;
    __syncthreads();  // the windows after the split are in buffer 0
    int32_t wa = 0, wb = 0;
    int base = 0;
    int lo = 0;  // low entries of the window made inexact by the matrices applied to it
    // lanes of no component read those of the last one (and ignore them)
    const int gl = g < GMAX ? g : GMAX - 1;
    auto read_window = [&](int buf) {
        const int ee = e < kSeg ? e : kSeg - 1;
        const int32_t va = sSeg[buf][gl][0][ee], vb = sSeg[buf][gl][1][ee];
        wa = e < kSeg ? va : 0;
        wb = e < kSeg ? vb : 0;
        base = sTop[buf][gl] - (kSeg - 2);
        lo = 0;
    };
    // entry x of this component's window (x in 0 .. LPC - 1)
    auto entry = [&](int32_t v, int x) { return __shfl(v, LPC * q + x); };
    // the window after matrix (m0 m1; m2 m3): limb k changes from limbs k
    // and k - 1 only, so the lowest entry lacks the high part entering from
    // below and one more entry becomes inexact; an identity or a zero matrix
    // (a stopped component) leaves it as it is
    auto window_update = [&](int32_t m0, int32_t m1, int32_t m2, int32_t m3) {
        const bool moved = !((m0 == 1) & (m1 == 0) & (m2 == 0) & (m3 == 1)) & ((m0 | m1 | m2 | m3) != 0);
        const int64_t va = (int64_t)m0 * wa + ((int64_t)m1 * wb + (1 << 29));
        const int64_t vb = (int64_t)m2 * wa + ((int64_t)m3 * wb + (1 << 29));
        const int32_t ha = (int32_t)(va >> 30), hb = (int32_t)(vb >> 30);
        int32_t ia, ib;
        if (LPC <= 16) {
            ia = __builtin_amdgcn_update_dpp(0, ha, 0x111, 0xf, 0xf, false);  // row_shr:1
            ib = __builtin_amdgcn_update_dpp(0, hb, 0x111, 0xf, 0xf, false);
        } else {
            ia = wave_ror1(ha);
            ib = wave_ror1(hb);
        }
        const int32_t na = e <= kSeg ? (int32_t)((uint32_t)va & 0x3fffffffu) - (1 << 29) + (e == 0 ? 0 : ia) : 0;
        const int32_t nb = e <= kSeg ? (int32_t)((uint32_t)vb & 0x3fffffffu) - (1 << 29) + (e == 0 ? 0 : ib) : 0;
        wa = moved ? na : wa;
        wb = moved ? nb : wb;
        lo += moved ? 1 : 0;
    };
    // The leading parts from limbs h, h - 1, h - 2 (entries top .. top - 2)
    // and a run of Euclidean steps on them.  The leading parts' signs start
    // the cofactor matrix, so the steps run on magnitudes.  Rows R_0 =
    // (A, B) and R_1 = (C, D) start the run, step k divides by y_{k-1} and
    // makes R_{k+1} = R_{k-1} - q_k R_k, and k steps give the matrix
    // (R_k; R_{k+1}).  k steps are acceptable when the divisors of steps
    // k - 1 and k are at least 2^26 and rows k and k + 1 stay below 2^26.
    // The rows need no test of their own: with q >= 0 throughout the signs
    // of each column alternate down the rows, so that |R_{k+1}| y_{k-1} +
    // |R_k| y_k keeps its starting value x or y (below 2^52) and a divisor
    // of at least 2^26 bounds the rows next to it by 2^26.  Every divisor is
    // at most the one two steps before it, so the acceptable runs are those
    // whose divisors so far are all at least 2^26; J counts them while the
    // steps run, in vector registers, and the steps' rows go to LDS, the
    // accepted pair read back at the end (rows 0 and 1 when J = 0).
    auto euclid_run = [&](int top, int& J, int32_t& m0, int32_t& m1, int32_t& m2, int32_t& m3) {
        const double fa = fma(fma((double)entry(wa, top), 0x1p30, (double)entry(wa, top - 1)), 0x1p30,
                              (double)entry(wa, top - 2));
        const double fb = fma(fma((double)entry(wb, top), 0x1p30, (double)entry(wb, top - 1)), 0x1p30,
                              (double)entry(wb, top - 2));
        int ex;
        (void)frexp(fmax(fabs(fa), fabs(fb)), &ex);
        double x = floor(ldexp(fabs(fa), 52 - ex)), y = floor(ldexp(fabs(fb), 52 - ex));
        double xs = x * (1.0 - 0x1p-22);
        double A = fa < 0.0 ? -1.0 : 1.0, B = 0.0, C = 0.0, D = fb < 0.0 ? -1.0 : 1.0;
        sRows[ew][0][q] = make_double2(A, B);
        sRows[ew][1][q] = make_double2(C, D);
        J = 0;
        double ymin = y;
#pragma unroll
        for (int k = 1; k <= kEuclidRun; k++) {
            ymin = fmin(ymin, y);
            J += ymin >= 0x1p26 ? 1 : 0;
            double ys, ny, nC, nD;
            euclid_step(x, xs, y, A, B, C, D, ys, ny, nC, nD);
            sRows[ew][k + 1][q] = make_double2(nC, nD);
            x = y, xs = ys, y = ny;
            A = C, B = D, C = nC, D = nD;
        }
        const double2 r0 = sRows[ew][J][q], r1 = sRows[ew][J + 1][q];
        m0 = (int32_t)r0.x;
        m1 = (int32_t)r0.y;
        m2 = (int32_t)r1.x;
        m3 = (int32_t)r1.y;
    };
    if (!stopped) read_window(0);
    // the component's result, written when the loop ends: 0 with the gcd in
    // gv, or 1 (the host finishes it)
    int result = 1;
    uint64_t gv = 0;
    const bool writer = e == 0 && g < G;  // the lane that issues the component's matrices
    // the matrices issued last round (applied by now to the limbs, and to
    // the window after the barrier)
    int32_t Mp[KM][4];
#pragma unroll
    for (int i = 0; i < KM; i++) Mp[i][0] = 1, Mp[i][1] = 0, Mp[i][2] = 0, Mp[i][3] = 1;
    bool idle = __ballot(!stopped) == 0;  // every component of the wave is done (its zero matrices issued)
    for (int r = 1;; r++) {
        bool pend = false;  // the last limbs are in view and exact: the gcd from them, after the matrices
        if (!idle) {
            // the window handed over trails by the matrices issued last round
#pragma unroll
            for (int i = 0; i < KM; i++) window_update(Mp[i][0], Mp[i][1], Mp[i][2], Mp[i][3]);
#pragma unroll
            for (int i = 0; i < KM; i++) {
                // (bitwise operators: no branch on the lane masks)
                const uint64_t nzm = __ballot(!stopped & ((wa | wb) != 0) & (e >= lo) & (e <= kSeg));
                const uint64_t gb = (nzm >> (LPC * q)) & (LPC == 64 ? ~0ull : ((1ull << LPC) - 1));
                const int top = gb ? 63 - __builtin_clzll(gb) : -1;  // entry of the top limb
                const int h = base + top;
                // no progress in sight, no limb in view or no headroom left: the host finishes
                const bool c_stop = (r > max_rounds) | (top < 0) | (h >= 64 * CW - 3);
                const bool c_exact = (h <= 3) & (base + lo <= 0);
                // the window lacks the limbs the leading parts (or the last four
                // limbs) need: the identity, and a fresh window next round
                const bool c_ident = (top - 2 < lo) | (h <= 3);
                // every lane takes the run (lanes of stopped or other cases drop it)
                int J;
                int32_t m0, m1, m2, m3;
                euclid_run(top < 2 ? 2 : (top > LPC - 1 ? LPC - 1 : top), J, m0, m1, m2, m3);
                const bool live = !stopped & !c_stop;
                const bool exact = live & c_exact;
                const bool main = live & !c_exact;
                const bool go = main & !c_ident & (J > 0);
                const bool idn = main & c_ident;
                const int32_t n0 = go ? m0 : (idn ? 1 : 0), n1 = go ? m1 : 0;
                const int32_t n2 = go ? m2 : 0, n3 = go ? m3 : (idn ? 1 : 0);
                pend = pend | exact;
                // stopped: the host finishes (result 1), or the exact gcd below
                stopped = stopped | c_stop | exact | (main & !c_ident & (J == 0));
                if (writer) sM[r & 1][g][i] = make_int4(n0, n1, n2, n3);
                Mp[i][0] = n0, Mp[i][1] = n1, Mp[i][2] = n2, Mp[i][3] = n3;
                if (i + 1 < KM) window_update(n0, n1, n2, n3);
            }
        }
        if (__ballot(pend) != 0 && pend) {
            // exact values from limbs 0..3, then the binary gcd (entries past
            // LPC - 1 are above the top and zero)
            __int128 xa = 0, xb = 0;
#pragma unroll
            for (int k = 3; k >= 0; k--) {
                const int x = k - base;
                const int32_t la = entry(wa, x < LPC ? x : LPC - 1), lb = entry(wb, x < LPC ? x : LPC - 1);
                xa = xa * (1 << 30) + (x < LPC ? la : 0);
                xb = xb * (1 << 30) + (x < LPC ? lb : 0);
            }
            unsigned __int128 u = (unsigned __int128)(xa < 0 ? -xa : xa);
            unsigned __int128 v = (unsigned __int128)(xb < 0 ? -xb : xb);
            auto ctz = [](unsigned __int128 x) -> int {
                const uint64_t lo64 = (uint64_t)x;
                return lo64 ? __builtin_ctzll(lo64) : 64 + __builtin_ctzll((uint64_t)(x >> 64));
            };
            if (u == 0) {
                u = v;
            } else if (v != 0) {
                const int sh = ctz(u | v);
                u >>= ctz(u);
                do {
                    v >>= ctz(v);
                    if (u > v) {
                        const unsigned __int128 t = u;
                        u = v;
                        v = t;
                    }
                    v -= u;
                } while (v != 0);
                u <<= sh;
            }
            if ((uint64_t)(u >> 64) == 0) {
                gv = (uint64_t)u;
                result = 0;
            }
        }
        idle = __ballot(!stopped) == 0;
        if (lane0) sDone[r & 1][ew] = idle ? 1 : 0;
        __syncthreads();  // matrices r are ready; the windows after matrices r - 1 are ready
        if (sDone[r & 1][0] & sDone[r & 1][1]) break;
        // the windows handed over after matrices r - 1 (read by every lane;
        // those of stopped components are not used); the next iteration
        // applies matrices r to them
        read_window((r & 1) ^ 1);
    }
    if (writer && live0) {
        gstat[j] = result;
        Gout[j] = gv;
    }
}

// ---------------------------------------------------------------- numerators
// One wave per component, lane l holding words [l CW, l CW + CW) of
// V = sum_col (V[j][col] + 128 rowsum_j) 256^col (the +128 undoes the -128
// offset of the weights).  t = round(V / M) comes from the twelve top columns
// in double precision, read by every lane in the same order (exact whenever
// |V - t M| is far below M / 2, as for every acceptable numerator); then
// y = V - t M word by word with a lane-local carry chain and the wave carry.
// status[j]: 0 when 0 <= y < 2^nbits, 1 when -2^nbits <= y < 0 (Y[j] holds
// words 0 .. nbits / 32 of y, two's complement), 2 otherwise (the host
// reconstructs that component alone).
// Adds the lane-local carries out (cout, signed) into the next lanes.
template <int CW>
__device__ __forceinline__ void wave_carry(uint32_t (&R)[CW], int64_t cout, int lane) {
    int64_t cin = __shfl_up(cout, 1);
    if (lane == 0) cin = 0;
    for (;;) {
#pragma unroll
        for (int c = 0; c < CW; c++) {
            const int64_t v = (int64_t)R[c] + cin;
            R[c] = (uint32_t)v;
            cin = v >> 32;
        }
        int64_t up = __shfl_up(cin, 1);
        if (lane == 0) up = 0;
        if (__ballot(up != 0) == 0) break;
        cin = up;
    }
}

template <int CW>
__global__ __launch_bounds__(256) void numer_kernel(const int* __restrict__ V, int Ncolsp,
                                                    const int* __restrict__ rowsum, int valid_rows,
                                                    const uint32_t* __restrict__ Mw, int TM, double Mtop, int nbits,
                                                    uint32_t* __restrict__ Y, int* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= valid_rows) return;
    const int64_t off = 128 * (int64_t)rowsum[j];
    const int NW = TM + 1;
    const int hw = nbits / 32, hb = nbits % 32, nw = hw + 1;
    const int* vj = V + (size_t)j * Ncolsp;
    double va = 0.0;  // V / 2^(32 (TM - 2)) from the columns of words TM - 2 .. TM
    for (int cidx = 4 * NW - 1; cidx >= 4 * (TM - 2); cidx--) va = va * 256.0 + (double)((int64_t)vj[cidx] + off);
    const int64_t t = (int64_t)rint(va / Mtop);
    uint32_t y[CW];
    int64_t carry = 0;
#pragma unroll
    for (int c = 0; c < CW; c++) {
        const int w = lane * CW + c;
        int64_t acc = carry;
        if (w < NW) {
            const int4 v4 = *(const int4*)(vj + 4 * w);
            acc += ((int64_t)v4.x + off) + ((int64_t)v4.y + off) * 256 + ((int64_t)v4.z + off) * 65536 +
                   ((int64_t)v4.w + off) * 16777216 - t * (int64_t)Mw[w];
        }
        y[c] = (uint32_t)acc;
        carry = acc >> 32;
    }
    wave_carry<CW>(y, carry, lane);
    // sign: the top word of the wave's 64 CW words
    const uint32_t sw = ((uint32_t)__builtin_amdgcn_readlane((int)y[CW - 1], 63) >> 31) ? 0xffffffffu : 0u;
    bool ok = true;
#pragma unroll
    for (int c = 0; c < CW; c++) {
        const int w = lane * CW + c;
        if (w > hw) ok = ok && y[c] == sw;
        if (w == hw) ok = ok && (y[c] >> hb) == (sw >> hb);
        if (w < nw) Y[(size_t)j * nw + w] = y[c];
    }
    const bool accept = __ballot(!ok) == 0;
    if (lane == 0) status[j] = accept ? (sw ? 1 : 0) : 2;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_digit_bytes(const uint64_t* digits, int dstride, int m, int j0, int valid_rows, int rows_pad,
                              int Kpad, int8_t* S, int* rowsum, hipStream_t st) {
    es_launch(digit_bytes_kernel, dim3(rows_pad), dim3(256), 0, st, digits, dstride, m, j0, valid_rows,
                       Kpad, S, rowsum);
    return hipGetLastError();
}

hipError_t launch_wchain(const uint32_t* T, const uint32_t* Mw, int m, int TM, double Md, int Ncolsp, uint8_t* W,
                         hipStream_t st) {
    const int NW = TM + 1;
    if (NW <= 64 * 8)
        es_launch(wchain_kernel<8>, dim3(m), dim3(192), 0, st, T, Mw, TM, Md, Ncolsp, W);
    else if (NW <= 64 * 32)
        es_launch(wchain_kernel<32>, dim3(m), dim3(192), 0, st, T, Mw, TM, Md, Ncolsp, W);
    else if (NW <= 64 * 64)
        es_launch(wchain_kernel<64>, dim3(m), dim3(192), 0, st, T, Mw, TM, Md, Ncolsp, W);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

int wchain_words_per_lane(int NW) { return NW <= 64 * 8 ? 8 : NW <= 64 * 32 ? 32 : NW <= 64 * 64 ? 64 : 0; }

hipError_t launch_transpose_offset(const uint8_t* W, int Kpad, int Ncolsp, int8_t* WT, hipStream_t st) {
    es_launch(transpose_offset_kernel, dim3(Ncolsp / 64, Kpad / 64), dim3(256), 0, st, W, Kpad, Ncolsp, WT);
    return hipGetLastError();
}

// Large products: block tile 256 x 256, four waves in a 2 x 2 arrangement,
// each owning 128 x 128 as 8 x 8 MFMA tiles (256 accumulators a lane, one
// wave a SIMD), so a block reads half the operand bytes per product of the
// 128 x 128 kernel, whose operand traffic from L2 bounds it.  The chunks of
// 64 bytes of k go through two LDS buffers.  While chunk k's products run
// (row by row), each fragment register is refilled with chunk k + 1's
// fragment from the other buffer right after its last product (the A
// fragment of row i after that row, the B fragments during the last row),
// so the LDS reads hide behind the products without a second register set;
// chunk k + 2 goes from registers into chunk k's buffer (free since the
// previous barrier) and chunk k + 3 is loaded from memory.  One barrier a
// chunk.  Same operand and output lane layouts as above; rows and columns
// are multiples of 256.
constexpr int kBigTile = 256;
constexpr size_t kBigLds = (size_t)2 * 2 * kBigTile * kGemmLds;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void recon_gemm_big_kernel(
    const int8_t* __restrict__ S, const int8_t* __restrict__ WT, int Kpad, int Ncolsp, int* __restrict__ V) {
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    int8_t* As = lds;                               // [2][256][kGemmLds]
    int8_t* Bs = lds + 2 * kBigTile * kGemmLds;     // [2][256][kGemmLds]
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int j0 = blockIdx.x * kBigTile, c0 = blockIdx.y * kBigTile;
    const int lr = lane & 15, lg = lane >> 4;
    // global -> registers -> LDS: thread t moves rows t / 4 + 64 q (q < 4),
    // 16-byte piece t % 4, of both operands
    const int gr = t >> 2, gc = (t & 3) * 16;
    const int8_t* Ag = S + (size_t)(j0 + gr) * Kpad + gc;
    const int8_t* Bg = WT + (size_t)(c0 + gr) * Kpad + gc;
    const size_t q64 = (size_t)64 * Kpad;
    const int nk = Kpad / 64;
    v4i ra[4], rb[4];
    // past the last chunk a load repeats the last chunk (never used)
    auto gload = [&](int kc) {
        kc = min(kc, nk - 1);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            ra[q] = *(const v4i*)(Ag + q * q64 + 64 * kc);
            rb[q] = *(const v4i*)(Bg + q * q64 + 64 * kc);
        }
    };
    auto lstore = [&](int buf) {
        int8_t* a = As + buf * kBigTile * kGemmLds;
        int8_t* b = Bs + buf * kBigTile * kGemmLds;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            *(v4i*)(a + (gr + 64 * q) * kGemmLds + gc) = ra[q];
            *(v4i*)(b + (gr + 64 * q) * kGemmLds + gc) = rb[q];
        }
    };
    // this wave's fragment rows in buffer `buf`
    auto afrag = [&](int buf, int i) {
        return *(const v4i*)(As + buf * kBigTile * kGemmLds + (128 * wr + 16 * i + lr) * kGemmLds + 16 * lg);
    };
    auto bfrag = [&](int buf, int i) {
        return *(const v4i*)(Bs + buf * kBigTile * kGemmLds + (128 * wc + 16 * i + lr) * kGemmLds + 16 * lg);
    };
    v4i acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; a++)
#pragma unroll
        for (int b = 0; b < 8; b++) acc[a][b] = v4i{0, 0, 0, 0};
    v4i fa[8], fb[8];
    gload(0);
    lstore(0);
    gload(1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; i++) fa[i] = afrag(0, i);
#pragma unroll
    for (int i = 0; i < 8; i++) fb[i] = bfrag(0, i);
    lstore(1);
    gload(2);
    __syncthreads();
    // entering chunk kc: its fragments in fa / fb, chunk kc + 1 in buffer
    // (kc + 1) & 1, chunk kc + 2 in ra / rb
    for (int kc = 0; kc < nk; kc++) {
        const int cur = kc & 1, nxt = cur ^ 1;
        if (kc + 2 < nk) lstore(cur);
        gload(kc + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 7; i++) {
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                acc[i][jj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[jj], acc[i][jj], 0, 0, 0);
            fa[i] = afrag(nxt, i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
            acc[7][jj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[7], fb[jj], acc[7][jj], 0, 0, 0);
            fb[jj] = bfrag(nxt, jj);
            __builtin_amdgcn_sched_barrier(0);
        }
        fa[7] = afrag(nxt, 7);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
            const int col = c0 + 128 * wc + 16 * jj + lr;
            const int j = j0 + 128 * wr + 16 * i + 4 * lg;
#pragma unroll
            for (int r = 0; r < 4; r++) V[(size_t)(j + r) * Ncolsp + col] = acc[i][jj][r];
        }
}

hipError_t launch_recon_gemm(const int8_t* S, const int8_t* WT, int Kpad, int NCcp, int Ncolsp, int* V,
                             hipStream_t st) {
    if (NCcp % 128 != 0 || Ncolsp % 128 != 0 || Kpad % 64 != 0) return hipErrorInvalidValue;
    // the 256 x 256 tiles once they give every CU two blocks or more
    static int big_ok = -1;
    if (big_ok < 0)
        big_ok = hipFuncSetAttribute((const void*)recon_gemm_big_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kBigLds) == hipSuccess
                     ? 1
                     : 0;
    (void)hipGetLastError();
    const int cus = device_cus();
    if (big_ok && cus > 0 && NCcp % kBigTile == 0 && Ncolsp % kBigTile == 0 &&
        (long)(NCcp / kBigTile) * (Ncolsp / kBigTile) >= 2L * cus) {
        // component tiles vary fastest, so the blocks in flight share weight tiles
        es_launch(recon_gemm_big_kernel, dim3(NCcp / kBigTile, Ncolsp / kBigTile), dim3(256), kBigLds, st, S, WT,
                  Kpad, Ncolsp, V);
        return hipGetLastError();
    }
    const int nx = NCcp / 128, tiles = nx * (Ncolsp / 128);
    es_launch(recon_gemm_kernel, dim3((tiles + 7) / 8 * 8), dim3(256), 0, st, S, WT, Kpad, Ncolsp, V, nx, tiles);
    return hipGetLastError();
}

// Limb slots per lane for numbers of up to `words` 32-bit words: 30-bit
// limbs with three limbs of headroom for the cofactor products
// (|A a + B b| < 2^27 max(|a|, |b|)).
int gcd_words_per_lane(int words) {
    const int limbs = (32 * words + 29) / 30 + 3;
    return limbs <= 64 * 8 ? 8 : limbs <= 64 * 16 ? 16 : limbs <= 64 * 32 ? 32 : 0;
}

// Compute units of the current device (0 if the device does not say).
static int device_cus() {
    static int cus = -1;
    if (cus < 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
    }
    return cus;
}

// Unused dynamic LDS per gcd block that caps the blocks a CU can hold at
// ceil(blocks / CUs): the components are latency-bound chains, and an even
// spread keeps every CU at the same small number of them.  Above 48 KB the
// kernel's dynamic LDS limit is raised first; zero when the device does not
// say or does not allow it.
static size_t gcd_lds_pad(const void* kernel, int blocks) {
    static int lds_cu = -1, lds_blk = 0;
    if (lds_cu < 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds_blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            lds_cu = 0;
    }
    const int cus = device_cus();
    if (cus <= 0 || lds_cu <= 0 || blocks <= 0) return 0;
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, kernel) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    // the kernel's own LDS, with a kilobyte of room for allocation granules
    const int own = (int)((fa.sharedSizeBytes + 1023) / 1024 * 1024) + 1024;
    const int cap = (blocks + cus - 1) / cus;
    const int pad = lds_cu / cap - own;
    if (pad <= 0 || pad + own > lds_blk) return 0;
    if (pad > 48 * 1024 && hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, pad) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return (size_t)pad;
}

// Components per gcd block: the components spread evenly over the compute
// units, at most gmax per block (gmax + 1 waves must fit one CU).  Three or
// four components per CU go as two blocks of two (each Euclid wave then
// waits for two components' runs, not four: 0.13 ms less at n = 1024).
static int gcd_group(int rows, int gmax) {
    const int cus = device_cus();
    int G = cus > 0 ? (rows + cus - 1) / cus : 4;
    if (G > 2 && G <= 4) G = 2;
    return G < 1 ? 1 : (G > gmax ? gmax : G);
}

// Blocks of at most kGcdWideGroup components take the wide windows
// (thirty-two lanes a component, four matrices a round): with few
// components per CU each Euclid chain's rounds set the time, and a round's
// barrier and hand-over then serve four matrices.
constexpr int kGcdWideGroup = 4;

// Waves of a gcd block of grp components: a wide block of more than two
// components has its second Euclid wave at wave 4.
static int gcd_waves(int grp) {
    const int w = gcd_block_waves(grp);
    return grp <= kGcdWideGroup && grp > 2 && w < 5 ? 5 : w;
}

// The gcd kernel for CW limb slots and a group of grp components.
template <int CW>
static const void* gcd_kernel_for(int grp) {
    return grp <= kGcdWideGroup ? (const void*)gcd_kernel<CW, kGcdWideGroup, 32, 4>
                                : (const void*)gcd_kernel<CW, kGcdMaxGroup, 8, 1>;
}

template <int CW>
static void launch_gcd_as(const uint32_t* Y, int nw, const int* status, int valid_rows, const uint32_t* Dw,
                          int nwd, uint64_t* G, int* gstat, int group, hipStream_t st) {
    const int grp = group > 0 ? group : gcd_group(valid_rows, kGcdMaxGroup);
    const int blocks = (valid_rows + grp - 1) / grp;
    const int waves = gcd_waves(grp);
    const size_t pad = gcd_lds_pad(gcd_kernel_for<CW>(grp), blocks);
    static const bool verbose = [] {
        const char* e = std::getenv("ES_VERBOSE");
        return e && *e && *e != '0';
    }();
    if (verbose)
        fprintf(stderr, "[es] gcd: %d components, %d per block, %d blocks, %zu bytes of LDS padding, %d slots\n",
                valid_rows, grp, blocks, pad, CW);
    if (grp <= kGcdWideGroup)
        es_launch(gcd_kernel<CW, kGcdWideGroup, 32, 4>, dim3(blocks), dim3(64 * waves), pad, st, Y, nw, status,
                  valid_rows, Dw, nwd, grp, G, gstat);
    else
        es_launch(gcd_kernel<CW, kGcdMaxGroup, 8, 1>, dim3(blocks), dim3(64 * waves), pad, st, Y, nw, status,
                  valid_rows, Dw, nwd, grp, G, gstat);
}

hipError_t launch_gcd(const uint32_t* Y, int nw, const int* status, int valid_rows, const uint32_t* Dw, int nwd,
                      uint64_t* G, int* gstat, int group, hipStream_t st) {
    const int cw = gcd_words_per_lane(nw > nwd ? nw : nwd);
    if (valid_rows <= 0) return hipSuccess;
    if (group > kGcdMaxGroup) return hipErrorInvalidValue;
    if (cw == 8)
        launch_gcd_as<8>(Y, nw, status, valid_rows, Dw, nwd, G, gstat, group, st);
    else if (cw == 16)
        launch_gcd_as<16>(Y, nw, status, valid_rows, Dw, nwd, G, gstat, group, st);
    else if (cw == 32)
        launch_gcd_as<32>(Y, nw, status, valid_rows, Dw, nwd, G, gstat, group, st);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Blocks of the gcd kernel one CU holds at once (waves and registers; the
// LDS padding only lowers it further); 0 when the device does not say.
template <int CW>
static int gcd_blocks_per_cu(int grp) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gcd_kernel_for<CW>(grp), 64 * gcd_waves(grp), 0) !=
        hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return nb;
}

int gcd_split(int valid_rows, int nw, int nwd, int* group) {
    const int cw = gcd_words_per_lane(nw > nwd ? nw : nwd);
    const int grp = gcd_group(valid_rows, kGcdMaxGroup);
    *group = grp;
    const int per_cu = cw == 8    ? gcd_blocks_per_cu<8>(grp)
                       : cw == 16 ? gcd_blocks_per_cu<16>(grp)
                       : cw == 32 ? gcd_blocks_per_cu<32>(grp)
                                  : 0;
    const int cus = device_cus();
    if (valid_rows <= 0 || per_cu <= 0 || cus <= 0) return valid_rows;
    const long per_round = (long)cus * per_cu;  // blocks resident at once
    const long blocks = (valid_rows + grp - 1) / grp;
    const long rounds = (blocks + per_round - 1) / per_round;
    if (rounds < 4) return valid_rows;
    const long second = rounds >= 10 ? rounds / 5 : 1;
    return (int)((rounds - second) * per_round * grp);
}

int numer_words_per_lane(int NW) {
    NW += 2;  // the result's sign word and one word of headroom
    return NW <= 64 * 8 ? 8 : NW <= 64 * 16 ? 16 : NW <= 64 * 32 ? 32 : NW <= 64 * 64 ? 64 : 0;
}

hipError_t launch_numer(const int* V, int Ncolsp, const int* rowsum, int valid_rows, const uint32_t* Mw, int TM,
                        double Mtop, int nbits, uint32_t* Y, int* status, hipStream_t st) {
    const dim3 grid((valid_rows + 3) / 4);
    switch (numer_words_per_lane(TM + 1)) {
        case 8:
            es_launch(numer_kernel<8>, grid, dim3(256), 0, st, V, Ncolsp, rowsum, valid_rows, Mw, TM, Mtop,
                               nbits, Y, status);
            break;
        case 16:
            es_launch(numer_kernel<16>, grid, dim3(256), 0, st, V, Ncolsp, rowsum, valid_rows, Mw, TM, Mtop,
                               nbits, Y, status);
            break;
        case 32:
            es_launch(numer_kernel<32>, grid, dim3(256), 0, st, V, Ncolsp, rowsum, valid_rows, Mw, TM, Mtop,
                               nbits, Y, status);
            break;
        case 64:
            es_launch(numer_kernel<64>, grid, dim3(256), 0, st, V, Ncolsp, rowsum, valid_rows, Mw, TM, Mtop,
                               nbits, Y, status);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace es
