// Host-side stages of the solver: workspace layout, prime-set selection and
// lift constants, bounds and step count, the singularity decision, and the
// rational reconstruction.
#pragma once
#include <cstdint>
#include <functional>
#include <vector>

#include "bignum.h"
#include "es_internal.h"

namespace es {

struct SolutionData {
    int n = 0, c = 0;
    std::vector<BigInt> num;  // [n*c], lowest terms
    // the denominators (> 0): component j's is dens[den_of[j]], so that the
    // components sharing one (most of them, as a rule) share its limbs
    std::vector<BigInt> dens;
    std::vector<uint32_t> den_of;  // [n*c]
    const BigInt& den(size_t j) const { return dens[den_of[j]]; }
    int live = 0, m = 0, nbits = 0, dbits = 0;
    int mbits = 0;  // bit length of M = P^m
};

// Live prime set: indices into the 53-prime table, ascending.
struct LiveSet {
    int E = 0;
    int idx[kNumPrimes];
    BigInt P;
    uint64_t Pinv = 0;  // P^-1 mod 2^64
};

LiveSet make_live_set(const int* flags);       // flags[j] != 0 drops prime j
LiveSet live_set_from_mask(uint64_t mask);
void fill_lift_params(const LiveSet& ls, LiftParams* prm);

// Bit sizes of the Hadamard bounds from the squared row/column norms of A and
// the squared column norms of b (fp64 sums, rounded up with a margin).
void hadamard_bits(const double* rownorm, const double* colnorm, const double* bnorm, int n, int c,
                   int* nbits, int* dbits);

// Least m with P^m > 2^(nbits + dbits + 1); also returns M = P^m.
int choose_m(const BigInt& P, int nbits, int dbits, BigInt* M);
// the same m, and the bit length of M = P^m, without forming M
int choose_m_bits(const BigInt& P, int nbits, int dbits, size_t* mbits);

// Exact rank test of A modulo a 62-bit prime (host Gaussian elimination).
bool full_rank_mod(const int64_t* A, int n, uint64_t p);

// digits: int64 [n*c][stride_m][6] (first m used), balanced base-P digits.
// Returns ES_OK or ES_EINTERNAL.
int reconstruct(const int64_t* digits, size_t stride_m, int n, int c, int m, const BigInt& P,
                const BigInt& M, int nbits, int dbits, int nthreads, SolutionData* out);

int default_threads();

// X = sum_{i<m} x_i P^i from one component's digits (int64 [m][6]).
BigInt assemble(const int64_t* dig, int m, const BigInt& P);
// the same from the powers pw[k] = P^k, k <= m (halves joined by one product)
BigInt assemble(const int64_t* dig, int m, const std::vector<BigInt>& pw);
// The same for `count` components (digits dig + k stride), each cut into
// `parts` (a power of two) ranges assembled on the pool's threads and joined
// pairwise: a shorter wait for a few long components.
void assemble_split(const int64_t* dig, size_t stride, size_t count, int m, const std::vector<BigInt>& pw,
                    int parts, int nthreads, BigInt* out);

// Runs fn(i) for i in [0, count) on up to nthreads host threads, the items
// claimed `grain` at a time (0: a quarter of an even share; 1 for items of
// very uneven cost).
void parallel_for_each(size_t count, int nthreads, const std::function<void(size_t)>& fn, size_t grain = 0);

// The sampled common denominator (card, "Method"): d = lcm of the reduced
// denominators of the sample components (the first row, i.e. one component
// of every right-hand side, then the components floor(k NC / 8) + (k mod c)
// for k = 1..7 in row-major order), each found by Wang reconstruction of
// X mod M.  xs[k] is
// the k-th sample's X.  Returns false if some sample has no fraction within
// the bounds.
std::vector<size_t> sample_indices(size_t NC, int c);
bool sample_denominator(const std::vector<BigInt>& xs, const BigInt& M, int nbits, int dbits, int nthreads,
                        BigInt* d);

}  // namespace es
