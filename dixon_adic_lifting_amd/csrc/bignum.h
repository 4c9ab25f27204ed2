// Host arbitrary-precision integers for the reconstruction stage.
//
// Sign-magnitude, 64-bit little-endian limbs.  Multiplication is schoolbook
// below a threshold and Karatsuba (1962) above; division is Knuth's
// Algorithm D (TAOCP vol. 2, 4.3.1); gcd and the extended Euclidean steps of
// rational reconstruction use Lehmer's method (Knuth 4.5.2, Algorithm L)
// with single-word simulation of the quotient sequence.
#pragma once
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace es {

using limb_t = uint64_t;

struct BigInt {
    std::vector<limb_t> d;  // magnitude, no leading zero limbs; empty = 0
    bool neg = false;       // never true for zero

    BigInt() = default;
    static BigInt from_i64(int64_t v);
    static BigInt from_u64(uint64_t v);
    // value of a little-endian two's-complement integer of `nlimbs` limbs
    static BigInt from_twos(const limb_t* w, size_t nlimbs);

    bool is_zero() const { return d.empty(); }
    size_t size() const { return d.size(); }
    size_t bit_length() const;
    void trim();
    std::string to_hex() const;  // "-1f", "0", ...
};

int cmp_abs(const BigInt& a, const BigInt& b);
int cmp(const BigInt& a, const BigInt& b);

BigInt add(const BigInt& a, const BigInt& b);
BigInt sub(const BigInt& a, const BigInt& b);
BigInt mul(const BigInt& a, const BigInt& b);
BigInt mul_small(const BigInt& a, int64_t s);
// truncated division: q = trunc(a / b), r = a - q b (sign of a); b != 0
void divmod_trunc(const BigInt& a, const BigInt& b, BigInt* q, BigInt* r);
// r = a mod m in [0, m) for m > 0
BigInt mod_floor(const BigInt& a, const BigInt& m);
BigInt divexact(const BigInt& a, const BigInt& b);  // a / b, exact (checked)
BigInt divexact_u64(const BigInt& a, uint64_t b);  // a / b for 0 < b < 2^64, exact (checked)
void divexact_u64_inplace(BigInt& a, uint64_t b);  // a <- a / b, exact (checked; a unspecified on a throw)
BigInt shl(const BigInt& a, size_t bits);
BigInt shr_abs(const BigInt& a, size_t bits);       // |a| >> bits
BigInt pow_u(const BigInt& a, unsigned e);

BigInt gcd(const BigInt& a, const BigInt& b);       // >= 0
BigInt lcm(const BigInt& a, const BigInt& b);       // >= 0

// Wang's rational reconstruction: the unique num/den with num == a * den
// (mod M), |num| <= N, 0 < den <= D, gcd(num, den) = 1, given 2 N D < M and
// 0 <= a < M.  Returns false if there is none.  With require_coprime false
// the final gcd(num, den) = 1 test is skipped: the result is then the
// remainder / cofactor pair where the Euclidean sequence first drops to N,
// whose den is the true denominator whenever such a fraction exists.
// split_cofactors runs the cofactor updates on a second thread (worth it for
// long inputs when cores are idle).
bool rational_reconstruct(const BigInt& a, const BigInt& M, const BigInt& N,
                          const BigInt& D, BigInt* num, BigInt* den, bool require_coprime = true,
                          bool split_cofactors = false);

// low-level magnitude routines (exposed for tests)
void mag_mul(limb_t* r, const limb_t* a, size_t la, const limb_t* b, size_t lb);
void mag_divmod(limb_t* q, limb_t* r, const limb_t* a, size_t la, const limb_t* b, size_t lb);

}  // namespace es
