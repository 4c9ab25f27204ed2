// Host arbitrary-precision integers (see bignum.h for the methods used).
#include "bignum.h"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <exception>
#include <stdexcept>
#include <thread>

namespace es {

typedef unsigned __int128 u128;
typedef __int128 i128;

static const size_t kKaratsuba = 40;  // limbs; below this schoolbook wins

// ------------------------------------------------------------------ basics

BigInt BigInt::from_u64(uint64_t v) {
    BigInt r;
    if (v) r.d.push_back(v);
    return r;
}

BigInt BigInt::from_i64(int64_t v) {
    BigInt r;
    if (v) {
        r.d.push_back(v < 0 ? (uint64_t)0 - (uint64_t)v : (uint64_t)v);
        r.neg = v < 0;
    }
    return r;
}

BigInt BigInt::from_twos(const limb_t* w, size_t nlimbs) {
    BigInt r;
    if (nlimbs == 0) return r;
    bool negative = (w[nlimbs - 1] >> 63) != 0;
    r.d.assign(w, w + nlimbs);
    if (negative) {  // magnitude = ~w + 1
        uint64_t carry = 1;
        for (size_t i = 0; i < nlimbs; i++) {
            u128 s = (u128)(~r.d[i]) + carry;
            r.d[i] = (uint64_t)s;
            carry = (uint64_t)(s >> 64);
        }
        r.neg = true;
    }
    r.trim();
    return r;
}

void BigInt::trim() {
    while (!d.empty() && d.back() == 0) d.pop_back();
    if (d.empty()) neg = false;
}

size_t BigInt::bit_length() const {
    if (d.empty()) return 0;
    return 64 * (d.size() - 1) + (64 - __builtin_clzll(d.back()));
}

std::string BigInt::to_hex() const {
    if (d.empty()) return "0";
    std::string s = neg ? "-" : "";
    char buf[32];
    snprintf(buf, sizeof buf, "%llx", (unsigned long long)d.back());
    s += buf;
    for (size_t i = d.size() - 1; i-- > 0;) {
        snprintf(buf, sizeof buf, "%016llx", (unsigned long long)d[i]);
        s += buf;
    }
    return s;
}

static int mag_cmp(const limb_t* a, size_t la, const limb_t* b, size_t lb) {
    if (la != lb) return la < lb ? -1 : 1;
    for (size_t i = la; i-- > 0;)
        if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
    return 0;
}

int cmp_abs(const BigInt& a, const BigInt& b) {
    return mag_cmp(a.d.data(), a.d.size(), b.d.data(), b.d.size());
}

int cmp(const BigInt& a, const BigInt& b) {
    if (a.neg != b.neg) return a.neg ? -1 : 1;
    int c = cmp_abs(a, b);
    return a.neg ? -c : c;
}

// r = x + y with lx >= ly; r has lx limbs; returns the carry out
static limb_t add_to(limb_t* r, const limb_t* x, size_t lx, const limb_t* y, size_t ly) {
    limb_t carry = 0;
    size_t i = 0;
    for (; i < ly; i++) {
        u128 s = (u128)x[i] + y[i] + carry;
        r[i] = (limb_t)s;
        carry = (limb_t)(s >> 64);
    }
    for (; i < lx; i++) {
        u128 s = (u128)x[i] + carry;
        r[i] = (limb_t)s;
        carry = (limb_t)(s >> 64);
    }
    return carry;
}

// x -= y in place (lx >= ly, x >= y); returns the borrow out (0 when x >= y)
static limb_t sub_in(limb_t* x, size_t lx, const limb_t* y, size_t ly) {
    limb_t borrow = 0;
    size_t i = 0;
    for (; i < ly; i++) {
        limb_t xi = x[i], yi = y[i];
        limb_t t = xi - yi;
        limb_t b1 = xi < yi;
        limb_t t2 = t - borrow;
        limb_t b2 = t < borrow;
        x[i] = t2;
        borrow = b1 | b2;
    }
    for (; borrow && i < lx; i++) {
        limb_t xi = x[i];
        x[i] = xi - 1;
        borrow = xi == 0;
    }
    return borrow;
}

// x += y in place (lx >= ly); returns the carry out
static limb_t add_in(limb_t* x, size_t lx, const limb_t* y, size_t ly) {
    limb_t carry = 0;
    size_t i = 0;
    for (; i < ly; i++) {
        u128 s = (u128)x[i] + y[i] + carry;
        x[i] = (limb_t)s;
        carry = (limb_t)(s >> 64);
    }
    for (; carry && i < lx; i++) {
        x[i] += 1;
        carry = x[i] == 0;
    }
    return carry;
}

// ------------------------------------------------------------------ multiply

static void school_mul(limb_t* r, const limb_t* a, size_t la, const limb_t* b, size_t lb) {
    std::memset(r, 0, (la + lb) * sizeof(limb_t));
    for (size_t i = 0; i < la; i++) {
        const limb_t ai = a[i];
        limb_t carry = 0;
        limb_t* ri = r + i;
        for (size_t j = 0; j < lb; j++) {
            u128 p = (u128)ai * b[j] + ri[j] + carry;
            ri[j] = (limb_t)p;
            carry = (limb_t)(p >> 64);
        }
        ri[lb] = carry;
    }
}

// r[0, 2n) = a * b, both n limbs; ws needs 8n + 64 limbs
static void kara_mul(limb_t* r, const limb_t* a, const limb_t* b, size_t n, limb_t* ws) {
    if (n < kKaratsuba) {
        school_mul(r, a, n, b, n);
        return;
    }
    const size_t h = n / 2, hh = n - h;
    kara_mul(r, a, b, h, ws);                  // z0 = a0 b0 -> r[0, 2h)
    kara_mul(r + 2 * h, a + h, b + h, hh, ws); // z2 = a1 b1 -> r[2h, 2n)
    limb_t* sa = ws;
    limb_t* sb = sa + (hh + 1);
    limb_t* z1 = sb + (hh + 1);
    limb_t* ws2 = z1 + 2 * (hh + 1);
    sa[hh] = add_to(sa, a + h, hh, a, h);
    sb[hh] = add_to(sb, b + h, hh, b, h);
    kara_mul(z1, sa, sb, hh + 1, ws2);         // (a0 + a1)(b0 + b1)
    sub_in(z1, 2 * hh + 2, r, 2 * h);
    sub_in(z1, 2 * hh + 2, r + 2 * h, 2 * hh); // z1 = a0 b1 + a1 b0
    size_t zl = 2 * hh + 2;
    while (zl > 0 && z1[zl - 1] == 0) zl--;
    add_in(r + h, 2 * n - h, z1, zl);
}

void mag_mul(limb_t* r, const limb_t* a, size_t la, const limb_t* b, size_t lb) {
    if (la < lb) {
        std::swap(a, b);
        std::swap(la, lb);
    }
    if (lb == 0) {
        std::memset(r, 0, la * sizeof(limb_t));
        return;
    }
    if (lb < kKaratsuba) {
        school_mul(r, a, la, b, lb);
        return;
    }
    std::vector<limb_t> ws(8 * lb + 64);
    if (la == lb) {
        kara_mul(r, a, b, lb, ws.data());
        return;
    }
    // unbalanced: multiply lb-limb slices of a by b and accumulate
    std::memset(r, 0, (la + lb) * sizeof(limb_t));
    std::vector<limb_t> tmp(2 * lb);
    for (size_t off = 0; off < la; off += lb) {
        size_t len = std::min(lb, la - off);
        if (len == lb) {
            kara_mul(tmp.data(), a + off, b, lb, ws.data());
        } else {
            mag_mul(tmp.data(), b, lb, a + off, len);
        }
        add_in(r + off, la + lb - off, tmp.data(), len + lb);
    }
}

BigInt mul(const BigInt& a, const BigInt& b) {
    BigInt r;
    if (a.is_zero() || b.is_zero()) return r;
    r.d.resize(a.size() + b.size());
    mag_mul(r.d.data(), a.d.data(), a.size(), b.d.data(), b.size());
    r.neg = a.neg != b.neg;
    r.trim();
    return r;
}

BigInt mul_small(const BigInt& a, int64_t s) {
    BigInt r;
    if (a.is_zero() || s == 0) return r;
    uint64_t m = s < 0 ? (uint64_t)0 - (uint64_t)s : (uint64_t)s;
    r.d.resize(a.size() + 1);
    limb_t carry = 0;
    for (size_t i = 0; i < a.size(); i++) {
        u128 p = (u128)a.d[i] * m + carry;
        r.d[i] = (limb_t)p;
        carry = (limb_t)(p >> 64);
    }
    r.d[a.size()] = carry;
    r.neg = a.neg != (s < 0);
    r.trim();
    return r;
}

// ------------------------------------------------------------------ add / sub

static BigInt add_signed(const BigInt& a, const BigInt& b, bool bneg) {
    BigInt r;
    if (b.is_zero()) return a;
    if (a.is_zero()) {
        r = b;
        r.neg = bneg;
        return r;
    }
    if (a.neg == bneg) {
        const BigInt& x = a.size() >= b.size() ? a : b;
        const BigInt& y = a.size() >= b.size() ? b : a;
        r.d.resize(x.size() + 1);
        r.d[x.size()] = add_to(r.d.data(), x.d.data(), x.size(), y.d.data(), y.size());
        r.neg = a.neg;
    } else {
        int c = cmp_abs(a, b);
        if (c == 0) return r;
        const BigInt& x = c > 0 ? a : b;
        const BigInt& y = c > 0 ? b : a;
        r.d = x.d;
        sub_in(r.d.data(), r.d.size(), y.d.data(), y.size());
        r.neg = c > 0 ? a.neg : bneg;
    }
    r.trim();
    return r;
}

BigInt add(const BigInt& a, const BigInt& b) { return add_signed(a, b, b.neg); }
BigInt sub(const BigInt& a, const BigInt& b) { return add_signed(a, b, b.is_zero() ? false : !b.neg); }

// ------------------------------------------------------------------ shifts

BigInt shl(const BigInt& a, size_t bits) {
    BigInt r;
    if (a.is_zero()) return r;
    size_t w = bits / 64, s = bits % 64;
    r.d.assign(a.size() + w + 1, 0);
    for (size_t i = 0; i < a.size(); i++) {
        r.d[i + w] |= a.d[i] << s;
        if (s) r.d[i + w + 1] |= a.d[i] >> (64 - s);
    }
    r.neg = a.neg;
    r.trim();
    return r;
}

BigInt shr_abs(const BigInt& a, size_t bits) {
    BigInt r;
    size_t w = bits / 64, s = bits % 64;
    if (w >= a.size()) return r;
    r.d.assign(a.size() - w, 0);
    for (size_t i = 0; i < r.d.size(); i++) {
        limb_t lo = a.d[i + w] >> s;
        limb_t hi = (s && i + w + 1 < a.size()) ? a.d[i + w + 1] << (64 - s) : 0;
        r.d[i] = lo | hi;
    }
    r.trim();
    return r;
}

// ------------------------------------------------------------------ division

// Knuth Algorithm D.  q: la - lb + 1 limbs, r: lb limbs.  la >= lb >= 1,
// b[lb - 1] != 0.
void mag_divmod(limb_t* q, limb_t* r, const limb_t* a, size_t la, const limb_t* b, size_t lb) {
    if (lb == 1) {
        limb_t rem = 0;
        const limb_t v = b[0];
        for (size_t i = la; i-- > 0;) {
            u128 cur = ((u128)rem << 64) | a[i];
            q[i] = (limb_t)(cur / v);
            rem = (limb_t)(cur % v);
        }
        r[0] = rem;
        return;
    }
    const int s = __builtin_clzll(b[lb - 1]);
    std::vector<limb_t> vn(lb), un(la + 1);
    for (size_t i = lb - 1; i > 0; i--) vn[i] = s ? (b[i] << s) | (b[i - 1] >> (64 - s)) : b[i];
    vn[0] = b[0] << s;
    un[la] = s ? a[la - 1] >> (64 - s) : 0;
    for (size_t i = la - 1; i > 0; i--) un[i] = s ? (a[i] << s) | (a[i - 1] >> (64 - s)) : a[i];
    un[0] = a[0] << s;
    const limb_t vtop = vn[lb - 1], vnext = vn[lb - 2];

    for (size_t jj = la - lb + 1; jj-- > 0;) {
        // estimate the quotient digit from the top two limbs
        u128 num = ((u128)un[jj + lb] << 64) | un[jj + lb - 1];
        u128 qhat = num / vtop;
        u128 rhat = num - qhat * vtop;
        while ((qhat >> 64) != 0 || qhat * vnext > ((rhat << 64) | un[jj + lb - 2])) {
            qhat -= 1;
            rhat += vtop;
            if ((rhat >> 64) != 0) break;
        }
        // un[jj .. jj+lb] -= qhat * vn
        limb_t mulcarry = 0, borrow = 0;
        for (size_t i = 0; i < lb; i++) {
            u128 p = qhat * vn[i] + mulcarry;
            mulcarry = (limb_t)(p >> 64);
            limb_t pl = (limb_t)p;
            limb_t u = un[i + jj];
            limb_t t = u - pl;
            limb_t b1 = u < pl;
            limb_t t2 = t - borrow;
            limb_t b2 = t < borrow;
            un[i + jj] = t2;
            borrow = b1 | b2;
        }
        limb_t u = un[jj + lb];
        limb_t t = u - mulcarry;
        limb_t b1 = u < mulcarry;
        limb_t t2 = t - borrow;
        limb_t b2 = t < borrow;
        un[jj + lb] = t2;
        if (b1 | b2) {  // estimate one too large: add the divisor back
            qhat -= 1;
            limb_t c = 0;
            for (size_t i = 0; i < lb; i++) {
                u128 sum = (u128)un[i + jj] + vn[i] + c;
                un[i + jj] = (limb_t)sum;
                c = (limb_t)(sum >> 64);
            }
            un[jj + lb] += c;
        }
        q[jj] = (limb_t)qhat;
    }
    for (size_t i = 0; i + 1 < lb; i++) r[i] = s ? (un[i] >> s) | (un[i + 1] << (64 - s)) : un[i];
    r[lb - 1] = un[lb - 1] >> s;
}

void divmod_trunc(const BigInt& a, const BigInt& b, BigInt* q, BigInt* r) {
    if (b.is_zero()) throw std::domain_error("division by zero");
    if (cmp_abs(a, b) < 0) {
        if (q) *q = BigInt();
        if (r) *r = a;
        return;
    }
    size_t la = a.size(), lb = b.size();
    BigInt qq, rr;
    qq.d.resize(la - lb + 1);
    rr.d.resize(lb);
    mag_divmod(qq.d.data(), rr.d.data(), a.d.data(), la, b.d.data(), lb);
    qq.neg = a.neg != b.neg;
    rr.neg = a.neg;
    qq.trim();
    rr.trim();
    if (q) *q = std::move(qq);
    if (r) *r = std::move(rr);
}

BigInt mod_floor(const BigInt& a, const BigInt& m) {
    BigInt r;
    divmod_trunc(a, m, nullptr, &r);
    if (r.neg) r = add(r, m);
    return r;
}

BigInt divexact(const BigInt& a, const BigInt& b) {
    BigInt q, r;
    divmod_trunc(a, b, &q, &r);
    if (!r.is_zero()) throw std::logic_error("inexact division");
    return q;
}

// Exact division by one word, in place: the factor 2^t of b shifts out,
// then the odd part's inverse modulo 2^64 (Newton's iteration, each pass
// doubling the correct low bits from 3) turns the division into a product,
// limb by limb from the bottom, carrying the high words of q_i b' as a
// borrow (Hensel).  Limb i of the quotient needs limbs i and i + 1 of a
// only, so it overwrites limb i.  Throws when b does not divide a (a is
// then left unspecified, unless the low bits of a already show it).
void divexact_u64_inplace(BigInt& a, uint64_t b) {
    if (b == 0) throw std::domain_error("division by zero");
    if (a.is_zero() || b == 1) return;
    const int t = __builtin_ctzll(b);
    const uint64_t bo = b >> t;
    if (t && (a.d[0] & ((1ULL << t) - 1))) throw std::logic_error("inexact division");
    const size_t n = a.size();
    limb_t* v = a.d.data();
    if (bo != 1) {
        uint64_t inv = bo;
        for (int i = 0; i < 5; i++) inv *= 2 - bo * inv;
        uint64_t borrow = 0;
        for (size_t i = 0; i < n; i++) {
            const uint64_t ai = t ? (v[i] >> t) | (i + 1 < n ? v[i + 1] << (64 - t) : 0) : v[i];
            const uint64_t s = ai - borrow;
            const uint64_t qi = s * inv;
            borrow = (uint64_t)(((u128)qi * bo) >> 64) + (ai < borrow);
            v[i] = qi;
        }
        if (borrow != 0) throw std::logic_error("inexact division");
    } else {
        // a power of two: a shift
        for (size_t i = 0; i + 1 < n; i++) v[i] = (v[i] >> t) | (v[i + 1] << (64 - t));
        v[n - 1] >>= t;
    }
    a.trim();
    if (a.is_zero()) a.neg = false;
}

BigInt divexact_u64(const BigInt& a, uint64_t b) {
    BigInt q = a;
    divexact_u64_inplace(q, b);
    return q;
}

BigInt pow_u(const BigInt& a, unsigned e) {
    BigInt result = BigInt::from_u64(1), base = a;
    while (e) {
        if (e & 1) result = mul(result, base);
        e >>= 1;
        if (e) base = mul(base, base);
    }
    return result;
}

// ------------------------------------------------------------------ Lehmer

// Algorithm L inner loop: the cofactor matrix [[A, B], [C, D]] of as many
// Euclidean steps as the leading words determine.  Returns false when not
// even one step is certain (B == 0).
static bool lehmer_matrix(int64_t xh, int64_t yh, int64_t* A, int64_t* B, int64_t* C, int64_t* D) {
    int64_t a = 1, b = 0, c = 0, d = 1;
    for (;;) {
        int64_t den1 = yh + c, den2 = yh + d;
        if (den1 <= 0 || den2 <= 0) break;
        int64_t num1 = xh + a, num2 = xh + b;
        if (num1 < 0 || num2 < 0) break;
        int64_t q = num1 / den1;
        if (q != num2 / den2) break;
        i128 t;
        t = (i128)a - (i128)q * c; a = c; c = (int64_t)t;
        t = (i128)b - (i128)q * d; b = d; d = (int64_t)t;
        t = (i128)xh - (i128)q * yh; xh = yh; yh = (int64_t)t;
    }
    *A = a; *B = b; *C = c; *D = d;
    return b != 0;
}

static void lincomb_rem(limb_t* x, limb_t* y, size_t n, int64_t A, int64_t B, int64_t C, int64_t D);

// u128 to double, within about 2^-52 relative
static inline double u128_to_double(u128 v) {
    return (double)(uint64_t)(v >> 64) * 0x1p64 + (double)(uint64_t)v;
}

// floor(num / den) for num < 2^127, 0 < den < 2^127, when it is below 2^40
// (false otherwise): a double estimate within one of it, then exact
// corrections (the products stay below num + den)
static bool small_quotient(u128 num, u128 den, uint64_t* q) {
    const double e = u128_to_double(num) / u128_to_double(den);
    if (!(e < 0x1p40)) return false;
    uint64_t qe = (uint64_t)e;
    u128 prod = (u128)qe * den;
    while (prod > num) {
        qe--;
        prod -= den;
    }
    while (num - prod >= den) {
        qe++;
        prod += den;
    }
    if (qe >> 40) return false;
    *q = qe;
    return true;
}

// Algorithm L on two-word leading parts x >= y (below 2^124, taken at the
// same bit position): the cofactor matrix of as many Euclidean steps as
// they determine, each quotient accepted when both bounds of the true
// ratio, (x + A) / (y + C) and (x + B) / (y + D), give it.  The cofactor
// magnitudes stay below 2^62 (so a matrix covers about 62 bits, twice the
// one-word form).  Returns false when not even one step is certain.
// floor(num / den), den > 0, when it is below 2^40 (false otherwise): the
// quotients 0 to 3 (about two in three of a Euclidean sequence's) by
// subtraction, larger ones by small_quotient
static inline bool quotient_below_2p40(u128 num, u128 den, uint64_t* q) {
    // den < 2^125 here (y + |c| with y below 2^124), so 4 den does not wrap;
    // the count of multiples reached is the quotient when it is below 4
    const u128 d2 = den << 1, d3 = d2 + den;
    const uint64_t k = (uint64_t)(num >= den) + (uint64_t)(num >= d2) + (uint64_t)(num >= d3);
    if (k < 3 || num < d3 + den) {
        *q = k;
        return true;
    }
    return small_quotient(num, den, q);
}

// whether floor(num / den) == q (den > 0, q < 2^40): q den <= num and
// num - q den < den, with q den formed without overflowing 128 bits
static inline bool quotient_is(u128 num, u128 den, uint64_t q) {
    const u128 hi = (den >> 64) * (u128)q;  // below 2^104
    if (hi >> 64) return false;             // q den >= 2^128 > num
    const u128 lo = (u128)(uint64_t)den * q;
    const u128 p = (hi << 64) + lo;
    if (p < lo || p > num) return false;    // wrapped (q den >= 2^128), or above num
    return num - p < den;
}

static bool lehmer_matrix2(u128 xh, u128 yh, int64_t* A, int64_t* B, int64_t* C, int64_t* D) {
    int64_t a = 1, b = 0, c = 0, d = 1;
    i128 x = (i128)xh, y = (i128)yh;
    for (;;) {
        const i128 den1 = y + c, den2 = y + d;
        if (den1 <= 0 || den2 <= 0) break;
        const i128 num1 = x + a, num2 = x + b;
        if (num1 < 0 || num2 < 0) break;
        // the step is certain when both bounds of the true ratio give the same quotient
        uint64_t q;
        if (!quotient_below_2p40((u128)num1, (u128)den1, &q) || !quotient_is((u128)num2, (u128)den2, q)) break;
        // |a - q c| <= |a| + q |c| (equal, as the signs alternate), likewise for b, d
        const u128 mc = (u128)(a < 0 ? -(i128)a : (i128)a) + (u128)q * (u128)(c < 0 ? -(i128)c : (i128)c);
        const u128 md = (u128)(b < 0 ? -(i128)b : (i128)b) + (u128)q * (u128)(d < 0 ? -(i128)d : (i128)d);
        if ((mc >> 62) != 0 || (md >> 62) != 0) break;
        const int64_t nc = (int64_t)((i128)a - (i128)q * c), nd = (int64_t)((i128)b - (i128)q * d);
        a = c;
        c = nc;
        b = d;
        d = nd;
        const i128 ny = x - (i128)q * y;  // |q y| < 2^126: q < 2^40 and y below 2^124
        x = y;
        y = ny;
    }
    *A = a;
    *B = b;
    *C = c;
    *D = d;
    return b != 0;
}

BigInt lcm(const BigInt& a, const BigInt& b) {
    if (a.is_zero() || b.is_zero()) return BigInt();
    BigInt g = gcd(a, b);
    BigInt r = mul(divexact(a, g), b);
    r.neg = false;
    return r;
}

// Raw-limb pieces of the extended Euclid below.  Lengths are kept trimmed
// (no leading zero limbs).
static size_t trimmed(const limb_t* x, size_t n) {
    while (n && x[n - 1] == 0) n--;
    return n;
}

static size_t bits_of(const limb_t* x, size_t n) {
    return n ? 64 * n - (size_t)__builtin_clzll(x[n - 1]) : 0;
}

// -1, 0, 1 as x < y, x == y, x > y
static int cmp_limbs(const limb_t* x, size_t nx, const limb_t* y, size_t ny) {
    if (nx != ny) return nx < ny ? -1 : 1;
    for (size_t i = nx; i-- > 0;)
        if (x[i] != y[i]) return x[i] < y[i] ? -1 : 1;
    return 0;
}

// (x, y) <- (A x + B y, C x + D y) for nonnegative x, y (n limbs each, zero
// padded) whose images are nonnegative; the cofactors have the sign pattern
// (+, -, -, +) (EVEN) or (-, +, +, -) and magnitudes a, b, c, d below 2^63,
// so every partial sum lies within +-2^127: formed modulo 2^128, its high
// word read as signed is the next carry.
template <bool EVEN>
static void lincomb_rem_range(limb_t* x, limb_t* y, size_t lo, size_t hi, uint64_t a, uint64_t b, uint64_t c,
                              uint64_t d, int64_t* cxo, int64_t* cyo) {
    int64_t cx = 0, cy = 0;
    for (size_t i = lo; i < hi; i++) {
        const uint64_t xi = x[i], yi = y[i];
        u128 tx, ty;
        if (EVEN) {
            tx = (u128)a * xi - (u128)b * yi + (u128)(i128)cx;
            ty = (u128)d * yi - (u128)c * xi + (u128)(i128)cy;
        } else {
            tx = (u128)b * yi - (u128)a * xi + (u128)(i128)cx;
            ty = (u128)c * xi - (u128)d * yi + (u128)(i128)cy;
        }
        x[i] = (limb_t)tx;
        y[i] = (limb_t)ty;
        cx = (int64_t)(uint64_t)(tx >> 64);
        cy = (int64_t)(uint64_t)(ty >> 64);
    }
    *cxo = cx;
    *cyo = cy;
}

// the limbs [lo, hi) of (x, y) <- (A x + B y, C x + D y), the signed carries
// out of limb hi - 1 returned (the sum over the range is the range's new
// limbs plus carry 2^(64 hi))
static void lincomb_rem_part(limb_t* x, limb_t* y, size_t lo, size_t hi, int64_t A, int64_t B, int64_t C, int64_t D,
                             int64_t* cx, int64_t* cy) {
    const uint64_t a = (uint64_t)(A < 0 ? -A : A), b = (uint64_t)(B < 0 ? -B : B);
    const uint64_t c = (uint64_t)(C < 0 ? -C : C), d = (uint64_t)(D < 0 ? -D : D);
    if (A >= 0 && B <= 0) lincomb_rem_range<true>(x, y, lo, hi, a, b, c, d, cx, cy);
    else lincomb_rem_range<false>(x, y, lo, hi, a, b, c, d, cx, cy);
}

static void lincomb_rem(limb_t* x, limb_t* y, size_t n, int64_t A, int64_t B, int64_t C, int64_t D) {
    int64_t cx, cy;
    lincomb_rem_part(x, y, 0, n, A, B, C, D, &cx, &cy);
    if (cx != 0 || cy != 0) throw std::logic_error("Lehmer step left a carry");
}

// (s, t) <- (a s + b t, c s + d t) for magnitudes below 2^62 (a s_i + b t_i
// plus the carry stays below 2^128); s, t hold n limbs and room for one more
static size_t lincomb_mag(limb_t* s, limb_t* t, size_t n, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
    if ((a | b | c | d) >> 62) throw std::logic_error("cofactor out of range");
    u128 cs = 0, ct = 0;
    for (size_t i = 0; i < n; i++) {
        const uint64_t si = s[i], ti = t[i];
        cs += (u128)a * si + (u128)b * ti;
        ct += (u128)c * si + (u128)d * ti;
        s[i] = (limb_t)cs;
        t[i] = (limb_t)ct;
        cs >>= 64;
        ct >>= 64;
    }
    s[n] = (limb_t)cs;
    t[n] = (limb_t)ct;
    return cs || ct ? n + 1 : n;
}

// 124 bits of v (n limbs) from bit sh up (zero above the top)
static u128 bits124_at(const limb_t* v, size_t n, size_t sh) {
    const size_t w = sh / 64, o = sh % 64;
    auto word = [&](size_t i) -> uint64_t { return i < n ? v[i] : 0; };
    u128 lo = ((u128)word(w + 1) << 64) | word(w);
    if (o) lo = (lo >> o) | ((u128)word(w + 2) << (128 - o));
    return lo & (((u128)1 << 124) - 1);
}

// One Euclidean step in place, x <- x - q y with q = floor(x / y), for
// trimmed x >= y > 0 whose quotient is below 2^62 (false, nothing changed,
// otherwise).  q starts from the leading 124 bits of x and y's bits at the
// same position: x >= xh 2^sh and y < (yh + 1) 2^sh, so floor(xh / (yh + 1))
// never exceeds q, and with yh >= 2^63 (lengths at most 60 bits apart) it
// falls short by at most two, which the comparisons afterwards add back
// (for x below 2^124 the leading parts are the numbers and q is exact).
static bool small_division_step(limb_t* x, size_t* nx, const limb_t* y, size_t ny, uint64_t* qo) {
    const size_t bx = bits_of(x, *nx), by = bits_of(y, ny);
    if (by == 0 || bx < by || bx - by > 60) return false;
    const size_t sh = bx > 124 ? bx - 124 : 0;
    const u128 xh = bits124_at(x, *nx, sh), yh = bits124_at(y, ny, sh);
    const u128 qe = sh == 0 ? xh / yh : xh / (yh + 1);
    if (qe >> 62) return false;
    uint64_t q = (uint64_t)qe;
    // x -= q y (q y <= x): multiply-subtract with a product carry and a borrow
    uint64_t mc = 0, br = 0;
    for (size_t i = 0; i < *nx; i++) {
        const u128 p = (i < ny ? (u128)q * y[i] : 0) + mc;
        mc = (uint64_t)(p >> 64);
        const uint64_t pl = (uint64_t)p, xi = x[i];
        const uint64_t t = xi - pl, t2 = t - br;
        br = (uint64_t)(xi < pl) + (uint64_t)(t < br);
        x[i] = t2;
    }
    if (mc != 0 || br != 0) throw std::logic_error("division step went below zero");
    *nx = trimmed(x, *nx);
    while (cmp_limbs(x, *nx, y, ny) >= 0) {
        sub_in(x, *nx, y, ny);
        *nx = trimmed(x, *nx);
        if (++q >> 62) throw std::logic_error("division step quotient out of range");
    }
    *qo = q;
    return true;
}

// gcd by Lehmer's method on raw limbs: matrices from two-word leading parts
// (about 62 bits a pass over the limbs), one-word quotients in place, a
// full division only for a quotient of 2^62 or more, and the last two limbs
// in 128-bit arithmetic.
BigInt gcd(const BigInt& a0, const BigInt& b0) {
    const size_t L = std::max(a0.size(), b0.size()) + 1;
    std::vector<limb_t> r0(L, 0), r1(L, 0);
    std::copy(a0.d.begin(), a0.d.end(), r0.begin());
    std::copy(b0.d.begin(), b0.d.end(), r1.begin());
    size_t n0 = a0.size(), n1 = b0.size();
    if (cmp_limbs(r0.data(), n0, r1.data(), n1) < 0) {
        std::swap(r0, r1);
        std::swap(n0, n1);
    }
    while (n1 > 0) {
        if (n0 <= 2) {
            u128 u = ((u128)(n0 > 1 ? r0[1] : 0) << 64) | (n0 > 0 ? r0[0] : 0);
            u128 v = ((u128)(n1 > 1 ? r1[1] : 0) << 64) | r1[0];
            while (v) {
                const u128 t = u % v;
                u = v;
                v = t;
            }
            BigInt g;
            g.d = {(limb_t)u, (limb_t)(u >> 64)};
            g.trim();
            return g;
        }
        // the top 124 bits of r0 (n0 >= 3: at least 129 bits) and r1's at the same position
        const size_t sh = bits_of(r0.data(), n0) - 124;
        const u128 xh = bits124_at(r0.data(), n0, sh), yh = bits124_at(r1.data(), n1, sh);
        int64_t A, B, C, D;
        if (yh != 0 && lehmer_matrix2(xh, yh, &A, &B, &C, &D)) {
            lincomb_rem(r0.data(), r1.data(), n0, A, B, C, D);  // images below the old r0
            n1 = trimmed(r1.data(), n0);
            n0 = trimmed(r0.data(), n0);
            continue;
        }
        uint64_t q;
        if (small_division_step(r0.data(), &n0, r1.data(), n1, &q)) {
            std::swap(r0, r1);
            std::swap(n0, n1);
            continue;
        }
        BigInt x, y, r;
        x.d.assign(r0.begin(), r0.begin() + n0);
        y.d.assign(r1.begin(), r1.begin() + n1);
        divmod_trunc(x, y, nullptr, &r);
        std::fill(r0.begin(), r0.end(), 0);
        std::copy(r1.begin(), r1.begin() + n1, r0.begin());
        n0 = n1;
        std::fill(r1.begin(), r1.end(), 0);
        std::copy(r.d.begin(), r.d.end(), r1.begin());
        n1 = r.size();
    }
    BigInt g;
    g.d.assign(r0.begin(), r0.begin() + n0);
    g.trim();
    return g;
}

// The cofactor magnitudes |t0|, |t1| of the extended Euclid below: Lehmer
// matrices and full-division steps act on them in order.  They depend on
// the remainders only through those matrices and quotients, so for long
// inputs the updates run on a second thread, fed through a single-producer
// ring, while the caller's thread works on the remainders.
class CofactorTrack {
  public:
    CofactorTrack(size_t L, bool threaded) : t0_(L, 0), t1_(L, 0), ring_(threaded ? kRing : 0) {
        t1_[0] = 1;
        if (threaded) {
            try {
                th_ = std::thread([this] { run(); });
            } catch (...) {
                ring_.clear();  // no thread: the updates run inline
            }
        }
    }
    ~CofactorTrack() {
        if (th_.joinable()) {
            done_.store(true, std::memory_order_release);
            th_.join();
        }
    }
    // (t0, t1) <- (a t0 + b t1, c t0 + d t1) on the magnitudes
    void matrix(uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
        Op op{a, b, c, d, false, BigInt()};
        push(std::move(op));
    }
    // (t0, t1) <- (t1, t0 + q t1)
    void division(BigInt&& q) {
        Op op{0, 0, 0, 0, true, std::move(q)};
        push(std::move(op));
    }
    // |t1| once every update has been applied
    BigInt finish() {
        if (th_.joinable()) {
            done_.store(true, std::memory_order_release);
            th_.join();
        }
        if (err_) std::rethrow_exception(err_);
        BigInt tt;
        tt.d.assign(t1_.begin(), t1_.begin() + nt_);
        tt.trim();
        return tt;
    }

  private:
    struct Op {
        uint64_t a, b, c, d;
        bool div;
        BigInt q;
    };
    static constexpr size_t kRing = 256;

    void apply(Op& op) {
        if (!op.div) {
            nt_ = lincomb_mag(t0_.data(), t1_.data(), nt_, op.a, op.b, op.c, op.d);
            return;
        }
        BigInt tm;
        tm.d.assign(t1_.begin(), t1_.begin() + nt_);
        tm.trim();
        BigInt t0b;
        t0b.d.assign(t0_.begin(), t0_.begin() + nt_);
        t0b.trim();
        const BigInt nt0 = add(t0b, mul(op.q, tm));
        std::fill(t0_.begin(), t0_.end(), 0);
        std::copy(t1_.begin(), t1_.begin() + nt_, t0_.begin());
        std::fill(t1_.begin(), t1_.end(), 0);
        std::copy(nt0.d.begin(), nt0.d.end(), t1_.begin());
        nt_ = std::max(nt_, nt0.size());
    }
    void push(Op&& op) {
        if (ring_.empty()) {
            apply(op);
            return;
        }
        const size_t h = head_.load(std::memory_order_relaxed);
        while (h - tail_.load(std::memory_order_acquire) >= kRing) std::this_thread::yield();
        ring_[h % kRing] = std::move(op);
        head_.store(h + 1, std::memory_order_release);
    }
    void run() {
        size_t t = 0;
        for (;;) {
            if (t < head_.load(std::memory_order_acquire)) {
                if (!err_) {
                    try {
                        apply(ring_[t % kRing]);
                    } catch (...) {
                        err_ = std::current_exception();
                    }
                }
                ring_[t % kRing].q = BigInt();
                tail_.store(++t, std::memory_order_release);
                continue;
            }
            if (done_.load(std::memory_order_acquire) && head_.load(std::memory_order_acquire) == t) break;
            __builtin_ia32_pause();
        }
    }

    std::vector<limb_t> t0_, t1_;
    size_t nt_ = 1;
    std::vector<Op> ring_;
    std::atomic<size_t> head_{0}, tail_{0};
    std::atomic<bool> done_{false};
    std::thread th_;
    std::exception_ptr err_;
};

bool rational_reconstruct(const BigInt& a, const BigInt& M, const BigInt& N, const BigInt& D,
                          BigInt* num, BigInt* den, bool require_coprime, bool split_cofactors) {
    // extended Euclid on (M, a) tracking the cofactor of a: r_k = s_k M + t_k a.
    // The t_k alternate in sign, so their magnitudes only add:
    // |t_{k+1}| = |t_{k-1}| + q_k |t_k|, and a Lehmer matrix acts on them as
    // (|A| |t0| + |B| |t1|, |C| |t0| + |D| |t1|).
    const size_t L = M.size() + 2;
    std::vector<limb_t> r0(L, 0), r1(L, 0);
    std::copy(M.d.begin(), M.d.end(), r0.begin());
    std::copy(a.d.begin(), a.d.end(), r1.begin());
    size_t n0 = M.size(), n1 = trimmed(r1.data(), a.size());
    CofactorTrack tr(L, split_cofactors && L > 256);
    bool t1neg = false;  // t0 has the other sign (or is 0)
    const size_t nbits = N.bit_length();
    auto above_N = [&]() { return cmp_limbs(r1.data(), n1, N.d.data(), N.size()) > 0; };
    // a Lehmer matrix applied to the remainders and the cofactor magnitudes
    auto apply = [&](int64_t A, int64_t B, int64_t C, int64_t D2) {
        lincomb_rem(r0.data(), r1.data(), n0, A, B, C, D2);
        n0 = trimmed(r0.data(), n0);
        n1 = trimmed(r1.data(), n0 > n1 ? n0 : n1);
        const uint64_t ua = (uint64_t)(A < 0 ? -A : A), ub = (uint64_t)(B < 0 ? -B : B);
        const uint64_t uc = (uint64_t)(C < 0 ? -C : C), ud = (uint64_t)(D2 < 0 ? -D2 : D2);
        if ((ua | ub | uc | ud) >> 62) throw std::logic_error("cofactor out of range");
        tr.matrix(ua, ub, uc, ud);
        if (D2 < 0) t1neg = !t1neg;
        if (cmp_limbs(r0.data(), n0, N.d.data(), N.size()) <= 0)
            throw std::logic_error("Lehmer step passed the stopping point");
    };
    while (above_N()) {
        const size_t b0 = bits_of(r0.data(), n0);
        const size_t b1 = bits_of(r1.data(), n1);
        if (b1 > nbits + 130 && b0 > 124) {
            // two-word leading parts: the top 124 bits of r0 and the bits of
            // r1 at the same position (a matrix of up to 62-bit cofactors
            // shrinks r0 by at most about 2^64, so it stops above N)
            const size_t sh = b0 - 124;
            auto lead2 = [&](const std::vector<limb_t>& v, size_t nv) -> u128 {
                const size_t w = sh / 64, o = sh % 64;
                auto word = [&](size_t i) -> uint64_t { return i < nv ? v[i] : 0; };
                u128 lo = ((u128)word(w + 1) << 64) | word(w);
                if (o) lo = (lo >> o) | ((u128)word(w + 2) << (128 - o));
                return lo & (((u128)1 << 124) - 1);
            };
            const u128 xh = lead2(r0, n0), yh = lead2(r1, n1);
            int64_t A, B, C, D2;
            if (yh != 0 && lehmer_matrix2(xh, yh, &A, &B, &C, &D2)) {
                apply(A, B, C, D2);
                continue;
            }
        }
        if (b1 > nbits + 64 && n0 > 1) {
            // leading 62 bits of r0 and the bits of r1 at the same position
            const size_t sh = b0 - 62;
            auto lead = [&](const std::vector<limb_t>& v, size_t nv) -> int64_t {
                const size_t w = sh / 64, o = sh % 64;
                if (w >= nv) return 0;
                uint64_t lo = v[w] >> o;
                if (o && w + 1 < nv) lo |= v[w + 1] << (64 - o);
                return (int64_t)(lo & ((1ULL << 63) - 1));
            };
            const int64_t xh = lead(r0, n0), yh = lead(r1, n1);
            int64_t A, B, C, D2;
            if (yh != 0 && lehmer_matrix(xh, yh, &A, &B, &C, &D2)) {
                apply(A, B, C, D2);
                continue;
            }
        }
        // one Euclidean step: in place when its quotient fits 62 bits
        // (the steps near N, where a Lehmer matrix could pass it), else a
        // full division
        uint64_t qs;
        if (small_division_step(r0.data(), &n0, r1.data(), n1, &qs)) {
            std::swap(r0, r1);
            std::swap(n0, n1);
            tr.matrix(0, 1, 1, qs);  // (t0, t1) <- (t1, t0 + q t1)
            t1neg = !t1neg;
            continue;
        }
        BigInt x, y, q, r;
        x.d.assign(r0.begin(), r0.begin() + n0);
        y.d.assign(r1.begin(), r1.begin() + n1);
        divmod_trunc(x, y, &q, &r);
        // t0 <- |t0| + q |t1| (then swap): the new cofactor takes t0's sign
        tr.division(std::move(q));
        std::fill(r0.begin(), r0.end(), 0);
        std::copy(r1.begin(), r1.begin() + n1, r0.begin());
        n0 = n1;
        std::fill(r1.begin(), r1.end(), 0);
        std::copy(r.d.begin(), r.d.end(), r1.begin());
        n1 = r.size();
        t1neg = !t1neg;
    }
    BigInt rr;
    rr.d.assign(r1.begin(), r1.begin() + n1);
    rr.trim();
    const BigInt tt = tr.finish();
    if (tt.is_zero() || cmp_abs(tt, D) > 0) return false;
    if (require_coprime) {
        BigInt g = gcd(rr, tt);
        if (!(g.size() == 1 && g.d[0] == 1)) return false;
    }
    // a == r1 / t1 (mod M): a negative t1 moves its sign to the numerator
    *num = rr;
    num->neg = t1neg && !rr.is_zero();
    *den = tt;
    return true;
}

}  // namespace es
