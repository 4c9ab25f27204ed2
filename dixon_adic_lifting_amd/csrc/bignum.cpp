// Host arbitrary-precision integers (see bignum.h for the methods used).
#include "bignum.h"

#include <algorithm>
#include <cstring>
#include <stdexcept>

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

// Leading 62 bits of x and the bits of y at the same position.
static void leading_pair(const BigInt& x, const BigInt& y, int64_t* xh, int64_t* yh) {
    size_t bl = x.bit_length();
    size_t sh = bl > 62 ? bl - 62 : 0;
    auto extract = [&](const BigInt& v) -> uint64_t {
        size_t w = sh / 64, s = sh % 64;
        if (w >= v.size()) return 0;
        uint64_t lo = v.d[w] >> s;
        uint64_t hi = (s && w + 1 < v.size()) ? v.d[w + 1] << (64 - s) : 0;
        return (lo | hi) & ((1ULL << 62) - 1 + (1ULL << 62));  // at most 63 bits
    };
    *xh = (int64_t)extract(x);
    *yh = (int64_t)extract(y);
}

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

// (x, y) <- (A x + B y, C x + D y) in place, for nonnegative x, y whose
// images are nonnegative (guaranteed by Algorithm L).  The cofactors come in
// sign pattern (+, -, -, +) or (-, +, +, -), so each new limb is a difference
// of two unsigned 64 x 64 -> 128-bit products.
static void apply_matrix(BigInt& x, BigInt& y, int64_t A, int64_t B, int64_t C, int64_t D) {
    const size_t n = std::max(x.size(), y.size());
    x.d.resize(n, 0);
    y.d.resize(n, 0);
    // new_x = p1 * u1 - p2 * u2, new_y = p3 * u3 - p4 * u4 with u in {x, y}
    const bool even = A >= 0 && B <= 0 && C <= 0 && D >= 0;
    const uint64_t a = (uint64_t)(A < 0 ? -A : A), b = (uint64_t)(B < 0 ? -B : B);
    const uint64_t c = (uint64_t)(C < 0 ? -C : C), d = (uint64_t)(D < 0 ? -D : D);
    limb_t* xp = x.d.data();
    limb_t* yp = y.d.data();
    u128 px = 0, mx = 0, py = 0, my = 0;  // running positive / negative partial sums (carries)
    for (size_t i = 0; i < n; i++) {
        const u128 xi = xp[i], yi = yp[i];
        // new_x: even -> a x - b y ; odd -> b y - a x.  new_y: even -> d y - c x ; odd -> c x - d y
        px += even ? a * xi : b * yi;
        mx += even ? b * yi : a * xi;
        py += even ? d * yi : c * xi;
        my += even ? c * xi : d * yi;
        // limb i of (px - mx): borrow handled by keeping both sums and carrying their high parts
        const limb_t lx = (limb_t)px - (limb_t)mx;
        const limb_t bx = (limb_t)px < (limb_t)mx;
        const limb_t ly = (limb_t)py - (limb_t)my;
        const limb_t by = (limb_t)py < (limb_t)my;
        xp[i] = lx;
        yp[i] = ly;
        px = (px >> 64);
        mx = (mx >> 64) + bx;
        py = (py >> 64);
        my = (my >> 64) + by;
    }
    if (px != mx || py != my) throw std::logic_error("Lehmer step left a carry");
    x.trim();
    y.trim();
}

BigInt gcd(const BigInt& a0, const BigInt& b0) {
    BigInt x = a0, y = b0;
    x.neg = y.neg = false;
    if (cmp_abs(x, y) < 0) std::swap(x, y);
    while (!y.is_zero()) {
        if (x.size() <= 1) {
            uint64_t u = x.is_zero() ? 0 : x.d[0], v = y.d[0];
            while (v) { uint64_t t = u % v; u = v; v = t; }
            return BigInt::from_u64(u);
        }
        int64_t xh, yh, A, B, C, D;
        leading_pair(x, y, &xh, &yh);
        if (yh != 0 && lehmer_matrix(xh, yh, &A, &B, &C, &D)) {
            apply_matrix(x, y, A, B, C, D);
        } else {
            BigInt r;
            divmod_trunc(x, y, nullptr, &r);
            x = std::move(y);
            y = std::move(r);
        }
    }
    return x;
}

BigInt lcm(const BigInt& a, const BigInt& b) {
    if (a.is_zero() || b.is_zero()) return BigInt();
    BigInt g = gcd(a, b);
    BigInt r = mul(divexact(a, g), b);
    r.neg = false;
    return r;
}

bool rational_reconstruct(const BigInt& a, const BigInt& M, const BigInt& N, const BigInt& D,
                          BigInt* num, BigInt* den) {
    // extended Euclid on (M, a) tracking the cofactor of a
    BigInt r0 = M, r1 = a, t0, t1 = BigInt::from_u64(1);
    r1.neg = false;
    const size_t nbits = N.bit_length();
    while (cmp_abs(r1, N) > 0) {
        if (r1.bit_length() > nbits + 64 && r0.size() > 1) {
            int64_t xh, yh, A, B, C, D2;
            leading_pair(r0, r1, &xh, &yh);
            if (yh != 0 && lehmer_matrix(xh, yh, &A, &B, &C, &D2)) {
                apply_matrix(r0, r1, A, B, C, D2);
                BigInt nt0 = add(mul_small(t0, A), mul_small(t1, B));
                BigInt nt1 = add(mul_small(t0, C), mul_small(t1, D2));
                t0 = std::move(nt0);
                t1 = std::move(nt1);
                if (cmp_abs(r0, N) <= 0) throw std::logic_error("Lehmer step passed the stopping point");
                continue;
            }
        }
        BigInt q, r;
        divmod_trunc(r0, r1, &q, &r);
        BigInt t = sub(t0, mul(q, t1));
        r0 = std::move(r1);
        r1 = std::move(r);
        t0 = std::move(t1);
        t1 = std::move(t);
    }
    if (t1.is_zero() || cmp_abs(t1, D) > 0) return false;
    BigInt g = gcd(r1, t1);
    if (!(g.size() == 1 && g.d[0] == 1)) return false;
    *num = r1;
    *den = t1;
    if (t1.neg) {
        num->neg = !r1.is_zero();
        den->neg = false;
    }
    return true;
}

}  // namespace es
