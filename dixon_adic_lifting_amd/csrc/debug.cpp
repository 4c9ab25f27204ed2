// Test hooks into the host bignum code (include/es_debug.h).
#include "../../include/es_debug.h"

#include <vector>

#include "bignum.h"
#include "host.h"

using es::BigInt;

namespace {

BigInt make(const uint64_t* p, int32_t len, int neg) {
    BigInt r;
    if (len > 0) r.d.assign(p, p + len);
    r.neg = neg != 0;
    r.trim();
    return r;
}

bool put(const BigInt& v, uint64_t* out, int32_t* len, int* neg, int32_t cap) {
    if ((int32_t)v.size() > cap) return false;
    for (size_t i = 0; i < v.size(); i++) out[i] = v.d[i];
    *len = (int32_t)v.size();
    if (neg) *neg = v.neg ? 1 : 0;
    return true;
}

}  // namespace

extern "C" int es_dbg_bignum(int op, const uint64_t* a, int32_t la, int a_neg, const uint64_t* b, int32_t lb,
                             int b_neg, uint64_t* r1, int32_t* l1, int* n1, uint64_t* r2, int32_t* l2, int* n2,
                             int32_t cap) {
    try {
        BigInt A = make(a, la, a_neg), B = make(b, lb, b_neg), x, y;
        switch (op) {
            case ES_DBG_MUL: x = es::mul(A, B); break;
            case ES_DBG_DIVMOD:
                if (B.is_zero()) return -1;
                es::divmod_trunc(A, B, &x, &y);
                break;
            case ES_DBG_GCD: x = es::gcd(A, B); break;
            case ES_DBG_ADD: x = es::add(A, B); break;
            case ES_DBG_SUB: x = es::sub(A, B); break;
            case ES_DBG_DIVEXACT1:
                if (B.size() != 1 || B.neg) return -1;
                x = es::divexact_u64(A, B.d[0]);
                break;
            default: return -1;
        }
        if (!put(x, r1, l1, n1, cap)) return -1;
        if (op == ES_DBG_DIVMOD && !put(y, r2, l2, n2, cap)) return -1;
        return 0;
    } catch (...) {
        return -6;
    }
}

extern "C" int es_dbg_assemble(const uint64_t* P, int32_t lP, const int64_t* digits, int32_t m, int32_t count,
                               int32_t parts, uint64_t* out, int32_t* lens, int* neg, int32_t cap) {
    if (!P || lP < 1 || !digits || m < 1 || count < 1 || parts < 1 || (parts & (parts - 1)) || !out || !lens ||
        !neg)
        return -1;
    try {
        const BigInt Pb = make(P, lP, 0);
        std::vector<BigInt> pw((size_t)m + 1);
        pw[0] = BigInt::from_u64(1);
        for (int i = 1; i <= m; i++) pw[i] = es::mul(pw[i - 1], Pb);
        const size_t stride = (size_t)m * 6;
        std::vector<BigInt> split((size_t)count);
        es::assemble_split(digits, stride, (size_t)count, m, pw, parts, es::default_threads(), split.data());
        for (int32_t k = 0; k < count; k++) {
            const BigInt whole = es::assemble(digits + (size_t)k * stride, m, pw);
            if (es::cmp(whole, split[k]) != 0) return -2;
            if (!put(whole, out + (size_t)k * cap, &lens[k], &neg[k], cap)) return -1;
        }
        return 0;
    } catch (...) {
        return -6;
    }
}

extern "C" int es_dbg_ratrec(const uint64_t* a, int32_t la, const uint64_t* M, int32_t lM, const uint64_t* N,
                             int32_t lN, const uint64_t* D, int32_t lD, uint64_t* num, int32_t* lnum, int* nneg,
                             uint64_t* den, int32_t* lden, int32_t cap) {
    try {
        const BigInt A = make(a, la, 0), Mm = make(M, lM, 0), Nn = make(N, lN, 0), Dd = make(D, lD, 0);
        BigInt nu, de, nu2, de2;
        const bool ok = es::rational_reconstruct(A, Mm, Nn, Dd, &nu, &de);
        const bool ok2 = es::rational_reconstruct(A, Mm, Nn, Dd, &nu2, &de2, true, true);
        if (ok != ok2 || (ok && (es::cmp(nu, nu2) != 0 || es::cmp(de, de2) != 0))) return -2;
        if (!ok) return 1;
        if (!put(nu, num, lnum, nneg, cap) || !put(de, den, lden, nullptr, cap)) return -1;
        return 0;
    } catch (...) {
        return -6;
    }
}

extern "C" int es_dbg_step_count(uint64_t mask, int32_t nbits, int32_t dbits, int32_t* m_exact, int64_t* bits_exact,
                                 int32_t* m_fast, int64_t* bits_fast) {
    if ((mask & ((1ULL << es::kNumPrimes) - 1)) == 0 || nbits < 1 || dbits < 1 || !m_exact || !bits_exact ||
        !m_fast || !bits_fast)
        return -1;
    try {
        const es::LiveSet ls = es::live_set_from_mask(mask);
        BigInt M;
        *m_exact = es::choose_m(ls.P, nbits, dbits, &M);
        *bits_exact = (int64_t)M.bit_length();
        size_t b = 0;
        *m_fast = es::choose_m_bits(ls.P, nbits, dbits, &b);
        *bits_fast = (int64_t)b;
        return 0;
    } catch (...) {
        return -6;
    }
}
