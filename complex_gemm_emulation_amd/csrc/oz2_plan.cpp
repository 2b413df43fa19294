// oz2_plan.cpp -- moduli selection and the per-s constant tables.
//
// "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs:
// Ozaki Scheme II on the Xe2 Architecture":
//  * Sec. 2.3 step 2 / Table 2: s pairwise-coprime moduli <= 256.  The set
//    used is the one of maximal product (it reproduces every log2 M of
//    Table 2); among equal products the lexicographically largest descending
//    sequence is taken.
//  * Sec. 4.1: t is the largest integer with k 2^(2t) <= M/4 (2k for ZGEMM).
//  * Sec. 4.2: residues from limbs of a_hat + 2^62 with the constants
//    2^(limb position) mod m and K_m = (h_m - 2^62) mod m, h_m = floor((m-1)/2);
//    the limbs here are bytes (the page's are 21 bits), four per 32-bit word.
//  * Sec. 4.4: q = rint(sum r_t y_t/m_t) from the fixed-point constants
//    Y_t = round(2^16 y_t/m_t) (the page uses fl32(y_t/m_t)); c_hat =
//    sum r_t W_t - q M in 16-bit limbs; N_L 32-bit words.
#include "oz2_plan.h"

#include <cmath>
#include <cstring>
#include <mutex>

namespace oz2 {

// ---------------------------------------------------------------- UBig
UBig::UBig() { std::memset(w, 0, sizeof w); }

UBig UBig::from_u64(uint64_t v) {
    UBig r;
    r.w[0] = (uint32_t)v;
    r.w[1] = (uint32_t)(v >> 32);
    return r;
}

void UBig::mul_small(uint32_t m) {
    uint64_t carry = 0;
    for (int i = 0; i < kWords; ++i) {
        uint64_t x = (uint64_t)w[i] * m + carry;
        w[i] = (uint32_t)x;
        carry = x >> 32;
    }
}

uint32_t UBig::mod_small(uint32_t m) const {
    uint64_t r = 0;
    for (int i = kWords - 1; i >= 0; --i) r = ((r << 32) | w[i]) % m;
    return (uint32_t)r;
}

UBig UBig::div_small(uint32_t m) const {
    UBig q;
    uint64_t r = 0;
    for (int i = kWords - 1; i >= 0; --i) {
        uint64_t cur = (r << 32) | w[i];
        q.w[i] = (uint32_t)(cur / m);
        r = cur % m;
    }
    return q;
}

UBig UBig::shl(int bits) const {
    UBig r;
    int ws = bits / 32, bs = bits % 32;
    for (int i = kWords - 1; i >= 0; --i) {
        uint64_t v = 0;
        int src = i - ws;
        if (src >= 0) v = (uint64_t)w[src] << bs;
        if (bs && src - 1 >= 0) v |= (uint64_t)w[src - 1] >> (32 - bs);
        r.w[i] = (uint32_t)v;
    }
    return r;
}

int UBig::cmp(const UBig& o) const {
    for (int i = kWords - 1; i >= 0; --i)
        if (w[i] != o.w[i]) return w[i] < o.w[i] ? -1 : 1;
    return 0;
}

int UBig::bitlen() const {
    for (int i = kWords - 1; i >= 0; --i)
        if (w[i]) return 32 * i + 32 - __builtin_clz(w[i]);
    return 0;
}

double UBig::log2() const {
    int L = bitlen();
    if (L == 0) return -INFINITY;
    // top 64 bits as a double, then add the exponent
    UBig t = *this;
    int drop = L > 64 ? L - 64 : 0;
    double top = 0.0;
    for (int b = L - 1; b >= drop; --b) top = top * 2.0 + (double)((t.w[b / 32] >> (b % 32)) & 1u);
    return std::log2(top) + drop;
}

uint32_t UBig::limb16(int i) const { return (w[i / 2] >> (16 * (i % 2))) & 0xffffu; }

// ------------------------------------------------------ moduli search
namespace {

struct Candidate {
    uint32_t value;
    uint64_t primes;  // bit b set <=> the b-th prime divides value
};

struct Search {
    int s = 0;
    Candidate cand[255];
    int ncand = 0;
    uint32_t pick[kMaxS] = {};
    uint32_t best_pick[kMaxS] = {};
    UBig best;  // zero until a full set is found

    // product of the r largest candidates from index i on that share no
    // prime with `used` (an upper bound for completing the set)
    bool bound(int i, int r, uint64_t used, const UBig& prod, UBig* out) const {
        UBig b = prod;
        int got = 0;
        for (int j = i; j < ncand && got < r; ++j) {
            if (cand[j].primes & used) continue;
            b.mul_small(cand[j].value);
            ++got;
        }
        *out = b;
        return got == r;
    }

    void run(int depth, int i, uint64_t used, const UBig& prod) {
        if (depth == s) {
            if (prod.cmp(best) > 0) {
                best = prod;
                std::memcpy(best_pick, pick, sizeof pick);
            }
            return;
        }
        UBig ub;
        if (!bound(i, s - depth, used, prod, &ub) || ub.cmp(best) <= 0) return;
        for (int j = i; j < ncand; ++j) {
            if (cand[j].primes & used) continue;
            // every completion from j on is at most prod * value^(s-depth)
            UBig cap = prod;
            for (int q = depth; q < s; ++q) cap.mul_small(cand[j].value);
            if (cap.cmp(best) <= 0) break;
            pick[depth] = cand[j].value;
            UBig next = prod;
            next.mul_small(cand[j].value);
            run(depth + 1, j + 1, used | cand[j].primes, next);
        }
    }
};

uint32_t pow2_mod(int e, uint32_t m) {
    uint64_t r = 1 % m;
    for (int i = 0; i < e; ++i) r = (r * 2) % m;
    return (uint32_t)r;
}

uint32_t inverse_mod(uint32_t a, uint32_t m) {
    // extended Euclid on small integers
    int64_t t = 0, nt = 1, r = m, nr = a % m;
    while (nr) {
        int64_t q = r / nr;
        int64_t tmp = t - q * nt; t = nt; nt = tmp;
        tmp = r - q * nr; r = nr; nr = tmp;
    }
    if (t < 0) t += m;
    return (uint32_t)t;
}

void build_plan(int s, ModuliPlan* p) {
    Search S;
    S.s = s;
    static const int primes[] = {2,   3,   5,   7,   11,  13,  17,  19,  23,  29,  31,  37,  41,  43,
                                 47,  53,  59,  61,  67,  71,  73,  79,  83,  89,  97,  101, 103, 107,
                                 109, 113, 127, 131, 137, 139, 149, 151, 157, 163, 167, 173, 179, 181,
                                 191, 193, 197, 199, 211, 223, 227, 229, 233, 239, 241, 251};
    const int np = (int)(sizeof primes / sizeof primes[0]);
    for (uint32_t v = 256; v >= 2; --v) {
        Candidate c{v, 0};
        for (int b = 0; b < np; ++b)
            if (v % primes[b] == 0) c.primes |= 1ull << b;
        S.cand[S.ncand++] = c;
    }
    S.run(0, 0, 0, UBig::from_u64(1));

    p->s = s;
    for (int i = 0; i < s; ++i) p->mod[i] = (int)S.best_pick[i];
    p->M = S.best;
    p->log2M = p->M.log2();
    int nl = (int)std::floor(p->log2M / 32.0) + 1;
    p->NL = nl < 2 ? 2 : nl;
    for (int l = 0; l < 2 * p->NL; ++l) p->M16[l] = p->M.limb16(l);
    for (int t = 0; t < s; ++t) {
        uint32_t m = (uint32_t)p->mod[t];
        UBig Mt = p->M.div_small(m);
        uint32_t y = inverse_mod(Mt.mod_small(m), m);
        UBig W = Mt;
        W.mul_small(y);
        for (int l = 0; l < 2 * p->NL; ++l) p->W16[t][l] = W.limb16(l);
        p->yfix[t] = (uint32_t)((((uint64_t)y << 17) + m) / (2ull * m));  // round(2^16 y / m)
        volatile float fm = (float)m;
        uint32_t h = (m - 1) / 2;
        p->h[t] = h;
        for (int q = 0; q < kExtWords; ++q) {
            uint32_t w = 0;
            for (int j = 0; j < 4; ++j) w |= pow2_mod(32 * q + 8 * j, m) << (8 * j);
            p->c4[t][q] = w;
        }
        p->Kstd[t] = (m - pow2_mod(62, m)) % m;
        p->Kext[t] = (m - pow2_mod(104, m)) % m;
        volatile float fone = 1.0f;
        p->frcp[t] = fone / fm;
        // offset-binary bytes (residue + 128 in [0, 255]): m = 256 takes the
        // window [-128, 127], whose bytes are those of [-127, 128]
        volatile float fhb = (float)(m == 256 ? 128u : h) + 0.5f - 128.0f;
        p->foffb[t] = fhb / fm;
        volatile double done = 1.0, dm = (double)m;
        p->drcp[t] = done / dm;
    }
    // limb pairs for the two-moduli-per-instruction CRT accumulation; past the
    // last modulus the high halves stay 0
    for (int u = 0; u < (s + 1) / 2; ++u) p->Y2[u] = p->yfix[2 * u] | (2 * u + 1 < s ? p->yfix[2 * u + 1] << 16 : 0u);
    for (int u = 0; u < (s + 1) / 2; ++u)
        for (int l = 0; l < 2 * p->NL; ++l)
            p->W2[u][l] = p->W16[2 * u][l] | (2 * u + 1 < s ? p->W16[2 * u + 1][l] << 16 : 0u);
}

std::once_flag g_once[kMaxS + 1];
ModuliPlan g_plans[kMaxS + 1];

}  // namespace

const ModuliPlan* moduli_plan(int s) {
    if (s < kMinS || s > kMaxS) return nullptr;
    std::call_once(g_once[s], [s] { build_plan(s, &g_plans[s]); });
    // every max-product set starts with 256 (2^8 is coprime to every odd
    // modulus); the encoders take that plane as the low byte of a_hat
    if (g_plans[s].mod[0] != 256) return nullptr;
    return &g_plans[s];
}

int scaling_width(const ModuliPlan& p, int64_t k, bool is_complex) {
    uint64_t kk = (uint64_t)(k < 1 ? 1 : k) * (is_complex ? 2u : 1u);
    UBig base = UBig::from_u64(kk);
    int t = 0;
    // k' * 4^(t+2) <= M  <=>  (k' << (2t + 4)) <= M
    while (t < 200 && base.shl(2 * t + 4).cmp(p.M) <= 0) ++t;
    return t;
}

}  // namespace oz2
