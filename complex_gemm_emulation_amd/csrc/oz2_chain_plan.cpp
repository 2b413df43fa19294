// oz2_chain_plan.cpp -- host planning of the persistent tensor-mode chain
// (OzII-RescaleBE).
//
// "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products":
//  - Sec. 5.1 Eq. (27) and Algorithm 5: every operator row is one encoding
//    group, f = b - E with 2^(E-1) <= max|row| < 2^E, rounded to nearest
//    (ties to even);
//  - Sec. 5.2 (after Eq. 28): in a chain longer than one pass, the row
//    scales 2^-f still pending on a direction multiply the columns of the
//    next operator on that direction before it is encoded; its own row
//    exponents then replace them (operator i acts on direction i mod 3);
//  - Sec. 4.3 Eq. (21): rho_i = maximal absolute row sum of the integer
//    operator;
//  - Sec. 4.3 Eq. (22)-(23), the drop schedule and the choice of b: the
//    bound B starts at 2^b and is multiplied by rho_i per product under
//    2 B < P; after a non-final product the smallest moduli leave while
//    floor(B/q) keeps b bits, each leaving floor(B/q) + 1 under
//    2 B' < P_L / q; b is the largest value <= 53 whose schedule passes
//    (exact wide-integer bounds throughout);
//  - Sec. 2.3 Eq. (11): centred residues, [v]_p in [-floor(p/2), ceil(p/2) - 1];
//  - Sec. 4.4 Eq. (24)-(26): mixed-radix weights omega_{i,p} = [prod_{l<i} m_l]_p.
// The basis is the max-product modulus set of the DGEMM emulation for s,
// descending, so 256 (its only even modulus) comes first.
#include <cmath>
#include <cstring>
#include <vector>

#include "oz2.h"
#include "oz2_internal.h"

namespace oz2 {
namespace {

int centered(int64_t v, int p) {
    int64_t r = v % p;
    if (r < 0) r += p;
    return (int)(r < (p + 1) / 2 ? r : r - p);
}

int64_t inverse_mod(int64_t a, int64_t p) {
    // extended Euclid; a and p coprime
    int64_t t = 0, nt = 1, r = p, nr = ((a % p) + p) % p;
    while (nr) {
        const int64_t q = r / nr;
        int64_t x = t - q * nt; t = nt; nt = x;
        x = r - q * nr; r = nr; nr = x;
    }
    return t < 0 ? t + p : t;
}

UBig add(const UBig& a, const UBig& b) {
    UBig c;
    uint64_t carry = 0;
    for (int i = 0; i < UBig::kWords; ++i) {
        const uint64_t s = (uint64_t)a.w[i] + b.w[i] + carry;
        c.w[i] = (uint32_t)s;
        carry = s >> 32;
    }
    return c;
}

UBig mul_u64(const UBig& a, uint64_t m) {
    UBig lo = a, hi = a;
    lo.mul_small((uint32_t)m);
    hi.mul_small((uint32_t)(m >> 32));
    return add(lo, hi.shl(32));
}

UBig pow2(int e) { return UBig::from_u64(1).shl(e); }

// Encode one operator at b (rows = groups) after folding the pending column
// scales 2^-pend[k] into it (exact: powers of two): integer entries and row
// exponents
bool encode_rows(const double* A, const int* pend, int n, int b, int64_t* Abar, int* f) {
    for (int a = 0; a < n; ++a) {
        double mx = 0.0;
        for (int k = 0; k < n; ++k) {
            const double x = std::ldexp(A[a + (int64_t)n * k], -pend[k]);
            if (!std::isfinite(x)) return false;
            mx = std::fmax(mx, std::fabs(x));
        }
        if (mx == 0.0) {
            f[a] = 0;
            for (int k = 0; k < n; ++k) Abar[a * n + k] = 0;
            continue;
        }
        int E = 0;
        (void)std::frexp(mx, &E);
        f[a] = b - E;
        for (int k = 0; k < n; ++k)
            Abar[a * n + k] = (int64_t)std::nearbyint(std::ldexp(std::ldexp(A[a + (int64_t)n * k], -pend[k]), f[a]));
    }
    return true;
}

uint64_t row_sum_bound(const int64_t* Abar, int n) {
    uint64_t rho = 0;
    for (int a = 0; a < n; ++a) {
        uint64_t r = 0;
        for (int k = 0; k < n; ++k) r += (uint64_t)std::llabs(Abar[a * n + k]);
        rho = r > rho ? r : rho;
    }
    return rho;
}

// The rescaling after a non-final product (the chain page, Sec. 4.3 around
// Eq. 23).  B bounds the product's entries; the moduli leave smallest first
// (the basis is descending, so from its end) while floor(B/q) keeps b bits
// and more than one modulus would remain, each leaving floor(B/q) + 1 (one
// unit for the rounding of the division), which must stay recoverable on
// the moduli left, 2 B' < P_L / q.  Sets *removed, B and *kept (the product
// of the moduli left); false when a removal breaks that condition.
bool greedy_rescale(UBig& B, int b, const int* basis, int s, const UBig& P, int* removed, UBig* kept) {
    const UBig two_b = pow2(b);
    UBig P_left = P;
    int left = s;
    *removed = 0;
    while (left > 1) {
        const uint32_t q = (uint32_t)basis[left - 1];
        const UBig quot = B.div_small(q);
        if (quot.cmp(two_b) < 0) break;
        B = add(quot, UBig::from_u64(1));
        P_left = P_left.div_small(q);
        if (B.shl(1).cmp(P_left) >= 0) return false;
        --left;
        ++*removed;
    }
    *kept = P_left;
    return true;
}

// Drop counts of a chain with row-sum bounds rho (Sec. 4.3, Eq. 21-23): the
// bound starts at 2^b and each product multiplies it by its rho (Eq. 22),
// keeping 2 B < P; after every product but the last, greedy_rescale, then
// base extension restores the whole basis for the next product (the
// proposed method's restoration).  The last product is decoded directly.
// crt[i]: 1 <= g[i] <= 14 (the packing of ChainCrtTable needs slots 0 and 1
// kept) and the bound B' left after product i's drops keeps 2^-13 from half
// the kept moduli's product, 2^13 B' <= (2^12 - 1) P_L
// (B' / P_L <= 1/2 - 2^-13).
bool drop_plan(int b, int d, const uint64_t* rho, const int* basis, int s, int* g, int* crt) {
    UBig P = UBig::from_u64(1);
    for (int i = 0; i < s; ++i) P.mul_small((uint32_t)basis[i]);
    UBig B = pow2(b);
    for (int i = 0; i < d; ++i) {
        B = mul_u64(B, rho[i]);
        if (B.shl(1).cmp(P) >= 0) return false;
        g[i] = 0;
        crt[i] = 0;
        if (i < d - 1) {
            UBig kept;
            if (!greedy_rescale(B, b, basis, s, P, &g[i], &kept)) return false;
            UBig lim = kept;
            lim.mul_small(4095);
            crt[i] = g[i] >= 1 && g[i] <= kChainMaxS - 2 && B.shl(13).cmp(lim) <= 0;
        }
    }
    return true;
}

}  // namespace

int chain_plan(int s, int n, int d, const double* const* ops, const int* modes, ChainParams* P,
               ChainTables* T, int8_t* ops_res, int* fexp) {
    const ModuliPlan* pl = moduli_plan(s);
    if (!pl || s > kChainMaxS || n < 1 || n > kChainMaxN || d < 1 || d > kChainMaxD) return OZ2_STATUS_INTERNAL;
    if (pl->mod[0] != 256) return OZ2_STATUS_INTERNAL;
    for (int i = 1; i < s; ++i)
        if (pl->mod[i] % 2 == 0) return OZ2_STATUS_INTERNAL;
    for (int i = 0; i < d; ++i)
        for (int x = 0; x < n * n; ++x)
            if (!std::isfinite(ops[i][x])) return -(i + 1);
    std::vector<int64_t> Abar((size_t)d * n * n);
    std::vector<int> f((size_t)d * n), pend((size_t)3 * n);
    int g[kChainMaxD] = {}, crt[kChainMaxD] = {};
    // the effective integer operators at b (the pending scales of a direction
    // folded into the next operator on it) and whether their schedule passes;
    // encoding depends on b, so the bounds are taken afresh for every b
    auto passes = [&](int b) {
        uint64_t rho[kChainMaxD];
        std::fill(pend.begin(), pend.end(), 0);
        for (int i = 0; i < d; ++i) {
            int* pm = &pend[(size_t)modes[i] * n];
            if (!encode_rows(ops[i], pm, n, b, &Abar[(size_t)i * n * n], &f[(size_t)i * n])) return false;
            rho[i] = row_sum_bound(&Abar[(size_t)i * n * n], n);
            std::memcpy(pm, &f[(size_t)i * n], sizeof(int) * n);
        }
        return drop_plan(b, d, rho, pl->mod, s, g, crt);
    };
    int b = 53;
    while (b >= 1 && !passes(b)) --b;
    if (b < 1) return OZ2_STATUS_RANGE;
    P->n = n;
    P->s = s;
    P->b = b;
    P->d = d;
    for (int i = 0; i < kChainMaxD; ++i) {
        P->g[i] = i < d ? g[i] : 0;
        P->crt[i] = i < d ? crt[i] : 0;
    }
    // residue layout: a product contracts position 0 and leaves its lane's
    // entries (the old position 1), fibres (old position 2) and outputs (its
    // own direction); the next direction to contract goes to position 0
    int pos[3] = {modes[0], (modes[0] + 1) % 3, (modes[0] + 2) % 3};
    P->m0 = modes[0];
    P->cyclic = 1;
    for (int i = 0; i < d; ++i) P->cyclic &= modes[i] == i % 3;
    for (int i = 0; i < kChainMaxD; ++i) P->kind[i] = 0;
    for (int i = 0; i < d; ++i) {
        const int de = pos[1], dt = pos[2], da = modes[i];
        if (i == d - 1) {
            P->fin[0] = de;
            P->fin[1] = dt;
            P->fin[2] = da;
            break;
        }
        const int next = modes[i + 1];
        if (next == de) {
            P->kind[i] = 0;  // layout (e, t, a)
            pos[0] = de, pos[1] = dt, pos[2] = da;
        } else if (next == dt) {
            P->kind[i] = 1;  // layout (t, e, a)
            pos[0] = dt, pos[1] = de, pos[2] = da;
        } else {
            P->kind[i] = 2;  // layout (a, e, t)
            pos[0] = da, pos[1] = de, pos[2] = dt;
        }
    }
    // alpha multiplier: the dropped moduli (the g smallest, smallest first)
    // in drop order, each product rounded to double
    double Qd = 1.0;
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < g[i]; ++j) Qd = Qd * (double)pl->mod[s - 1 - j];
    P->Qd = Qd;
    for (int m = 0; m < 3; ++m) {
        for (int a = 0; a < n; ++a) fexp[m * n + a] = pend[(size_t)m * n + a];
        for (int a = 0; a < kChainN; ++a) T->fexp[m][a] = a < n ? pend[(size_t)m * n + a] : 0;
    }
    for (int i = 0; i < d; ++i)
        for (int q = 0; q < s; ++q)
            for (int a = 0; a < n; ++a)
                for (int k = 0; k < n; ++k)
                    ops_res[(((size_t)i * s + q) * n + a) * n + k] =
                        (int8_t)centered(Abar[((size_t)i * n + a) * n + k], pl->mod[q]);
    // kernel tables in slot order: the s moduli right-aligned in kChainMaxS
    // slots (descending), the unused leading slots with the modulus 1
    const int first = kChainMaxS - s;
    int slot[kChainMaxS];
    for (int u = 0; u < kChainMaxS; ++u) slot[u] = u < first ? 1 : pl->mod[u - first];
    for (int u = 0; u < kChainMaxS; ++u) {
        T->mod[u] = (float)slot[u];
        T->rmod[u] = 1.0f / (float)slot[u];
        T->ohalf[u] = 0.5f - 128.0f * T->rmod[u];
    }
    for (int i = 0; i < kChainMaxS; ++i)
        for (int j = 0; j < kChainMaxS; ++j)
            T->inv[i][j] = i != j ? (float)inverse_mod(slot[i], slot[j]) : 0.0f;
    for (int j = 0; j < kChainMaxS; ++j) {
        int64_t w = 1;  // prod_{l<i} slot[l] reduced mod slot[j]
        for (int i = 0; i < kChainMaxS; ++i) {
            T->omega[i][j] = (float)centered(w, slot[j]);
            w = (w * slot[i]) % slot[j];
        }
    }
    return OZ2_STATUS_SUCCESS;
}

void chain_drop_table(const ChainTables& T, int g, ChainDropTable* D) {
    std::memset(D, 0, sizeof(*D));
    if (g < 1 || g > kChainMaxS - 1) return;
    int slot[kChainMaxS];
    for (int u = 0; u < kChainMaxS; ++u) slot[u] = (int)T.mod[u];
    const int keep = kChainMaxS - 1 - g;
    for (int p = 0; p <= keep; ++p) {
        const int m = slot[p];
        if (m == 1) continue;  // residues modulo 1 are zero
        int64_t Q = 1;  // prod_j q_j reduced mod m
        for (int j = 0; j < g; ++j) Q = Q * slot[kChainMaxS - 1 - j] % m;
        const int64_t qi = inverse_mod(Q, m);
        D->qinv[p] = (float)centered(qi, m);
        int64_t w = 1;  // prod_{l<j} q_l reduced mod m
        for (int j = 0; j < g; ++j) {
            D->nw[j][p] = (float)-centered(w * qi % m, m);
            w = w * slot[kChainMaxS - 1 - j] % m;
        }
    }
}

void chain_split_table(const ChainTables& T, int split, ChainDropTable* D) {
    std::memset(D, 0, sizeof(*D));
    if (split < 1 || kChainMaxS % split != 0 || (kChainMaxS / split - 1) * (split + 1) > kChainMaxS) return;
    int slot[kChainMaxS];
    for (int u = 0; u < kChainMaxS; ++u) slot[u] = (int)T.mod[u];
    // row r of the table: qinv for r = 0, nw[r - 1] after
    auto row = [D](int r) -> float* { return r == 0 ? D->qinv : D->nw[r - 1]; };
    for (int b = 0; b + 1 < kChainMaxS / split; ++b) {
        const int lo = b * split, hi = lo + split;
        for (int p = hi; p < kChainMaxS; ++p) {
            const int m = slot[p];
            if (m == 1) continue;
            int64_t Mb = 1;  // the block's modulus product reduced mod m
            for (int l = lo; l < hi; ++l) Mb = Mb * slot[l] % m;
            const int64_t qi = inverse_mod(Mb, m);
            row(b * (split + 1))[p] = (float)centered(qi, m);
            int64_t w = 1;  // prod_{lo <= l < lo + i} m_l reduced mod m
            for (int i = 0; i < split; ++i) {
                row(b * (split + 1) + 1 + i)[p] = (float)-centered(w * qi % m, m);
                w = w * slot[lo + i] % m;
            }
        }
    }
}

void chain_crt_table(const ChainTables& T, int g, ChainCrtTable* C) {
    std::memset(C, 0, sizeof(*C));
    if (g < 1 || g > kChainMaxS - 2) return;
    int slot[kChainMaxS];
    for (int u = 0; u < kChainMaxS; ++u) slot[u] = (int)T.mod[u];
    const int keep = kChainMaxS - 1 - g;
    // M / m_i reduced mod m (the kept moduli but m_i; modulus-1 slots add nothing)
    auto cofactor = [&](int i, int m) {
        int64_t w = 1 % m;
        for (int l = 0; l <= keep; ++l)
            if (l != i) w = w * slot[l] % m;
        return w;
    };
    for (int i = 0; i <= keep; ++i)
        if (slot[i] > 1) C->w[0][i] = (float)centered(inverse_mod(cofactor(i, slot[i]), slot[i]), slot[i]);
    for (int p = keep + 1; p < kChainMaxS; ++p) {
        const int m = slot[p];
        if (m == 1) continue;
        int64_t M = 1;
        for (int l = 0; l <= keep; ++l) M = M * slot[l] % m;
        C->w[1][p] = (float)centered(M, m);
        for (int i = 0; i <= keep; ++i)
            if (slot[i] > 1) C->w[p][i] = (float)centered(cofactor(i, m), m);
    }
}

}  // namespace oz2
