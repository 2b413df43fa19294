// Host sanitizer driver for the library's host planners (oz2_plan.cpp: UBig,
// the moduli plans and scaling widths; oz2_chain_plan.cpp: the persistent
// chain's planner and the weight tables of its one-pass drops and two-block
// reconstruction), built with -fsanitize=address,undefined by
// tests/test_sanitizers.py.  Every s, a spread of k, and chain plans over
// n, s, depth and mode orders, including non-finite and all-zero operators.
// The weight tables are also checked against their definitions, in exact
// integers on random residue vectors: the one-pass drop against g repeated
// RnsDrops, the digits in blocks against one elimination over all slots,
// the CRT base extension against the residues of the integer it extends.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "oz2.h"
#include "oz2_internal.h"

using namespace oz2;

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static double uniform() { return (double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0; }

static int centered_i(int64_t v, int m) {
    int64_t r = v % m;
    if (r < 0) r += m;
    return (int)(r < (m + 1) / 2 ? r : r - m);
}

// a random centred residue vector over the table's slots (0 for modulus 1)
static void random_residues(const int (&m)[kChainMaxS], int (&r)[kChainMaxS]) {
    for (int u = 0; u < kChainMaxS; ++u) r[u] = m[u] == 1 ? 0 : centered_i((int64_t)(next_u64() % 65536), m[u]);
}

// one-pass drop (chain_drop_table's weights) against g repeated RnsDrops
static int check_drop_table(const ChainTables& T, int g) {
    ChainDropTable D;
    chain_drop_table(T, g, &D);
    int m[kChainMaxS], bad = 0;
    for (int u = 0; u < kChainMaxS; ++u) m[u] = (int)T.mod[u];
    const int keep = kChainMaxS - 1 - g;
    for (int trial = 0; trial < 20; ++trial) {
        int r[kChainMaxS], a[kChainMaxS], b[kChainMaxS];
        random_residues(m, r);
        for (int u = 0; u < kChainMaxS; ++u) a[u] = r[u], b[u] = r[u] + 128;
        for (int qs = kChainMaxS - 1; qs > keep; --qs)
            for (int p = 0; p < qs; ++p)
                a[p] = m[p] == 1 ? 0 : centered_i((int64_t)(a[p] - a[qs]) * (int)T.inv[qs][p], m[p]);
        for (int jp = 1; jp < g; ++jp)
            for (int j = 0; j < jp; ++j) {
                const int p = kChainMaxS - 1 - jp, qs = kChainMaxS - 1 - j;
                b[p] = centered_i((int64_t)(b[p] - b[qs]) * (int)T.inv[qs][p], m[p]);
            }
        for (int p = 0; p <= keep; ++p) {
            int64_t acc = (int64_t)b[p] * (int)D.qinv[p];
            for (int j = 0; j < kChainMaxS - 1; ++j) acc += (int64_t)b[kChainMaxS - 1 - j] * (int)D.nw[j][p];
            bad += acc >= (1 << 19) || acc <= -(1 << 19);
            b[p] = m[p] == 1 ? 0 : centered_i(acc, m[p]);
        }
        for (int p = 0; p <= keep; ++p) bad += a[p] != b[p];
    }
    return bad;
}

// the mixed-radix digits in blocks of `split` slots (chain_split_table's
// weights) against one elimination over all slots, entries offset by 128 as
// in the kernels
static int check_split_table(const ChainTables& T, int split) {
    ChainDropTable D;
    chain_split_table(T, split, &D);
    const auto row = [&D](int r) -> const float* { return r == 0 ? D.qinv : D.nw[r - 1]; };
    int m[kChainMaxS], bad = 0;
    for (int u = 0; u < kChainMaxS; ++u) m[u] = (int)T.mod[u];
    const auto step = [&](int (&x)[kChainMaxS], int i, int j) {
        x[j] = m[j] == 1 ? 0 : centered_i((int64_t)(x[j] - x[i]) * (int)T.inv[i][j], m[j]);
    };
    for (int trial = 0; trial < 20; ++trial) {
        int r[kChainMaxS], a[kChainMaxS], b[kChainMaxS];
        random_residues(m, r);
        for (int u = 0; u < kChainMaxS; ++u) a[u] = b[u] = r[u] + 128;
        for (int i = 0; i < kChainMaxS - 1; ++i)
            for (int j = i + 1; j < kChainMaxS; ++j) step(a, i, j);
        for (int lo = 0; lo < kChainMaxS; lo += split) {
            const int hi = lo + split;
            for (int i = lo; i < hi - 1; ++i)
                for (int j = i + 1; j < hi; ++j) step(b, i, j);
            if (hi == kChainMaxS) break;
            const int rb = (lo / split) * (split + 1);
            for (int p = hi; p < kChainMaxS; ++p) {
                int64_t acc = (int64_t)b[p] * (int)row(rb)[p];
                for (int i = 0; i < split; ++i) acc += (int64_t)b[lo + i] * (int)row(rb + 1 + i)[p];
                bad += acc >= (1 << 19) || acc <= -(1 << 19);
                b[p] = m[p] == 1 ? 0 : centered_i(acc, m[p]);
            }
        }
        for (int u = 1; u < kChainMaxS; ++u) bad += a[u] != b[u];
        bad += a[0] != b[0];  // both still offset by 128
    }
    return bad;
}

// CRT base extension (chain_crt_table's packed weights and the kernels' FP32
// rounding of alpha; 1 <= g <= 14) against the residues of the integer
// itself: X drawn in |X| <= (1/2 - 2^-13) M, the plan's condition, with both
// ends of that range
static int check_crt_table(const ChainTables& T, int g) {
    ChainCrtTable C;
    chain_crt_table(T, g, &C);
    int m[kChainMaxS], bad = 0;
    for (int u = 0; u < kChainMaxS; ++u) m[u] = (int)T.mod[u];
    const int keep = kChainMaxS - 1 - g;
    __int128 M = 1;  // at most 15 moduli below 2^8: below 2^120
    for (int i = 0; i <= keep; ++i) M *= m[i];
    const __int128 lim = M / 2 - (M + 8191) / 8192;  // <= (1/2 - 2^-13) M
    const auto res = [](__int128 x, int q) { return centered_i((int64_t)(x % q), q); };
    for (int trial = 0; trial < 24; ++trial) {
        const unsigned __int128 rnd = (unsigned __int128)next_u64() << 64 | next_u64();
        __int128 X = (__int128)(rnd % (unsigned __int128)(lim + 1));
        if (trial % 2) X = -X;
        if (trial < 2) X = trial ? -lim : lim;
        int xi[kChainMaxS] = {};
        float S = 0.0f;
        __int128 sum = 0;
        for (int i = 0; i <= keep; ++i) {
            if (m[i] == 1) continue;
            xi[i] = centered_i((int64_t)res(X, m[i]) * (int)C.w[0][i], m[i]);
            S = std::fmaf((float)xi[i], T.rmod[i], S);
            sum += (__int128)xi[i] * (M / m[i]);
        }
        const int alpha = (int)std::floor(S + 0.5f);
        bad += (sum - X) % M != 0 || (sum - X) / M != alpha;
        for (int p = keep + 1; p < kChainMaxS; ++p) {
            int64_t acc = -(int64_t)alpha * (int)C.w[1][p];
            for (int i = 0; i <= keep; ++i) acc += (int64_t)xi[i] * (int)C.w[p][i];
            bad += acc >= (1 << 18) || acc <= -(1 << 18);
            bad += centered_i(acc, m[p]) != res(X, m[p]);
        }
    }
    return bad;
}

int main() {
    int bad = 0;
    for (int s = -1; s <= 26; ++s) {
        const ModuliPlan* pl = moduli_plan(s);
        if (s < kMinS || s > kMaxS) {
            bad += pl != nullptr;
            continue;
        }
        if (!pl) { ++bad; continue; }
        for (int64_t k : {1LL, 7LL, 4096LL, 131071LL, 300000LL, 1LL << 40})
            for (bool c : {false, true}) (void)scaling_width(*pl, k, c);
        UBig x = pl->M;
        for (uint32_t q : {3u, 256u, 65535u}) {
            (void)x.mod_small(q);
            x = x.div_small(q);
        }
        (void)pl->M.shl(17).cmp(x);
        (void)pl->M.log2();
        for (int l = 0; l < kMaxLimb16; ++l) (void)pl->M.limb16(l);
    }
    for (int rep = 0; rep < 40; ++rep) {
        // sides of the LDS kernel and, every fifth plan, of the HBM kernels
        const int n = rep % 5 == 4 ? 17 + (int)(next_u64() % 80) : 1 + (int)(next_u64() % 16);
        const int d = 1 + (int)(next_u64() % 8);
        const int s = 6 + 2 * (int)(next_u64() % 6);
        std::vector<std::vector<double>> ops(d, std::vector<double>((size_t)n * n));
        std::vector<const double*> ptr(d);
        std::vector<int> modes(d);
        for (int i = 0; i < d; ++i) {
            for (auto& v : ops[i]) v = rep % 9 == 5 ? 0.0 : uniform() * std::exp(4.0 * uniform());
            ptr[i] = ops[i].data();
            modes[i] = (int)(next_u64() % 3);
        }
        if (rep % 7 == 3) ops[d - 1][0] = NAN;
        ChainParams P{};
        ChainTables T{};
        std::vector<int8_t> residues((size_t)d * s * n * n);
        std::vector<int> fexp((size_t)3 * n);
        const int st = chain_plan(s, n, d, ptr.data(), modes.data(), &P, &T, residues.data(), fexp.data());
        if (rep % 7 == 3) bad += st != -d;
        if (st == 0) {
            for (int i = 0; i + 1 < d; ++i)
                if (P.g[i] >= 1) bad += check_drop_table(T, P.g[i]) + (P.g[i] <= 14 ? check_crt_table(T, P.g[i]) : 0);
            bad += check_split_table(T, kChainSplit) + check_split_table(T, 8);
        }
    }
    // the tables at every drop count the kernels accept, for s = 2 .. 16
    for (int s = kMinS; s <= kChainMaxS; ++s) {
        const ModuliPlan* pl = moduli_plan(s);
        ChainTables T{};
        const int first = kChainMaxS - s;
        for (int u = 0; u < kChainMaxS; ++u) T.mod[u] = (float)(u < first ? 1 : pl->mod[u - first]);
        for (int i = 0; i < kChainMaxS; ++i)
            for (int j = 0; j < kChainMaxS; ++j) {
                const int mi = (int)T.mod[i], mj = (int)T.mod[j];
                int iv = 0;
                if (i != j && mj > 1)
                    for (int x = 1; x < mj; ++x)
                        if ((int64_t)mi * x % mj == 1) { iv = x; break; }
                T.inv[i][j] = (float)iv;
            }
        for (int u = 0; u < kChainMaxS; ++u) T.rmod[u] = 1.0f / T.mod[u];
        for (int g = 1; g < s; ++g) bad += check_drop_table(T, g) + (g <= 14 ? check_crt_table(T, g) : 0);
        bad += check_split_table(T, kChainSplit) + check_split_table(T, 8);
    }
    std::printf("planner driver: %d unexpected results\n", bad);
    return bad != 0;
}
