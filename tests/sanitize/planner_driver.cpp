// Host sanitizer driver for the library's host planners (oz2_plan.cpp: UBig,
// the moduli plans and scaling widths; oz2_chain_plan.cpp: the persistent
// chain's planner), built with -fsanitize=address,undefined by
// tests/test_sanitizers.py.  Every s, a spread of k, and chain plans over
// n, s, depth and mode orders, including non-finite and all-zero operators.
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
    }
    std::printf("planner driver: %d unexpected results\n", bad);
    return bad != 0;
}
