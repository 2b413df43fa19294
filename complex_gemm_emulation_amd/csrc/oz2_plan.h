// oz2_plan.h -- host-side tables of the Ozaki scheme II method (O(s) work per
// modulus set, computed once per s and cached).
//
// Method: "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc
// GPUs: Ozaki Scheme II on the Xe2 Architecture" -- Sec. 2.3 (moduli, CRT
// weights), Sec. 4.1 (scaling width t, Table 2), Sec. 4.2 (residue
// constants of the byte-limb method), Sec. 4.4 (the quotient's fixed-point
// constants round(2^16 y_t/m_t), 16-bit limbs of W_t and M, N_L).
#pragma once

#include <cstdint>

namespace oz2 {

constexpr int kMinS = 2;
constexpr int kMaxS = 24;
constexpr int kMaxNL = 6;            // 32-bit words of c_hat for s <= 24 (log2 M < 192)
constexpr int kMaxLimb16 = 2 * kMaxNL;
constexpr int kStdWords = 2;         // 32-bit words (four byte limbs each) of a_hat + 2^62 (t <= 61)
constexpr int kExtWords = 4;         // 32-bit words of a_hat + 2^104 (t <= 100)
constexpr int kMaxStdT = 61;

// Small unsigned big integer (little-endian 32-bit words), enough for M < 2^192
// and the shifts used to compare k * 4^(t+1) with M.
struct UBig {
    static constexpr int kWords = 10;
    uint32_t w[kWords];
    UBig();
    static UBig from_u64(uint64_t v);
    void mul_small(uint32_t m);
    uint32_t mod_small(uint32_t m) const;
    UBig div_small(uint32_t m) const;
    UBig shl(int bits) const;
    int cmp(const UBig& o) const;
    int bitlen() const;
    double log2() const;
    uint32_t limb16(int i) const;
};

struct ModuliPlan {
    int s = 0;
    int mod[kMaxS] = {};          // descending, pairwise coprime, <= 256
    UBig M;                       // product of the moduli
    double log2M = 0.0;
    int NL = 0;                   // 32-bit words of c_hat: max(2, floor(log2 M / 32) + 1)
    // reconstruction (Sec. 4.4)
    uint32_t yfix[kMaxS] = {};    // round(2^16 y_t / m_t), y_t = (M/m_t)^-1 mod m_t
    uint32_t Y2[kMaxS / 2] = {};  // yfix of moduli 2u and 2u+1 in 16-bit halves
    uint32_t W16[kMaxS][kMaxLimb16] = {};  // 16-bit limbs of W_t = (M/m_t) y_t
    uint32_t M16[kMaxLimb16] = {};         // 16-bit limbs of M
    uint32_t W2[kMaxS / 2][kMaxLimb16] = {};  // W16 of moduli 2u and 2u+1 packed in 16-bit halves
    // residue generation (Sec. 4.2)
    uint32_t h[kMaxS] = {};       // floor((m-1)/2)
    uint32_t c4[kMaxS][kExtWords] = {};    // byte j of word p: 2^(32p + 8j) mod m
    uint32_t Kstd[kMaxS] = {};    // (-2^62) mod m
    uint32_t Kext[kMaxS] = {};    // (-2^104) mod m
    float frcp[kMaxS] = {};       // fl32(1 / m)
    float foffb[kMaxS] = {};      // fl32((hb + 1/2 - 128) / m), hb = h (128 for m = 256)
    double drcp[kMaxS] = {};      // fl64(1 / m), for the reduction of INT32 accumulators
};

// Max-product set of s pairwise-coprime integers <= 256 and its constants;
// nullptr for s outside [2, 24].  Thread-safe, computed once per s.
const ModuliPlan* moduli_plan(int s);

// Largest t with k' 4^(t+1) <= M, k' = k (real) or 2k (complex); 0 if none.
int scaling_width(const ModuliPlan& p, int64_t k, bool is_complex);

}  // namespace oz2
