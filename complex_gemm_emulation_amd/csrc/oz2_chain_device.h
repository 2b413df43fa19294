// oz2_chain_device.h -- per-entry residue arithmetic of the persistent
// tensor-mode chain (OzII-RescaleBE), shared by its two kernels: the
// one-block-per-tensor kernel with residues in LDS (oz2_chain.hip, n <= 16)
// and the HBM-resident kernels for larger tensors (oz2_chain_hbm.hip).
//
// "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products":
//  - Sec. 2.3 Eq. (11): centred residues, [v]_m in [-floor(m/2), ceil(m/2) - 1];
//  - Sec. 2.3.1 Eq. (15), Algorithm 1 (RnsDrop): dropping the modulus q maps
//    the residue r_p of every other modulus p to [(r_p - r_q) q^{-1}]_p;
//  - Sec. 4.4 Eq. (24)-(26), Algorithm 4 (MrcDigits, BaseExtend): centred
//    mixed-radix digits by successive elimination and the residues on the
//    dropped moduli from the weights omega_{i,p} = [prod_{l<i} m_l]_p;
//  - Algorithm 5 (ReconstructFP64): FP64 Horner over the digits.
// The kernels reach the integers of the page's steps by two shortcuts built
// on the uniqueness of mixed-radix digits, the g drops at once (drop_extend)
// and the final digits in two blocks (mrc_horner_split), and by a third,
// the base extension by the Chinese remainder theorem (extend_crt, where the
// plan's bound leaves the margin its FP32 rounding needs; else the page's
// mixed-radix form, extend_dropped).
//
// Moduli sit right-aligned in kChainMaxS slots, descending, so the smallest
// (the ones dropped) are always the last slots; unused leading slots carry
// the modulus 1, which leaves every mixed-radix step, weight and Horner step
// unchanged.  A lane works on four entries at once, so one read of a table
// entry serves four modular steps.  All modular arithmetic is on exact small
// integers held as floats: [x]_m = x - m floor(x fl32(1/m) + 1/2), exact for
// odd m while |x| < 2^19 and for m = 256 outright (cmod), or with the
// quotient rounded to nearest by two adds where the modulus cannot be 256
// with x outside [-128, 127] (cmod_odd).
#pragma once

#include "oz2_internal.h"

namespace oz2 {
namespace chain {

constexpr int kSlots = kChainMaxS;  // 16

__device__ __forceinline__ float cmod(float x, float m, float rm) {
    return fmaf(-m, floorf(fmaf(x, rm, 0.5f)), x);
}

// the same reduction where m is odd or 1, or m = 256 with x in [-128, 127]:
// q = x fl32(1/m) rounded to nearest by adding and subtracting 1.5 2^23
// (exact while |x fl32(1/m)| < 2^22).  For odd m, x / m is never a
// half-integer, and for |x| < 2^19 it lies within 2^-5 / m of x fl32(1/m),
// less than its distance 1 / (2m) to one, so q = floor(x / m + 1/2) as in
// cmod; for m = 256 and x in [-128, 127], x / 256 is in [-1/2, 1/2) and q = 0
// in both (the tie at -1/2 goes to the even 0).  Two FP32 adds in place of
// a floor, which issues at about half their rate.
constexpr float kRound = 12582912.0f;  // 1.5 2^23: adding and subtracting it rounds |y| < 2^22 to nearest

__device__ __forceinline__ float cmod_odd(float x, float m, float rm) {
    const float q = fmaf(x, rm, kRound) - kRound;
    return fmaf(-m, q, x);
}

// the same reduction of x - 128, offset by 128: [x - 128]_m + 128 in
// [0, 255] for m <= 256 (oh = fl32(1/2 - 128 fl32(1/m)); the floor argument
// is within 2^-5 / m + 2^-12 of (x - 128) / m + 1/2, and exact for m = 256
// and m = 1), the offset-binary byte that v_cvt_pk_u8_f32 packs
__device__ __forceinline__ float cmod128(float x, float m, float rm, float oh) {
    return fmaf(-m, floorf(fmaf(x, rm, oh)), x);
}

// byte `e` of a word of four offset-binary residues, as a float: the
// residue plus 128 (v_cvt_f32_ubyte)
__device__ __forceinline__ float unpack128(uint32_t w, int e) {
    return (float)((w >> (8 * e)) & 0xffu);
}

// four centred residues (exact integers held as floats) as one word
__device__ __forceinline__ uint32_t pack4(float r0, float r1, float r2, float r3) {
    return ((uint32_t)(int)r0 & 0xffu) | (((uint32_t)(int)r1 & 0xffu) << 8) |
           (((uint32_t)(int)r2 & 0xffu) << 16) | (((uint32_t)(int)r3 & 0xffu) << 24);
}

// the four entries of a lane into one plane: contiguous (step 0, one 32-bit
// store) or step bytes apart (byte stores; only when ANY)
template <bool ANY, class I>
__device__ __forceinline__ void store4(int8_t* p, I step, float r0, float r1, float r2, float r3) {
    if (!ANY || step == 0) {
        *(uint32_t*)p = pack4(r0, r1, r2, r3);
    } else {
        p[0] = (int8_t)(int)r0;
        p[step] = (int8_t)(int)r1;
        p[2 * step] = (int8_t)(int)r2;
        p[3 * step] = (int8_t)(int)r3;
    }
}

// the four accumulators of a 16 x 16 MFMA tile of slot u (each offset by the
// accumulator input 128), reduced modulo the slot's modulus and packed as
// offset-binary bytes
__device__ __forceinline__ uint32_t pack_products(const int (&acc)[4], const ChainTables* T, int u) {
    const float m = T->mod[u], rm = T->rmod[u], oh = T->ohalf[u];
    uint32_t w = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) w = __builtin_amdgcn_cvt_pk_u8_f32(cmod128((float)acc[q], m, rm, oh), q, w);
    return w;
}

// the four entries of every slot as floats, still offset by 128
__device__ __forceinline__ void unpack_tile(const uint32_t (&pk)[kSlots], float (&r)[4][kSlots]) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q][u] = unpack128(pk[u], q);
}

// After RnsDrop: store the kept slots (0 .. 15 - g), MrcDigits on them and
// BaseExtend to the dropped slots (Algorithm 4, Eq. 26), storing those too.
// With G >= 0 the drop count is a compile-time constant and the guards fold
// away, with G < 0 it is g_rt and the guards are uniform branches.
// put(u, r0, r1, r2, r3) stores slot u's four entries.
template <int G, class Put>
__device__ __forceinline__ void extend_dropped(int g_rt, float (&r)[4][kSlots], const ChainTables* T, const Put& put) {
    const int g = G >= 0 ? G : g_rt;
    const int keep = kSlots - 1 - g;  // last slot of the reduced basis
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
        if (u <= keep) put(u, r[0][u], r[1][u], r[2][u], r[3][u]);
    if (g == 0) return;  // nothing to extend to
    // mixed-radix digits of the kept residues, in place
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i)
#pragma unroll
        for (int j = i + 1; j < kSlots; ++j)
            if (j <= keep) {
                const float iv = T->inv[i][j], m = T->mod[j], rm = T->rmod[j];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e][j] = cmod_odd((r[e][j] - r[e][i]) * iv, m, rm);
            }
#pragma unroll
    for (int p = 1; p < kSlots; ++p)
        if (p > keep) {
            float ts[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < kSlots - 1; ++i)
                if (i <= keep) {
                    const float w = T->omega[i][p];
#pragma unroll
                    for (int e = 0; e < 4; ++e) ts[e] = fmaf(r[e][i], w, ts[e]);
                }
            const float m = T->mod[p], rm = T->rmod[p];
            put(p, cmod_odd(ts[0], m, rm), cmod_odd(ts[1], m, rm), cmod_odd(ts[2], m, rm), cmod_odd(ts[3], m, rm));
        }
}

// extend_dropped's residues by the Chinese remainder theorem (the table C,
// see ChainCrtTable; 1 <= g <= 14): the kept slots are stored, then turned
// in place into xi_i = [r_i cinv_i]_{m_i}, and every dropped slot p gets
// [sum_i xi_i [M / m_i]_{m_p} - alpha [M]_{m_p}]_{m_p} with alpha the
// integer nearest S = sum_i xi_i fl32(1/m_i).  Exactly, S = X_g / M + alpha
// with |X_g| / M <= 1/2 - 2^-13 (the plan's condition for C).  In FP32, S is
// within 2^-17 of its exact value (at most 15 terms of magnitude <= 1/2, each
// off by <= 2^-25 through fl32(1/m_i), 15 roundings of <= 2^-22 in partial
// sums below 8), so rounding it to nearest gives alpha.  The other sums are
// of exact integers below 2^18.  Both forms give the residues of the same
// integer X_g, so the results are bitwise equal, with k + 1 products per
// dropped slot and k reductions in place of extend_dropped's k (k - 1) / 2
// digit steps (k kept slots).
template <int G, class Put>
__device__ __forceinline__ void extend_crt(int g_rt, float (&r)[4][kSlots], const ChainTables* T,
                                           const ChainCrtTable* C, const Put& put) {
    const int g = G >= 0 ? G : g_rt;
    const int keep = kSlots - 1 - g;
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
        if (u <= keep) put(u, r[0][u], r[1][u], r[2][u], r[3][u]);
    if (g == 0) return;
    float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i)
        if (i <= keep) {
            const float c = C->w[0][i], m = T->mod[i], rm = T->rmod[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r[e][i] = cmod(r[e][i] * c, m, rm);
                S[e] = fmaf(r[e][i], rm, S[e]);
            }
        }
    float al[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) al[e] = (S[e] + kRound) - kRound;
#pragma unroll
    for (int p = 1; p < kSlots; ++p)
        if (p > keep) {
            const float cm = C->w[1][p];
            float ts[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ts[e] = -al[e] * cm;
#pragma unroll
            for (int i = 0; i < kSlots - 1; ++i)
                if (i <= keep) {
                    const float w = C->w[p][i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) ts[e] = fmaf(r[e][i], w, ts[e]);
                }
            const float m = T->mod[p], rm = T->rmod[p];
            put(p, cmod_odd(ts[0], m, rm), cmod_odd(ts[1], m, rm), cmod_odd(ts[2], m, rm), cmod_odd(ts[3], m, rm));
        }
}

// After a non-final product, for the four entries of a lane, the page's g
// successive RnsDrops (Algorithm 1, Eq. 15: slot 15 - j holds the smallest
// modulus left) taken at once (g >= 1; G >= 1 a compile-time drop count,
// G < 0 the run-time g_rt):
// g successive RnsDrops by the moduli q_0, q_1, .. (slots 15, 14, ..) turn
// the entry X into X_g = (X - D) / Q, Q = prod_j q_j and
// D = sum_j d_j prod_{l<j} q_l, with d_j the centred mixed-radix digits of X
// over q_0, q_1, .. (Algorithm 1 applied g times; Eq. 24 for the digits).
// So the digits come from successive elimination among the dropped slots
// alone (g (g - 1) / 2 steps, each slot's steps in the order the repeated
// drop takes them), and every kept slot p gets
// [X_g]_p = [r_p qinv_p + sum_j d_j nw_{j,p}]_{m_p} with the per-product
// table D (qinv_p = [Q^-1]_p, nw_{j,p} = -[prod_{l<j} q_l Q^-1]_p, centred,
// zero for j >= g): one exact integer sum (|sum| < 2^19) and one reduction
// instead of g modular steps.  The residues and digits are integers, so the
// result is bitwise that of the g repeated drops.  d_0 and the r_p come in
// offset by 128; nw_{0,p} = -qinv_p cancels it.  With a run-time g the sum
// runs over j < 8 without guards (zero weights) and over 8 <= j < 15 only
// when g > 8; a compile-time G takes its terms alone.  The base
// extension takes the CRT form with CRT (extend_crt, table C), else the
// mixed-radix form (extend_dropped); a compile-time choice, since the
// register allocation of a kernel holding both spills hundreds of bytes.
template <int G, bool CRT, class Put>
__device__ __forceinline__ void drop_extend(int g_rt, float (&r)[4][kSlots], const ChainTables* T,
                                            const ChainDropTable* D, const ChainCrtTable* C, const Put& put) {
    const int g = G >= 0 ? G : g_rt;
    const int keep = kSlots - 1 - g;
    // digits over the dropped slots: slot 15 - jp takes its steps with the
    // earlier dropped slots 15, 14, .. 15 - jp + 1 in that order
#pragma unroll
    for (int jp = 1; jp < kSlots - 1; ++jp)
        if (jp < g) {
            const int p = kSlots - 1 - jp;
            const float m = T->mod[p], rm = T->rmod[p];
#pragma unroll
            for (int j = 0; j < jp; ++j) {
                const int qs = kSlots - 1 - j;
                const float iv = T->inv[qs][p];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e][p] = cmod_odd((r[e][p] - r[e][qs]) * iv, m, rm);
            }
        }
    // the kept slots, in place (a zero weight may meet an updated slot)
#pragma unroll
    for (int p = 0; p < kSlots - 1; ++p)
        if (p <= keep) {
            const float qi = D->qinv[p];
            float acc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = r[e][p] * qi;
            // a compile-time G takes exactly its G terms (up to 8 here)
            constexpr int J8 = G >= 0 && G < 8 ? G : 8;
#pragma unroll
            for (int j = 0; j < J8; ++j) {
                const float w = D->nw[j][p];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(r[e][kSlots - 1 - j], w, acc[e]);
            }
            if (g > 8) {
#pragma unroll
                for (int j = 8; j < kSlots - 1; ++j) {
                    const float w = D->nw[j][p];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = fmaf(r[e][kSlots - 1 - j], w, acc[e]);
                }
            }
            const float m = T->mod[p], rm = T->rmod[p];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e][p] = cmod(acc[e], m, rm);
        }
    if constexpr (CRT)
        extend_crt<G>(g_rt, r, T, C, put);
    else
        extend_dropped<G>(g_rt, r, T, put);
}

// ReconstructFP64's integer part (Algorithm 5) for the four entries of a
// lane: the centred mixed-radix digits of the residues of every slot, then
// the FP64 Horner sum V = d_0 + m_0 (d_1 + m_1 (...)), each step one rounding
// of the exact value.  The page takes the digits by successive elimination
// over all 16 slots (120 steps); here they come in two blocks of kSplit:
//  - the digits of slots 0 .. kSplit - 1 by elimination among themselves;
//  - the residues of X' = (X - A) / M1 at slots kSplit .. 15, with
//    A = sum_{i<kSplit} d_i prod_{l<i} m_l and M1 = prod_{l<kSplit} m_l,
//    from one exact integer sum each, [X']_p = [r_p qinv_p +
//    sum_{i<kSplit} d_i nw_{i,p}]_{m_p}, with the table D (qinv_p =
//    [M1^-1]_p, nw_{i,p} = -[prod_{l<i} m_l M1^-1]_p, centred);
//  - the digits of X' over slots kSplit .. 15, which are X's digits there
//    (mixed-radix digits are unique).
// So the digits, and the Horner sum over them, are bitwise those of the
// single elimination, in 28 + 8 reductions + 28 steps instead of 120.  d_0
// and the r_p come in offset by 128: nw_{0,p} = -qinv_p cancels the offset
// in the sums (|sum| < 2^19), and d_0 loses it after the steps.
template <int kSplit>
__device__ __forceinline__ void mrc_horner_split(const uint32_t (&pk)[kSlots], const ChainTables* T,
                                                 const ChainDropTable* D, double (&V)[4]) {
    static_assert(kSlots % kSplit == 0 && (kSlots / kSplit - 1) * (kSplit + 1) <= kSlots, "table rows");
    float dg[4][kSlots];
    unpack_tile(pk, dg);
    // row r of the table: qinv for r = 0, nw[r - 1] after
    const auto row = [D](int r) -> const float* { return r == 0 ? D->qinv : D->nw[r - 1]; };
#pragma unroll
    for (int b = 0; b < kSlots / kSplit; ++b) {
        const int lo = b * kSplit, hi = lo + kSplit;
        // the block's digits, by elimination among its slots
#pragma unroll
        for (int i = lo; i < hi - 1; ++i)
#pragma unroll
            for (int j = i + 1; j < hi; ++j) {
                const float iv = T->inv[i][j], m = T->mod[j], rm = T->rmod[j];
#pragma unroll
                for (int q = 0; q < 4; ++q) dg[q][j] = cmod_odd((dg[q][j] - dg[q][i]) * iv, m, rm);
            }
        if (hi < kSlots) {
            // the later slots: the residues of (X_b - A_b) / M_b
            const float* qr = row(b * (kSplit + 1));
#pragma unroll
            for (int p = hi; p < kSlots; ++p) {
                const float qi = qr[p];
                float acc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = dg[q][p] * qi;
#pragma unroll
                for (int i = 0; i < kSplit; ++i) {
                    const float w = row(b * (kSplit + 1) + 1 + i)[p];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] = fmaf(dg[q][lo + i], w, acc[q]);
                }
                const float m = T->mod[p], rm = T->rmod[p];
#pragma unroll
                for (int q = 0; q < 4; ++q) dg[q][p] = cmod(acc[q], m, rm);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) dg[q][0] -= 128.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) V[q] = (double)dg[q][kSlots - 1];
#pragma unroll
    for (int j = kSlots - 2; j >= 0; --j) {
        const double m = (double)T->mod[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) V[q] = fma(m, V[q], (double)dg[q][j]);
    }
}

}  // namespace chain
}  // namespace oz2
