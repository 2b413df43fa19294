// oz2_device.h -- device arithmetic shared by the kernels of oz2: exact
// scaling and integerization, residues from byte-limb dot products, CRT
// reconstruction in 16-bit limbs and the correctly rounded conversion back
// to double.
//
// "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs:
// Ozaki Scheme II on the Xe2 Architecture":
//   Sec. 4.1  D_i = t - e(max_p |a_ip|)            -> scale_of()
//   Sec. 2.3  a_hat = rint(a 2^D), ties to even     -> make_limbs()
//   Sec. 4.2  residues from limbs of a_hat + 2^62 with precomputed
//             2^(limb position) mod m and a constant K_m; the page uses
//             21-bit limbs, here byte limbs read four at a time by
//             v_dot4_u32_u8 (the same congruence) -> residue_word();
//             modulo 256 the low byte of a_hat     -> low_byte_word()
//   Sec. 4.4  the quotient q = rint(sum r_t y_t/m_t): the page sums FP32
//             products; here the sum is taken in 16.16 fixed point,
//             sum r_t round(2^16 y_t/m_t) by v_dot2_u32_u16, within 0.05 of
//             Z/M, well inside the page's 1/4 margin, so q is the same;
//             c_hat = sum r_t W_t - q M in 16-bit limbs (two moduli per
//             v_dot2), one carry pass, top 64 bits + sticky rounded once
//             to double -> Crt, words_to_double()
// Device-only; included by the .hip translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "oz2_plan.h"

namespace oz2 {
namespace dev {

constexpr uint64_t kAbsMask = 0x7FFFFFFFFFFFFFFFull;
constexpr uint64_t kInfBits = 0x7FF0000000000000ull;

__device__ __forceinline__ uint64_t abs_bits(double x) {
    return (uint64_t)__double_as_longlong(x) & kAbsMask;
}

// e(x) with 2^(e-1) <= x < 2^e for a positive finite double given by its bits
__device__ __forceinline__ int frexp_exp_bits(uint64_t b) {
    int eb = (int)(b >> 52);
    return eb ? eb - 1022 : (64 - __clzll((long long)b)) - 1074;
}

// D = t - e(amax); 0 for an all-zero vector; `bad` for a non-finite one
__device__ __forceinline__ int scale_of(uint64_t amax, int t, bool& bad) {
    bad = amax >= kInfBits;
    return (bad || amax == 0) ? 0 : t - frexp_exp_bits(amax);
}

// residue limbs of one element: the 32-bit words of a_hat + 2^62 (standard
// width) or a_hat + 2^104 (extended width), each read as four byte limbs;
// the sign is absorbed by the bias
template <bool EXT>
struct Limbs {
    uint32_t w[EXT ? kExtWords : kStdWords];
};

// In FP64, exactly and branch-free: a 2^D is exact (a value that underflows
// is below 1/2 and rints to 0 either way) and rint rounds ties to even.  The
// integer x (|x| <= 2^61, or 2^100 at the extended width) then splits
// exactly into 32-bit words by floor(x 2^-32) and x - hi 2^32 (one fma, whose
// exact result 0 <= lo < 2^32 is representable); the bias 2^62 (2^104) adds
// 2^30 (2^8) to the signed top word.  Full-rate FP64 on this GPU makes this
// cheaper than shifting and rounding the significand in integers.
template <bool EXT>
__device__ __forceinline__ Limbs<EXT> make_limbs(double a, int D, bool zero) {
    Limbs<EXT> L;
    double x = __builtin_rint(__builtin_ldexp(zero ? 0.0 : a, D));
    constexpr int W = EXT ? kExtWords : kStdWords;
#pragma unroll
    for (int i = 0; i + 1 < W; ++i) {
        const double hi = __builtin_floor(x * 0x1p-32);
        L.w[i] = (uint32_t)__builtin_fma(hi, -0x1p32, x);
        x = hi;
    }
    L.w[W - 1] = (uint32_t)((int32_t)x + (EXT ? (1 << 8) : (1 << 30)));
    return L;
}

// v' = K128 + sum_j b_j (2^(8j) mod m) over the bytes b_j of a_hat + 2^62
// (or 2^104), four bytes per v_dot4_u32_u8 against c4[p] (byte j of c4[p] is
// 2^(32p + 8j) mod m).  With K128 = K_m + 128 and K_m = (-2^62) mod m (or
// (-2^104) mod m), v' = a_hat + 128 (mod m), and v' < 16 255^2 + 2^9 < 2^20.
template <bool EXT>
__device__ __forceinline__ uint32_t dot_limbs(const Limbs<EXT>& L, uint32_t K128, const uint32_t* c4) {
    uint32_t v = K128;
#pragma unroll
    for (int p = 0; p < (EXT ? kExtWords : kStdWords); ++p) v = __builtin_amdgcn_udot4(L.w[p], c4[p], v, false);
    return v;
}

// offset-binary residue: f = v' - m floor((v' + hb + 1/2 - 128) / m) = r + 128
// in [0, 255], where r is the centred residue of v' - 128 (hb = h, or 128 for
// m = 256, whose window [-128, 127] has the same bytes as [-127, 128]).  The
// floor argument is the one of centred_residue, and for v' < 2^21 and
// m <= 256 the FP32 evaluation is within 2^-3 / m + 2^-11 < 1 / (2m) of it,
// so f is exact.
__device__ __forceinline__ float offset_residue(uint32_t v, float m, float rcp, float offb) {
    const float vf = (float)v;
    return fmaf(-m, floorf(fmaf(vf, rcp, offb)), vf);
}

// the centred residues of four elements (one modulus) as the four bytes of a
// word, byte e from L[e]: v_cvt_pk_u8_f32 puts each offset-binary residue
// r + 128 in its byte, and XOR 0x80 per byte turns it into the two's
// complement byte of r.
template <bool EXT>
__device__ __forceinline__ uint32_t residue_word(const Limbs<EXT>* L, uint32_t K128, const uint32_t* c4, float m,
                                                 float rcp, float offb) {
    uint32_t w = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        w = __builtin_amdgcn_cvt_pk_u8_f32(offset_residue(dot_limbs<EXT>(L[e], K128, c4), m, rcp, offb), e, w);
    return w ^ 0x80808080u;
}

// residues modulo 256 in the window [-128, 127] of four elements: the low
// byte of a_hat in two's complement, which is byte 0 of the first word (the
// bias changes only the top word)
template <bool EXT>
__device__ __forceinline__ uint32_t low_byte_word(const Limbs<EXT>* L) {
    return (L[0].w[0] & 0xffu) | ((L[1].w[0] & 0xffu) << 8) | ((L[2].w[0] & 0xffu) << 16) | (L[3].w[0] << 24);
}

// the same for a complex element's real and imaginary parts and their sum
// (3M operands): the sum's v' is v'_re + v'_im - 128 < 2^21, which needs no
// further dot products
template <bool EXT>
__device__ __forceinline__ void residue_words3(const Limbs<EXT>* Lr, const Limbs<EXT>* Li, uint32_t K128,
                                               const uint32_t* c4, float m, float rcp, float offb, uint32_t& wr,
                                               uint32_t& wi, uint32_t& ws) {
    wr = wi = ws = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t vr = dot_limbs<EXT>(Lr[e], K128, c4), vi = dot_limbs<EXT>(Li[e], K128, c4);
        wr = __builtin_amdgcn_cvt_pk_u8_f32(offset_residue(vr, m, rcp, offb), e, wr);
        wi = __builtin_amdgcn_cvt_pk_u8_f32(offset_residue(vi, m, rcp, offb), e, wi);
        ws = __builtin_amdgcn_cvt_pk_u8_f32(offset_residue(vr + vi - 128u, m, rcp, offb), e, ws);
    }
    wr ^= 0x80808080u;
    wi ^= 0x80808080u;
    ws ^= 0x80808080u;
}

// c_hat from the residues of one entry, accumulated over the moduli two at a
// time with one v_dot2_u32_u16 per limb: the 16-bit limbs of
// r_t W_t + r_(t+1) W_(t+1) (r and the two limbs of W packed as 16-bit
// pairs; every term r W16 < 2^8 2^16, so the limb sums of 24 moduli stay
// below 2^29), and the quotient estimate z = sum r_t y_t / m_t in 16.16
// fixed point, sum r_t Y_t with Y_t = round(2^16 y_t / m_t) < 2^16.
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

template <int NL>
struct Crt {
    static constexpr int L16 = 2 * NL;
    uint32_t zq;
    uint32_t L[L16];
    __device__ __forceinline__ void init() {
        zq = 0u;
#pragma unroll
        for (int l = 0; l < L16; ++l) L[l] = 0u;
    }
    // moduli t, t+1: residues packed as ra | rb << 16 (rb = 0 past the last
    // modulus, where the high halves of Y2 and W2 are 0 too);
    // Y2 = Y_t | Y_(t+1) << 16, W2[l] = W16[t][l] | W16[t+1][l] << 16
    __device__ __forceinline__ void add2(uint32_t packed, uint32_t Y2, const uint32_t* W2) {
        const v2u16 r = __builtin_bit_cast(v2u16, packed);
        zq = __builtin_amdgcn_udot2(r, __builtin_bit_cast(v2u16, Y2), zq, false);
#pragma unroll
        for (int l = 0; l < L16; ++l)
            L[l] = __builtin_amdgcn_udot2(r, __builtin_bit_cast(v2u16, W2[l]), L[l], false);
    }
    __device__ __forceinline__ void add2(uint32_t ra, uint32_t rb, uint32_t Y2, const uint32_t* W2) {
        add2(ra | (rb << 16), Y2, W2);
    }
    // c_hat = Z - q M mod 2^(32 NL), two's complement words.  |q| <= 24 * 256
    // and M16 < 2^16, so q M16 fits the 24-bit multiplier; one carry pass.
    __device__ __forceinline__ void finish(const uint32_t* M16, uint32_t w[NL]) {
        // |zq 2^-16 - Z/M| <= sum r_t |Y_t 2^-16 - y_t/m_t| <= 24 255 2^-17 < 0.05
        // and Z/M lies within 1/4 of q (|c_hat| <= M/4): rounding zq gives q
        const int32_t q = (int32_t)((zq + 0x8000u) >> 16);
        int32_t carry = 0;
        uint32_t lo16 = 0;
#pragma unroll
        for (int l = 0; l < L16; ++l) {
            const int32_t c = (int32_t)L[l] + __mul24(-q, (int32_t)M16[l]) + carry;
            if (l & 1)
                w[l >> 1] = lo16 | ((uint32_t)c << 16);
            else
                lo16 = (uint32_t)c & 0xffffu;
            carry = c >> 16;
        }
    }
};

// RN(c * 2^-S) of a two's-complement integer c given by NL 32-bit words:
// the top 64 bits below the leading one OR-ed with a sticky bit of the rest,
// converted once with round-to-nearest-even, then scaled by a power of two
// (a second rounding only when the result is subnormal).  The magnitude by
// xor and carry; the leading word moved to the top in steps of 4, 2 and 1
// words, which a wave-uniform branch skips when every lane's top word is
// already nonzero.
template <int NL>
__device__ __forceinline__ double words_to_double(uint32_t w[NL], int S) {
    const uint32_t sgn = (uint32_t)((int32_t)w[NL - 1] >> 31);
    uint32_t c = sgn & 1u;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const uint32_t y = (w[i] ^ sgn) + c;
        c = y < c ? 1u : 0u;
        w[i] = y;
    }
    int shift = 0;
    // word shifts only when some lane's top word is zero (|c_hat| far below
    // M: rare for real data), decided by a wave vote so the branch is uniform
    if (!__all(w[NL - 1] != 0)) {
        if (NL > 4) {
            const bool z4 = (w[NL - 1] | w[NL - 2] | w[NL - 3] | w[NL - 4]) == 0;
#pragma unroll
            for (int i = NL - 1; i >= 0; --i) w[i] = z4 ? (i >= 4 ? w[i - 4] : 0u) : w[i];
            shift += z4 ? 4 : 0;
        }
        if (NL > 2) {
            const bool z2 = (w[NL - 1] | w[NL - 2]) == 0;
#pragma unroll
            for (int i = NL - 1; i >= 0; --i) w[i] = z2 ? (i >= 2 ? w[i - 2] : 0u) : w[i];
            shift += z2 ? 2 : 0;
        }
        {
            const bool z1 = w[NL - 1] == 0;
#pragma unroll
            for (int i = NL - 1; i >= 0; --i) w[i] = z1 ? (i >= 1 ? w[i - 1] : 0u) : w[i];
            shift += z1 ? 1 : 0;
        }
    }
    const uint32_t x3 = w[NL - 1];
    const int lz = __clz((int)x3);
    const uint64_t hi = ((uint64_t)x3 << 32) | w[NL - 2];
    const uint64_t lo = NL >= 4 ? (((uint64_t)w[NL - 3] << 32) | w[NL - 4]) : (NL == 3 ? ((uint64_t)w[0] << 32) : 0ull);
    uint32_t below = 0;
#pragma unroll
    for (int i = 0; i + 4 < NL; ++i) below |= w[i];
    uint64_t win = hi, rest = lo;
    if (lz) {
        win = (hi << lz) | (lo >> (64 - lz));
        rest = lo << lz;
    }
    win |= (uint64_t)((rest | below) != 0);
    // u64 -> double with a single rounding: hi*2^32 is exact, the FMA rounds once
    const double dh = (double)(uint32_t)(win >> 32);
    const double dl = (double)(uint32_t)win;
    const double d = __builtin_fma(dh, 4294967296.0, dl);
    const int e2 = 32 * (NL - 1 - shift) + 31 - lz - 63 - S;
    const double r = x3 ? __builtin_ldexp(d, e2) : 0.0;  // integer zero gives +0
    return sgn ? -r : r;
}

}  // namespace dev
}  // namespace oz2
