// oz2_small.hip -- Ozaki scheme II fused into one kernel for products with a
// short inner dimension (k <= 32), batched: every step of the method for a
// 16 x 16 tile of one product runs in one wavefront's registers.
//
// Method ("Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc
// GPUs: Ozaki Scheme II on the Xe2 Architecture", Sec. 2.3 and Sec. 4): row
// and column exponents over the whole of k (Sec. 4.1), integerization and
// exact residues from byte limbs (Sec. 2.3, Sec. 4.2), s exact INT8 products
// (Sec. 4.3), CRT in 16-bit limbs with the quotient estimated in 16.16 fixed
// point (the page sums FP32 products; both give the same q under its 1/4
// margin) and one correctly rounded conversion (Sec. 4.4).  The workload it serves is the chained tensor mode
// product ("You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode
// Products", Sec. 2.1 Eq. (5) and Sec. 5.1, OzII-Composed): every mode is a
// batch of small products with one shared operator, whose row (column)
// exponents are the per-fiber and per-operator-row scales of that page.
//
// Layout of the work: one wavefront per 16 x 16 output tile, with all of k.
// Lane l holds the vector l mod 16 of the tile (a row of op(A), a column of
// op(B)) at k = 8 (l / 16) .. + 7, i.e. exactly the 8 bytes it feeds to
// v_mfma_i32_16x16x32_i8 for one modulus; the tile's exponents come from a
// max over the 8 values and the three other lanes of the same vector.  After
// the MFMA of modulus t, lane l holds C^(t) at rows 4 (l / 16) + e of column
// l mod 16; the residue is reduced and added into that entry's CRT limbs at
// once, so no residue ever leaves the registers.  A wavefront walks a
// contiguous run of tiles; a tile operand equal to the previous tile's
// (a shared operator, stride 0) is not loaded or encoded again.  Reads A, B
// (and C when beta != 0) once from HBM and writes C once.
//
// For k <= 16 (the tensor chain's modes) half of the instruction's k would be
// zero padding, and so would half of every lane's encode work.  There a
// wavefront takes two tiles at a time instead: lanes 0-31 hold the first
// tile's k = 0..15, lanes 32-63 the second's, and each tile's products use
// op(A) with the other half's lanes zeroed (PAIR below).
#include "oz2_device.h"
#include "oz2_internal.h"

namespace oz2 {
namespace {

using namespace dev;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));

// the 8 values of lane l: vector v, k = 8 kq .. 8 kq + 7 (zero outside)
__device__ __forceinline__ void load8(const double* X, int64_t ld, bool contig, int64_t v, int64_t nvec,
                                      int64_t k, int kq, double x[8]) {
    const bool vok = v < nvec;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t p = 8 * kq + e;
        x[e] = 0.0;
        if (vok && p < k) x[e] = contig ? X[v * ld + p] : X[v + p * ld];
    }
}

// per-modulus constants, staged in LDS once per block: read at uniform
// addresses where used, so they neither occupy SGPRs nor spill into VGPR lanes.
// Past the last modulus every field is zero.
struct ModConst {
    float fm, frcp, foffb;          // m, fl32(1 / m), residue_word's offset
    uint32_t K128;                  // K_m + 128 (residue_word)
    uint32_t c4[kExtWords];
    int32_t mu;                     // ceil(2^29 / m) (acc_mod)
    int32_t negm;                   // -m
};
constexpr int kTableWords = (kMaxS / 2) * kMaxLimb16 + kMaxLimb16 + kMaxS / 2;
struct SmallConsts {
    ModConst q[kMaxS + 1];
    uint32_t W2[kMaxS / 2][kMaxLimb16];
    uint32_t M16[kMaxLimb16];
    uint32_t Y2[kMaxS / 2];
};
static_assert(sizeof(SmallConsts) == sizeof(ModConst) * (kMaxS + 1) + 4 * kTableWords, "table layout");

// exponent of the vector held by lanes l, l^16, l^32, l^48 (PAIR: l, l^16,
// the lanes of one tile) and the residue bytes of this lane's 8 values for
// every modulus (byte e = k 8 kq + e)
template <int SMAX, bool EXT, bool PAIR>
__device__ __forceinline__ void encode8(const double x[8], const SmallParams& P, const SmallConsts& Q,
                                        long frag[SMAX], int& D, bool& bad) {
    uint64_t mx = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = max(mx, abs_bits(x[e]));
    unsigned long long o = __shfl_xor((unsigned long long)mx, 16);
    mx = mx > o ? mx : o;
    if (!PAIR) {
        o = __shfl_xor((unsigned long long)mx, 32);
        mx = mx > o ? mx : o;
    }
    D = scale_of(mx, P.t, bad);
    Limbs<EXT> L[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) L[e] = make_limbs<EXT>(x[e], D, bad);
#pragma unroll
    for (int t = 0; t < SMAX; ++t) {
        if (t < P.s) {
            const ModConst& C = Q.q[t];
            // the first modulus is 256: the low byte of a_hat
            const uint32_t w0 = t == 0 ? low_byte_word<EXT>(L) : residue_word<EXT>(L, C.K128, C.c4, C.fm, C.frcp, C.foffb);
            const uint32_t w1 =
                t == 0 ? low_byte_word<EXT>(L + 4) : residue_word<EXT>(L + 4, C.K128, C.c4, C.fm, C.frcp, C.foffb);
            frag[t] = (long)((uint64_t)w0 | ((uint64_t)w1 << 32));
        }
    }
}

// A residue of a product acc (|acc| <= 2^19: k <= 32 terms of magnitude
// <= 2^14) modulo m <= 255, as r = acc - q m with q = floor(8 acc mu / 2^32),
// mu = ceil(2^29 / m) < 2^22: v_mul_hi_i32_i24 of 8 acc (|8 acc| <= 2^22
// fits its signed 24-bit operand) and one v_mad_i32_i24, three full-rate
// integer instructions.  acc mu / 2^29 = acc / m + acc d / 2^29 with
// 0 <= d < 1, an error below 2^-10 in magnitude, while acc / m lies at least
// 1/m > 2^-10 from the next integer above it, and from the one below it
// unless it is an integer itself: so q = floor(acc / m), except that a
// negative multiple of m gives q one less and r = m.  Hence r in [0, m], r
// congruent to acc: the CRT sums below take any representative <= 255 (a
// residue m adds m W_t, a multiple of M, to the sum and exactly y_t to the
// quotient estimate, whose error bound holds for every r <= 255), so c_hat
// is unchanged.  The first modulus, 256, is the low byte of acc instead.
// Past the last modulus (all constants 0) acc = 0 and r = 0.
// (Written as instructions: the compiler would otherwise pick the
// quarter-rate 32-bit v_mul_hi_i32 and v_mad_u64_u32.)
__device__ __forceinline__ uint32_t acc_mod(int32_t acc, const ModConst& C) {
    int32_t q, r;
    asm("v_mul_hi_i32_i24 %0, %1, %2" : "=v"(q) : "v"(acc << 3), "v"(C.mu));
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(q), "v"(C.negm), "v"(acc));
    return (uint32_t)r;
}

// PAIR (k <= 16): the instruction's k of 32 holds two tiles.  Lanes 0-31
// carry tile n at k = 0..15 and lanes 32-63 carry tile n + 1 there, so every
// lane encodes useful values; the product of tile n + h takes the lanes of
// half h of op(A) and zeros in the other half, which removes the other
// tile's terms from the sum.
// Occupancy: 3 wavefronts per SIMD up to 16 moduli (at most 168 registers;
// with 16 moduli the compiler spills about 50 bytes per lane, and the chain's
// modes still run 4% faster than at 2), 2 up to 20, 1 beyond.
template <int NL, bool BETA, bool PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NL >= 6 ? 1 : NL >= 5 ? 2 : 3))) void small_gemm_kernel(SmallParams P) {
    constexpr int SMAX = 4 * NL;     // N_L words hold products of up to 4 N_L moduli <= 256
    constexpr bool EXT = NL >= 5;    // t > 61 is only reachable with more than 16 moduli
    constexpr int STEP = PAIR ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t first = wave * P.tiles_per_wave;
    const int64_t last = min(first + (int64_t)P.tiles_per_wave, P.tiles_total);
    const int vi = lane & 15;
    const int kq = PAIR ? (lane >> 4) & 1 : lane >> 4;  // k = 8 kq .. 8 kq + 7 of the lane's tile
    const int half = PAIR ? lane >> 5 : 0;              // which tile of the pair the lane carries
    const int64_t per_batch = (int64_t)P.tiles_m * P.tiles_n;

    __shared__ SmallConsts Q;
    {
        // stage the constant tables (a few hundred words) in LDS
        const int i = threadIdx.x;
        if (i <= kMaxS) {
            ModConst c{};
            if (i < P.s) {
                c.fm = (float)P.mod[i];
                c.frcp = P.frcp[i];
                c.foffb = P.foffb[i];
                c.mu = (int32_t)((536870912u + P.mod[i] - 1) / P.mod[i]);
                c.negm = -(int32_t)P.mod[i];
                c.K128 = P.K[i] + 128u;
#pragma unroll
                for (int l = 0; l < kExtWords; ++l) c.c4[l] = P.c[i][l];
            }
            Q.q[i] = c;
        }
        for (int j = i; j < kTableWords; j += blockDim.x) {
            uint32_t v;
            if (j < (kMaxS / 2) * kMaxLimb16) v = P.W2[j / kMaxLimb16][j % kMaxLimb16];
            else if (j < (kMaxS / 2 + 1) * kMaxLimb16) v = P.M16[j - (kMaxS / 2) * kMaxLimb16];
            else v = P.Y2[j - (kMaxS / 2 + 1) * kMaxLimb16];
            (&Q.W2[0][0])[j] = v;
        }
        __syncthreads();
    }

    // fragments past the last modulus stay zero, so that the moduli can be
    // taken in pairs without a guard
    long fa[SMAX], fb[SMAX];
#pragma unroll
    for (int t = 0; t < SMAX; ++t) fa[t] = fb[t] = 0;
    int DA = 0, EB = 0;
    bool badA = false, badB = false;
    // operand tiles held in fa / fb, for the first and the second tile of a pair
    int64_t keyA0 = -1, keyA1 = -1, keyB0 = -1, keyB1 = -1;

    // batch entry and tile coordinates (wave-uniform: scalar registers), one
    // division at the start of the run, then stepped tile by tile
    int64_t cb = first / per_batch, ctm = 0, ctn = 0;
    {
        const int64_t rem = first - cb * per_batch;
        ctm = rem / P.tiles_n;
        ctn = rem - ctm * P.tiles_n;
    }
    auto step = [&](int64_t& b, int64_t& tm, int64_t& tn) {
        if (++tn == P.tiles_n) {
            tn = 0;
            if (++tm == P.tiles_m) {
                tm = 0;
                ++b;
            }
        }
    };

    for (int64_t tile = first; tile < last; tile += STEP) {
        // keeps the LDS constant reads inside the loop (no hoisting into registers)
        asm volatile("" ::: "memory");
        // a lone last tile fills both halves with itself
        const int64_t tile1 = (PAIR && tile + 1 < last) ? tile + 1 : tile;
        const int64_t b0 = cb, tm0 = ctm, tn0 = ctn;
        int64_t b1 = b0, tm1 = tm0, tn1 = tn0;
        if (tile1 != tile) step(b1, tm1, tn1);
        cb = b1;
        ctm = tm1;
        ctn = tn1;
        step(cb, ctm, ctn);
        // the tile whose values this lane loads
        const int64_t b = half ? b1 : b0, tm = half ? tm1 : tm0, tn = half ? tn1 : tn0;
        // operand tiles as cache keys: rows tm.. of op(A_b), columns tn.. of
        // op(B_b) (a zero stride shares the operand across the batch)
        const int64_t ka0 = (P.strideA ? b0 : 0) * P.tiles_m + tm0, ka1 = (P.strideA ? b1 : 0) * P.tiles_m + tm1;
        if (ka0 != keyA0 || ka1 != keyA1) {
            // rows tm.. of op(A_b): contiguous in memory for op = T
            double x[8];
            load8(P.A + b * P.strideA, P.lda, P.transa != 0, tm * 16 + vi, P.m, P.k, kq, x);
            encode8<SMAX, EXT, PAIR>(x, P, Q, fa, DA, badA);
            keyA0 = ka0;
            keyA1 = ka1;
        }
        const int64_t kb0 = (P.strideB ? b0 : 0) * P.tiles_n + tn0, kb1 = (P.strideB ? b1 : 0) * P.tiles_n + tn1;
        if (kb0 != keyB0 || kb1 != keyB1) {
            // columns tn.. of op(B_b): contiguous for op = N
            double x[8];
            load8(P.B + b * P.strideB, P.ldb, P.transb == 0, tn * 16 + vi, P.n, P.k, kq, x);
            encode8<SMAX, EXT, PAIR>(x, P, Q, fb, EB, badB);
            keyB0 = kb0;
            keyB1 = kb1;
        }

#pragma unroll
        for (int h = 0; h < STEP; ++h) {
            if (h == 1 && tile1 == tile) break;
            const long amask = (!PAIR || half == h) ? -1L : 0L;
            Crt<NL> acc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e].init();
            const v4i zero = {0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < SMAX; t += 2) {
                if (t < P.s) {
                    // past the last modulus: zero fragments, constants and limbs
                    const ModConst& C0 = Q.q[t];
                    const ModConst& C1 = Q.q[t + 1];
                    const v4i ca = __builtin_amdgcn_mfma_i32_16x16x32_i8(fa[t] & amask, fb[t], zero, 0, 0, 0);
                    const v4i cb = __builtin_amdgcn_mfma_i32_16x16x32_i8(fa[t + 1] & amask, fb[t + 1], zero, 0, 0, 0);
                    // residues of moduli t, t + 1 as the 16-bit halves of one
                    // word; modulus 256 (always the first) is the low byte of the sum
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = t == 0 ? ((uint32_t)ca[e] & 0xffu) : acc_mod(ca[e], C0);
                        acc[e].add2((acc_mod(cb[e], C1) << 16) | lo, Q.Y2[t >> 1], Q.W2[t >> 1]);
                    }
                }
            }

            // entry (row 4 (lane / 16) + e, column vi) of tile + h; the
            // exponents of its rows and column sit in the lanes of half h
            const int64_t ob = h ? b1 : b0, otm = h ? tm1 : tm0, otn = h ? tn1 : tn0;
            const int64_t col = otn * 16 + vi;
            const int Ec = PAIR ? __shfl(EB, 32 * h + vi) : EB;
            const bool badc = PAIR ? __shfl((int)badB, 32 * h + vi) != 0 : badB;
            // the lane's four rows are contiguous in C: two 16-byte stores
            // when they are all in range and 16-byte aligned
            const int64_t row0 = otm * 16 + 4 * (lane >> 4);
            double* c0 = P.C + ob * P.strideC + row0 + col * P.ldc;
            const bool vec = row0 + 3 < P.m && col < P.n && (((uintptr_t)c0 & 15u) == 0);
            double out[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * (lane >> 4) + e;
                const int Dr = __shfl(DA, 32 * h + r);
                const bool badr = __shfl((int)badA, 32 * h + r) != 0;
                uint32_t w[NL];
                acc[e].finish(Q.M16, w);
                double x = words_to_double<NL>(w, Dr + Ec);
                if (badr || badc) x = __builtin_nan("");
                const bool in = row0 + e < P.m && col < P.n;
                const double t1 = P.alpha * x;
                if (BETA) {
                    const double t2 = P.beta * (in ? c0[e] : 0.0);
                    out[e] = t1 + t2;
                } else {
                    out[e] = t1;
                }
            }
            if (vec) {
                ((v2d*)c0)[0] = v2d{out[0], out[1]};
                ((v2d*)c0)[1] = v2d{out[2], out[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (row0 + e < P.m && col < P.n) c0[e] = out[e];
            }
        }
    }
}

template <int NL, bool PAIR>
hipError_t small_go(const SmallParams& P, bool beta, hipStream_t st) {
    const int64_t waves = (P.tiles_total + P.tiles_per_wave - 1) / P.tiles_per_wave;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (beta)
        hipLaunchKernelGGL((small_gemm_kernel<NL, true, PAIR>), grid, block, 0, st, P);
    else
        hipLaunchKernelGGL((small_gemm_kernel<NL, false, PAIR>), grid, block, 0, st, P);
    return hipGetLastError();
}

template <int NL>
hipError_t small_go(const SmallParams& P, bool beta, hipStream_t st) {
    return P.k <= 16 ? small_go<NL, true>(P, beta, st) : small_go<NL, false>(P, beta, st);
}

}  // namespace

hipError_t launch_small_gemm(SmallParams P, int NL, bool beta_nonzero, hipStream_t st) {
    if (P.k < 1 || P.k > kSmallMaxK || P.m < 1 || P.n < 1 || P.batch < 1) return hipErrorInvalidValue;
    if (P.s < kMinS || P.s > 4 * NL || NL < 2 || NL > kMaxNL) return hipErrorInvalidValue;
    P.tiles_m = (int)((P.m + 15) / 16);
    P.tiles_n = (int)((P.n + 15) / 16);
    P.tiles_total = P.batch * P.tiles_m * P.tiles_n;
    // about 8 wavefronts per SIMD over the whole device, each on a contiguous run
    const int64_t target_waves = 8192;
    P.tiles_per_wave = (int)((P.tiles_total + target_waves - 1) / target_waves);
    if (P.tiles_per_wave < 1) P.tiles_per_wave = 1;
    // k <= 16 takes tiles in pairs: an even run leaves no half-empty pair
    // except at the very end
    if (P.k <= 16) P.tiles_per_wave += P.tiles_per_wave & 1;
    switch (NL) {
        case 2: return small_go<2>(P, beta_nonzero, st);
        case 3: return small_go<3>(P, beta_nonzero, st);
        case 4: return small_go<4>(P, beta_nonzero, st);
        case 5: return small_go<5>(P, beta_nonzero, st);
        default: return small_go<6>(P, beta_nonzero, st);
    }
}

}  // namespace oz2
