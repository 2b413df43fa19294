// oz2_small.hip -- Ozaki scheme II fused into one kernel for products with a
// short inner dimension (k <= 32), batched: every step of the method for a
// 16 x 16 tile of one product runs in one wavefront's registers.
//
// Method ("Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc
// GPUs: Ozaki Scheme II on the Xe2 Architecture", Sec. 2.3 and Sec. 4): row
// and column exponents over the whole of k (Sec. 4.1), integerization and
// integer-only residues (Sec. 2.3, Sec. 4.2), s exact INT8 products (Sec. 4.3),
// CRT with an FP32 quotient in 16-bit limbs and one correctly rounded
// conversion (Sec. 4.4).  The workload it serves is the chained tensor mode
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
#include "oz2_device.h"
#include "oz2_internal.h"

namespace oz2 {
namespace {

using namespace dev;
typedef int v4i __attribute__((ext_vector_type(4)));

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
// addresses where used, so they neither occupy SGPRs nor spill into VGPR lanes
struct ModConst {
    uint32_t mod, rcp_lo, rcp_hi, K;  // rcp: the two words of fl64(1 / m)
    uint32_t c4[kExtWords];
    float frcp, foff;
};
static_assert(offsetof(ModConst, foff) == 4 * (5 + kExtWords), "staging order of ModConst");
struct SmallConsts {
    ModConst q[kMaxS + 1];            // one zeroed entry past the last modulus
    uint32_t W2[kMaxS / 2][kMaxLimb16];
    uint32_t M16[kMaxLimb16];
    uint32_t Y2[kMaxS / 2];
};
static_assert(offsetof(SmallConsts, Y2) == offsetof(SmallConsts, M16) + 4 * kMaxLimb16, "staging order");

// exponent of the vector held by lanes l, l^16, l^32, l^48 and the residue
// bytes of this lane's 8 values for every modulus (byte e = k 8 kq + e)
template <int SMAX, bool EXT>
__device__ __forceinline__ void encode8(const double x[8], const SmallParams& P, const SmallConsts& Q,
                                        long frag[SMAX], int& D, bool& bad) {
    uint64_t mx = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = max(mx, abs_bits(x[e]));
    unsigned long long o = __shfl_xor((unsigned long long)mx, 16);
    mx = mx > o ? mx : o;
    o = __shfl_xor((unsigned long long)mx, 32);
    mx = mx > o ? mx : o;
    D = scale_of(mx, P.t, bad);
    Limbs<EXT> L[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) L[e] = make_limbs<EXT>(x[e], D, bad);
#pragma unroll
    for (int t = 0; t < SMAX; ++t) {
        if (t < P.s) {
            const ModConst& C = Q.q[t];
            const float m = (float)C.mod;
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t r = (uint32_t)centred_residue<EXT>(L[e], C.K, C.c4, m, C.frcp, C.foff);
                w[e >> 2] |= (r & 0xffu) << (8 * (e & 3));
            }
            frag[t] = (long)((uint64_t)w[0] | ((uint64_t)w[1] << 32));
        }
    }
}

// INT32 accumulator -> [0, m), exact in FP64 as in the residue GEMM:
// r = acc - m floor((acc + 1/2) / m), |acc| < 2^31
__device__ __forceinline__ uint32_t acc_mod(int32_t acc, const ModConst& C) {
    const double a = (double)acc, m = (double)C.mod;
    const double rcp = __hiloint2double((int)C.rcp_hi, (int)C.rcp_lo);
    return (uint32_t)(int)fma(-m, floor(fma(a, rcp, 0.5 * rcp)), a);
}

template <int NL, bool BETA>
__global__ __launch_bounds__(256) void small_gemm_kernel(SmallParams P) {
    constexpr int SMAX = 4 * NL;     // N_L words hold products of up to 4 N_L moduli <= 256
    constexpr bool EXT = NL >= 5;    // t > 61 is only reachable with more than 16 moduli
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t first = wave * P.tiles_per_wave;
    const int64_t last = min(first + (int64_t)P.tiles_per_wave, P.tiles_total);
    const int vi = lane & 15, kq = lane >> 4;
    const int64_t per_batch = (int64_t)P.tiles_m * P.tiles_n;

    __shared__ SmallConsts Q;
    {
        // stage the constant tables (a few hundred words) in LDS
        uint32_t* dst = (uint32_t*)&Q;
        constexpr int nq = (int)(sizeof(ModConst) / 4);
        for (int i = threadIdx.x; i < (int)(sizeof(SmallConsts) / 4); i += blockDim.x) {
            uint32_t v = 0u;
            if (i < (kMaxS + 1) * nq) {
                const int t = i / nq, f = i % nq;
                if (t < P.s) {
                    if (f == 0) v = P.mod[t];
                    else if (f == 1) v = (uint32_t)__double2loint(P.rcp[t]);
                    else if (f == 2) v = (uint32_t)__double2hiint(P.rcp[t]);
                    else if (f == 3) v = P.K[t];
                    else if (f < 4 + kExtWords) v = P.c[t][f - 4];
                    else if (f == 4 + kExtWords) v = __float_as_uint(P.frcp[t]);
                    else v = __float_as_uint(P.foff[t]);
                }
            } else if (i < (kMaxS + 1) * nq + (kMaxS / 2) * kMaxLimb16) {
                const int j = i - (kMaxS + 1) * nq;
                v = P.W2[j / kMaxLimb16][j % kMaxLimb16];
            } else if (i < (kMaxS + 1) * nq + (kMaxS / 2) * kMaxLimb16 + kMaxLimb16) {
                v = P.M16[i - (kMaxS + 1) * nq - (kMaxS / 2) * kMaxLimb16];
            } else {
                v = P.Y2[i - (kMaxS + 1) * nq - (kMaxS / 2 + 1) * kMaxLimb16];
            }
            dst[i] = v;
        }
        __syncthreads();
    }

    long fa[SMAX], fb[SMAX];
    int DA = 0, EB = 0;
    bool badA = false, badB = false;
    int64_t keyA = -1, keyB = -1;

    for (int64_t tile = first; tile < last; ++tile) {
        // keeps the LDS constant reads inside the loop (no hoisting into registers)
        asm volatile("" ::: "memory");
        const int64_t b = tile / per_batch;
        const int64_t rem = tile - b * per_batch;
        const int64_t tm = rem / P.tiles_n, tn = rem - tm * P.tiles_n;
        const int64_t i0 = tm * 16, j0 = tn * 16;
        // rows i0.. of op(A_b): contiguous in memory for op = T
        const int64_t ka = (P.strideA ? b : 0) * P.tiles_m + tm;
        if (ka != keyA) {
            double x[8];
            load8(P.A + b * P.strideA, P.lda, P.transa != 0, i0 + vi, P.m, P.k, kq, x);
            encode8<SMAX, EXT>(x, P, Q, fa, DA, badA);
            keyA = ka;
        }
        // columns j0.. of op(B_b): contiguous for op = N
        const int64_t kb = (P.strideB ? b : 0) * P.tiles_n + tn;
        if (kb != keyB) {
            double x[8];
            load8(P.B + b * P.strideB, P.ldb, P.transb == 0, j0 + vi, P.n, P.k, kq, x);
            encode8<SMAX, EXT>(x, P, Q, fb, EB, badB);
            keyB = kb;
        }

        Crt<NL> acc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e].init();
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < SMAX; t += 2) {
            if (t < P.s) {
                const v4i ca = __builtin_amdgcn_mfma_i32_16x16x32_i8(fa[t], fb[t], zero, 0, 0, 0);
                const bool two = t + 1 < P.s;
                const v4i cb = two ? __builtin_amdgcn_mfma_i32_16x16x32_i8(fa[t + 1], fb[t + 1], zero, 0, 0, 0) : zero;
                const ModConst& C0 = Q.q[t];
                const ModConst& C1 = Q.q[t + 1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t ra = acc_mod(ca[e], C0);
                    const uint32_t rb = two ? acc_mod(cb[e], C1) : 0u;
                    acc[e].add2(ra, rb, Q.Y2[t >> 1], Q.W2[t >> 1]);
                }
            }
        }

        // entry (row 4 kq + e, column vi) of the tile
        const int64_t col = j0 + vi;
        double* Cb = P.C + b * P.strideC;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * kq + e;
            const int Dr = __shfl(DA, r);
            const bool badr = __shfl((int)badA, r) != 0;
            uint32_t w[NL];
            acc[e].finish(Q.M16, w);
            double x = words_to_double<NL>(w, Dr + EB);
            if (badr || badB) x = __builtin_nan("");
            const int64_t row = i0 + r;
            if (row < P.m && col < P.n) {
                double* c = Cb + row + col * P.ldc;
                const double t1 = P.alpha * x;
                if (BETA) {
                    const double t2 = P.beta * c[0];
                    c[0] = t1 + t2;
                } else {
                    c[0] = t1;
                }
            }
        }
    }
}

template <int NL>
hipError_t small_go(const SmallParams& P, bool beta, hipStream_t st) {
    const int64_t waves = (P.tiles_total + P.tiles_per_wave - 1) / P.tiles_per_wave;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (beta)
        hipLaunchKernelGGL((small_gemm_kernel<NL, true>), grid, block, 0, st, P);
    else
        hipLaunchKernelGGL((small_gemm_kernel<NL, false>), grid, block, 0, st, P);
    return hipGetLastError();
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
    switch (NL) {
        case 2: return small_go<2>(P, beta_nonzero, st);
        case 3: return small_go<3>(P, beta_nonzero, st);
        case 4: return small_go<4>(P, beta_nonzero, st);
        case 5: return small_go<5>(P, beta_nonzero, st);
        default: return small_go<6>(P, beta_nonzero, st);
    }
}

}  // namespace oz2
