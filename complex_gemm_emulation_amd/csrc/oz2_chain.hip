// oz2_chain.hip -- persistent Ozaki scheme II for chained tensor mode
// products (OzII-RescaleBE): Y = X x1 A1 x2 A2 x3 A3 for a batch of
// n x n x n tensors, every step of the chain in one kernel.
//
// "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products":
//  - Sec. 5.2 and Algorithm 7: the tensor is encoded once with one exponent,
//    multiplied mode after mode on its residue planes, rescaled by g_i
//    moduli (Algorithm 1, Eq. 15) and base-extended (Algorithm 4, Eq. 26)
//    after each non-final mode, and reconstructed once;
//  - Algorithm 5: Encode (rounding to nearest, ties to even), ToRns and
//    ReconstructFP64 (centred mixed-radix digits, FP64 Horner, scaling by
//    alpha * Gamma, Eq. 28);
//  - Sec. 2.3 Eq. (11): centred residues, [v]_m in [-floor(m/2), ceil(m/2) - 1].
//
// Design (CDNA4): one block of 8 wavefronts per tensor.  The tensor's residue
// planes (up to 16 moduli x 16^3 bytes) stay in LDS for the whole chain, in
// two buffers that alternate between modes, so HBM sees each input entry
// read once and each output entry written once.  A mode product is, per
// modulus, Y^T = R^T Abar^T on v_mfma_i32_16x16x32_i8: the 256 rows of R^T
// (the fibres along the contracted index) form 16 tiles of 16 rows, two per
// wavefront; k = 16 fills half of the MFMA's 32.  Each lane then holds four
// output entries of one fibre position for every modulus, and runs the
// modular reduction, the scheduled drops and the base extension on them in
// registers.  The output is stored so that the next mode's contraction
// index is the contiguous one: the four entries of a lane are four
// consecutive bytes of the next layout (one 32-bit LDS write per modulus).
//
// Moduli sit right-aligned in 16 slots, descending, so that the smallest
// (the ones dropped) are always slots 15, 14, ... at compile time; unused
// leading slots carry the modulus 1, which leaves every mixed-radix step,
// weight and Horner step unchanged.  All modular arithmetic is on exact
// small integers held as floats: [x]_m = x - m floor(x / m + 1/2), with
// fl32(x * fl32(1/m)) close enough to x/m that the floor is exact for odd m
// (|x| < 2^19 here), and exact outright for m = 256.
#include "oz2_internal.h"

namespace oz2 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSlots = kChainMaxS;  // 16
constexpr int kPlane = kChainN * kChainN * kChainN;  // 4096 entries per residue plane

__device__ __forceinline__ float cmod(float x, float m, float rm) {
    return fmaf(-m, floorf(fmaf(x, rm, 0.5f)), x);
}

// centred residue of an integer-valued double |v| <= 2^53 modulo an odd m
// (the quotient estimate can be one off; two corrections bring r into range)
__device__ __forceinline__ float dmod_odd(double v, double m, double rm) {
    const double q = rint(v * rm);
    double r = fma(-m, q, v);  // exact: |r| < 2m
    const double h = 0.5 * (m - 1.0);
    r = r > h ? r - m : r;
    r = r < -h ? r + m : r;
    return (float)r;
}

// the signed byte of entry `ent` in a word of four packed residues, as a float
__device__ __forceinline__ float unpack(uint32_t w, int ent) {
    return (float)(int)(int8_t)(w >> (8 * ent));
}


__global__ __launch_bounds__(512, 1) void chain_kernel(ChainParams P) {
    __shared__ __attribute__((aligned(16))) int8_t buf0[kSlots * kPlane];
    __shared__ __attribute__((aligned(16))) int8_t buf1[kSlots * kPlane];
    __shared__ __attribute__((aligned(16))) int8_t ops[3][kSlots][kChainN * kChainN];
    __shared__ ChainTables KT;
    __shared__ unsigned long long smax;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = P.n;
    const int64_t n3 = (int64_t)n * n * n;
    const int first = kSlots - P.s;  // first active slot
    const double* X = P.X + (int64_t)blockIdx.x * n3;
    double* Y = P.Y + (int64_t)blockIdx.x * n3;
    // stage the constant tables and the operator residues (slot order) in LDS
    // (read per use: as kernel-argument or scalar loads the compiler would
    // hoist all of them out of the loops and spill registers)
    static_assert(sizeof(ChainTables) % 4 == 0, "words");
    for (int x = tid; x < (int)(sizeof(ChainTables) / 4); x += 512)
        ((uint32_t*)&KT)[x] = ((const uint32_t*)P.tab)[x];
    const ChainTables* T = &KT;
    for (int x = tid; x < 3 * kSlots * kChainN * kChainN / 8; x += 512) {
        const int mode = x / (kSlots * 32), u = (x / 32) % kSlots, w = x % 32;
        long v = 0;
        if (u >= first) v = *(const long*)(P.ops + ((mode * kSlots + (u - first)) * kChainN * kChainN) + 8 * w);
        *(long*)(&ops[mode][u][8 * w]) = v;
    }
    if (tid == 0) smax = 0;
    __syncthreads();

    // ---------------------------------------------------------------- encode
    // thread: entries idx = 8 tid .. 8 tid + 7 of the padded 16^3 tensor,
    // idx = k1 + 16 (k2 + 16 k3) -- the mode-1 layout [slot][fibre][k1]
    const int idx0 = 8 * tid;
    const int k1_0 = idx0 & 15, k2 = (idx0 >> 4) & 15, k3 = idx0 >> 8;
    double x[8];
    unsigned long long mx = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int k1 = k1_0 + j;
        const bool in = k1 < n && k2 < n && k3 < n;
        x[j] = in ? X[k1 + (int64_t)n * (k2 + (int64_t)n * k3)] : 0.0;
        const unsigned long long bits = (unsigned long long)__double_as_longlong(x[j]) & 0x7fffffffffffffffull;
        mx = bits > mx ? bits : mx;
    }
    atomicMax(&smax, mx);
    __syncthreads();
    const unsigned long long M = smax;
    if (M >= 0x7ff0000000000000ull) {
        // a non-finite entry: the whole tensor's result is NaN
        for (int64_t i = tid; i < n3; i += 512) Y[i] = __builtin_nan("");
        return;
    }
    int e = 0;
    if (M) {
        int E = 0;
        (void)frexp(__longlong_as_double((long long)M), &E);
        e = P.b - E;
    }
    double xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xb[j] = rint(ldexp(x[j], e));  // |xb| <= 2^b
#pragma unroll 1
    for (int u = first; u < kSlots; ++u) {
        uint32_t w[2] = {0u, 0u};
        if (u == first) {
            // m = 256: the low byte of the two's-complement integer
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j >> 2] |= ((uint32_t)(int64_t)xb[j] & 0xffu) << (8 * (j & 3));
        } else {
            const double m = (double)T->mod[u], rm = 1.0 / m;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                w[j >> 2] |= ((uint32_t)(int)dmod_odd(xb[j], m, rm) & 0xffu) << (8 * (j & 3));
        }
        *(uint2*)(buf0 + u * kPlane + idx0) = make_uint2(w[0], w[1]);
    }
    __syncthreads();

    // ----------------------------------------------------------- mode loop
    const int a = lane & 15;   // MFMA row of A / column of B and of the output
    const int kq = lane >> 4;  // k group of the operands (0, 1 hold k < 16), output row group
    const int8_t* src = buf0;
    int8_t* dst = buf1;
#pragma unroll 1
    for (int mode = 0; mode < 3; ++mode) {
        const int g = P.g[mode];
        const int keep = kSlots - 1 - g;  // last slot of the reduced basis
#pragma unroll 1
        for (int tt = 0; tt < 2; ++tt) {
            const int t = wave + 8 * tt;  // tile: fibres 16 t .. 16 t + 15
            // residue products, reduced and packed: pk[u] = four entries' bytes
            uint32_t pk[kSlots];
            {
                v4i acc[kSlots];
#pragma unroll
                for (int u = 0; u < kSlots; ++u) {
                    acc[u] = v4i{0, 0, 0, 0};
                    if (u < first) continue;
                    long af = 0, bf = 0;
                    if (kq < 2) {
                        af = *(const long*)(src + u * kPlane + (16 * t + a) * kChainN + 8 * kq);
                        bf = *(const long*)(&ops[mode][u][a * kChainN + 8 * kq]);
                    }
                    acc[u] = __builtin_amdgcn_mfma_i32_16x16x32_i8(af, bf, acc[u], 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < kSlots; ++u) {
                    const float m = T->mod[u], rm = T->rmod[u];
                    uint32_t w = 0u;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w |= ((uint32_t)(int)cmod((float)acc[u][q], m, rm) & 0xffu) << (8 * q);
                    pk[u] = w;
                }
            }
            if (mode < 2) {
                uint32_t out[kSlots];
#pragma unroll
                for (int u = 0; u < kSlots; ++u) out[u] = 0u;
#pragma unroll 1
                for (int ent = 0; ent < 4; ++ent) {
                    asm volatile("" ::: "memory");  // keep the constant reads inside the loop
                    float r[kSlots];
#pragma unroll
                    for (int u = 0; u < kSlots; ++u) r[u] = unpack(pk[u], ent);
                    if (g > 0) {
                        // RnsDrop (Algorithm 1): slot 15 - j is the smallest
                        // modulus left; the outer loops run with uniform
                        // indices, the slot loops unrolled
#pragma unroll 1
                        for (int qs = kSlots - 1; qs > keep; --qs) {
                            const float S = r[qs];
#pragma unroll
                            for (int p = 0; p < kSlots - 1; ++p)
                                if (p < qs) r[p] = cmod((r[p] - S) * T->inv[qs][p], T->mod[p], T->rmod[p]);
                        }
                        // MrcDigits (Algorithm 4) on slots 0 .. keep, in a copy
                        float d[kSlots];
#pragma unroll
                        for (int u = 0; u < kSlots; ++u) d[u] = r[u];
#pragma unroll 1
                        for (int i = 0; i < keep; ++i) {
                            const float di = d[i];
#pragma unroll
                            for (int j = 1; j < kSlots; ++j)
                                if (j > i && j <= keep) d[j] = cmod((d[j] - di) * T->inv[i][j], T->mod[j], T->rmod[j]);
                        }
                        // BaseExtend: the dropped slots from the shared digits
#pragma unroll 1
                        for (int p = keep + 1; p < kSlots; ++p) {
                            float tsum = 0.0f;
#pragma unroll
                            for (int i = 0; i < kSlots - 1; ++i)
                                if (i <= keep) tsum = fmaf(d[i], T->omega[i][p], tsum);
                            r[p] = cmod(tsum, T->mod[p], T->rmod[p]);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < kSlots; ++u)
                        out[u] = (out[u] >> 8) | (((uint32_t)(int)r[u] & 0xffu) << 24);
                }
                // next layout: fibre (t + 16 a), index 4 kq .. 4 kq + 3
#pragma unroll
                for (int u = 0; u < kSlots; ++u)
                    if (u >= first) *(uint32_t*)(dst + u * kPlane + (t + 16 * a) * kChainN + 4 * kq) = out[u];
            } else {
                // ReconstructFP64 (Algorithm 5): entries (a1, a2, a3) =
                // (4 kq + ent, t, a); sigma = alpha Gamma
                const double alpha = ldexp(P.Qd, -e);
#pragma unroll 1
                for (int ent = 0; ent < 4; ++ent) {
                    asm volatile("" ::: "memory");
                    float d[kSlots];
#pragma unroll
                    for (int u = 0; u < kSlots; ++u) d[u] = unpack(pk[u], ent);
#pragma unroll 1
                    for (int i = 0; i < kSlots - 1; ++i) {
                        const float di = d[i];
#pragma unroll
                        for (int j = 1; j < kSlots; ++j)
                            if (j > i) d[j] = cmod((d[j] - di) * T->inv[i][j], T->mod[j], T->rmod[j]);
                    }
                    double V = (double)d[kSlots - 1];
#pragma unroll
                    for (int j = kSlots - 2; j >= 0; --j) V = fma((double)T->mod[j], V, (double)d[j]);
                    const int a1 = 4 * kq + ent, a2 = t, a3 = a;
                    if (a1 < n && a2 < n && a3 < n) {
                        const double sigma = ldexp(alpha, -(T->fexp[0][a1] + T->fexp[1][a2] + T->fexp[2][a3]));
                        Y[a1 + (int64_t)n * (a2 + (int64_t)n * a3)] = sigma * V;
                    }
                }
            }
        }
        __syncthreads();
        const int8_t* nsrc = dst;
        dst = (int8_t*)src;
        src = nsrc;
    }
}

}  // namespace

hipError_t launch_chain(const ChainParams& P, hipStream_t st) {
    if (P.n < 1 || P.n > kChainN || P.s < kMinS || P.s > kChainMaxS || P.batch < 1 || P.batch > INT32_MAX)
        return hipErrorInvalidValue;
    if (P.g[2] != 0 || P.g[0] < 0 || P.g[1] < 0 || P.g[0] >= P.s || P.g[1] >= P.s) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chain_kernel, dim3((unsigned)P.batch), dim3(512), 0, st, P);
    return hipGetLastError();
}

}  // namespace oz2
