// oz2_chain.hip -- persistent Ozaki scheme II for chained tensor mode
// products (OzII-RescaleBE): Y = X x1 A1 x2 A2 x3 A3 x1 A4 ... (depth d <= 8,
// operator i along direction i mod 3) for a batch of n x n x n tensors,
// every step of the chain in one kernel.
//
// "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products":
//  - Sec. 5.2 and Algorithm 7: the tensor is encoded once with one exponent,
//    multiplied mode after mode on its residue planes, rescaled by g_i
//    moduli (Algorithm 1, Eq. 15) and base-extended (Algorithm 4, Eq. 26;
//    here in the CRT form where the plan allows it, with the same residues)
//    after each non-final mode, and reconstructed once; the pending row
//    scales of a direction are folded into the next operator on it on the
//    host, before encoding;
//  - Algorithm 5: Encode (rounding to nearest, ties to even), ToRns and
//    ReconstructFP64 (centred mixed-radix digits, FP64 Horner, scaling by
//    alpha * Gamma, Eq. 28);
//  - Sec. 2.3 Eq. (11): centred residues, [v]_m in [-floor(m/2), ceil(m/2) - 1].
//
// Design (CDNA4): one block of 8 wavefronts per tensor.  The tensor's residue
// planes (up to 16 moduli x 16^3 bytes) stay in LDS for the whole chain, so
// HBM sees each input entry read once and each output entry written once.
// A mode is done in place in one 64 KB buffer: every wavefront first reduces
// and packs its products into registers, then a barrier, then the rescaled
// planes overwrite the old ones; at about 78 KB of LDS a block, two tensors
// share a compute unit (4 wavefronts per SIMD).  A mode product is, per
// modulus, Y^T = R^T Abar^T on v_mfma_i32_16x16x32_i8: the 256 rows of R^T
// (the fibres along the contracted index) form 16 tiles of 16 rows, two per
// wavefront; k = 16 fills half of the MFMA's 32.  Each lane then holds four
// output entries of one fibre position for every modulus, and runs the
// modular reduction, the scheduled drops and the base extension on them in
// registers.  The output is stored so that the next mode's contraction
// index is the contiguous one: the four entries of a lane are four
// consecutive bytes of the next layout (one 32-bit LDS write per modulus).
// Each product thus rotates the layout by one direction, which is what a
// chain visiting the directions in turn needs; the final store undoes the
// rotation.  The operators' residues cycle through three LDS slots.
//
// The per-entry residue arithmetic (drops, mixed-radix digits, base
// extension, Horner) is shared with the HBM-resident kernels for larger
// tensors (oz2_chain_device.h).
#include "oz2_chain_device.h"
#include "oz2_device.h"

namespace oz2 {
namespace {

using namespace chain;

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kPlane = kChainN * kChainN * kChainN;  // 4096 entries per residue plane

// residue products of one 16-fibre tile for every slot, reduced modulo the
// slot's modulus and packed: pk[u] holds the four entries of this lane
__device__ __forceinline__ void tile_products(const int8_t* buf, const int8_t (*opm)[kChainN * kChainN],
                                              const ChainTables* T, int t, int a, int kq,
                                              uint32_t (&pk)[kSlots]) {
#pragma unroll
    for (int u0 = 0; u0 < kSlots; u0 += 4) {
        v4i acc[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // lanes with kq >= 2 hold k >= 16: zero operands (the loads stay
            // in bounds and unconditional); unused slots have zero operators
            const int u = u0 + v;
            const long a8 = *(const long*)(buf + u * kPlane + (16 * t + a) * kChainN + 8 * (kq & 1));
            const long b8 = *(const long*)(&opm[u][a * kChainN + 8 * (kq & 1)]);
            // C = 128: the accumulators come out offset by 128
            acc[v] = __builtin_amdgcn_mfma_i32_16x16x32_i8(kq < 2 ? a8 : 0l, kq < 2 ? b8 : 0l, v4i{128, 128, 128, 128},
                                                           0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int a4[4] = {acc[v][0], acc[v][1], acc[v][2], acc[v][3]};
            pk[u0 + v] = pack_products(a4, T, u0 + v);
        }
    }
}

// unpack the four entries of every slot of one tile and rescale them: the g
// drops at once with the product's drop table D, then the base extension
// (CRT: in the CRT form, on the table T->crt)
template <int G0, int G1, bool ANY, bool CRT>
__device__ __forceinline__ void rescale_tile(int mode, const int* g, const uint32_t (&pk)[kSlots],
                                             const ChainTables* T, const ChainDropTable* D, int8_t* at, int step) {
    // offset by 128; the first drop's differences remove the offset from
    // every kept slot, and without drops it is subtracted here
    float r[4][kSlots];
    unpack_tile(pk, r);
    if (G0 < 0 && g[mode] == 0) {
#pragma unroll
        for (int u = 0; u < kSlots; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) r[q][u] -= 128.0f;
    }
    // unused leading slots (modulus 1) hold zeros after every step; they are
    // stored like the others, and their zero operators make them inert
    const auto put = [&](int u, float r0, float r1, float r2, float r3) {
        store4<ANY>(at + u * kPlane, step, r0, r1, r2, r3);
    };
    if (G0 >= 0 && G0 == G1)
        drop_extend<G0, CRT>(0, r, T, D, &T->crt, put);
    else if (G0 >= 0 && mode == 0)
        drop_extend<G0, CRT>(0, r, T, D, &T->crt, put);
    else if (G0 >= 0)
        drop_extend<G1, CRT>(0, r, T, D, &T->crt, put);
    else if (g[mode] > 0)
        drop_extend<-1, CRT>(g[mode], r, T, D, &T->crt, put);
    else
        extend_dropped<-1>(0, r, T, put);
}

// G0, G1: the drop counts after products 1 and 2 when fixed at compile time
// (G0 = G1: after every product but the last), -1 to read them from P.g;
// D: the depth when fixed at compile time with the modes 1, 2, 3 (every
// residue store contiguous), 0 to read the depth, modes and layouts from P;
// CRT: every rescaling extends in the CRT form, each product's table
// (P.crts) copied into the mixed-radix weights' place in LDS before it
template <int G0, int G1, int D, bool CRT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(4, 4)))
void chain_kernel(ChainParams P) {
    __shared__ __attribute__((aligned(16))) int8_t buf[kSlots * kPlane];
    __shared__ __attribute__((aligned(16))) int8_t ops[3][kSlots][kChainN * kChainN];  // operator i in i mod 3
    __shared__ ChainTables KT;
    __shared__ ChainDropTable KS;  // the current product's drop table; for the last, the reconstruction's
    __shared__ unsigned long long smax;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = P.n;
    const int64_t n3 = (int64_t)n * n * n;
    const int first = kSlots - P.s;  // first active slot
    const double* X = P.X + (int64_t)blockIdx.x * n3;
    double* Y = P.Y + (int64_t)blockIdx.x * n3;
    // constant tables and operator residues (slot order) staged in LDS and
    // read per use (hoisted into registers they would not fit)
    // With CRT and one drop count for every rescaling (G0 = G1), the CRT
    // table is the same for every product and takes the mixed-radix weights'
    // place here, once; otherwise each product copies its own (below).
    constexpr bool kCrtOnce = CRT && G0 >= 0 && G0 == G1;
    static_assert(sizeof(ChainTables) % 4 == 0, "words");
    constexpr int kCrtWord = (int)(offsetof(ChainTables, crt) / 4), kCrtWords = (int)(sizeof(ChainCrtTable) / 4);
    for (int x = tid; x < (int)(sizeof(ChainTables) / 4); x += 512)
        ((uint32_t*)&KT)[x] = kCrtOnce && x >= kCrtWord && x < kCrtWord + kCrtWords
                                  ? ((const uint32_t*)P.crts)[x - kCrtWord]
                                  : ((const uint32_t*)P.tab)[x];
    static_assert(sizeof(ChainDropTable) % 4 == 0, "words");
    for (int x = tid; x < (int)(sizeof(ChainDropTable) / 4); x += 512)
        ((uint32_t*)&KS)[x] = ((const uint32_t*)P.split)[x];
    const ChainTables* T = &KT;
    // operator i's residues (slot order) into LDS buffer i mod 3: 512 words of 8 bytes
    auto stage_ops = [&](int i) {
        static_assert(kSlots * kChainN * kChainN / 8 == 512, "one word per thread");
        const int u = tid >> 5, w = tid & 31;
        long v = 0;
        if (u >= first) v = *(const long*)(P.ops + ((i * kSlots + (u - first)) * kChainN * kChainN) + 8 * w);
        *(long*)(&ops[i % 3][u][8 * w]) = v;
    };
    const int d = D > 0 ? D : P.d;
    const int m0 = D > 0 ? 0 : P.m0;
    for (int i = 0; i < 3 && i < d; ++i) stage_ops(i);
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
    // xbar = rint(2^e x) (|xbar| <= 2^b) as exact byte limbs; its centred
    // residues: the low byte for m = 256, the GEMM path's byte-limb identity
    // (two v_dot4_u32_u8, an FP32 floor, a byte insert) for the odd moduli
    dev::Limbs<false> L[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) L[j] = dev::make_limbs<false>(x[j], e, false);
#pragma unroll 1
    for (int u = first; u < kSlots; ++u) {
        uint32_t w[2];
        if (u == first) {
            w[0] = dev::low_byte_word<false>(L);
            w[1] = dev::low_byte_word<false>(L + 4);
        } else {
            const int q = u - first;
            const ChainEncodeConsts& E = P.enc;
            w[0] = dev::residue_word<false>(L, E.K128[q], E.c4[q], E.mod[q], E.frcp[q], E.foffb[q]);
            w[1] = dev::residue_word<false>(L + 4, E.K128[q], E.c4[q], E.mod[q], E.frcp[q], E.foffb[q]);
        }
        if (D > 0 || m0 == 0) {
            *(uint2*)(buf + u * kPlane + idx0) = make_uint2(w[0], w[1]);
        } else {
            // first product along direction m0 + 1: position 0 holds k_m0
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kk[3] = {k1_0 + j, k2, k3};
                buf[u * kPlane + kk[m0] + 16 * kk[(m0 + 1) % 3] + 256 * kk[(m0 + 2) % 3]] =
                    (int8_t)(w[j >> 2] >> (8 * (j & 3)));
            }
        }
    }
    __syncthreads();

    // --------------------------------- every product but the last, in place
    const int a = lane & 15;   // MFMA row of A / column of B and of the output
    const int kq = lane >> 4;  // k group of the operands (0, 1 hold k < 16), output row group
#pragma unroll 1
    for (int mode = 0; mode + 1 < d; ++mode) {
        asm volatile("" ::: "memory");  // keep the table reads inside the loop
        if (CRT && !kCrtOnce) {
            // this product's CRT table: read only after the barrier below,
            // written after the previous product's last read of it (the
            // barrier that closed that product)
            static_assert(kCrtWords <= 512, "one word per thread");
            if (tid < kCrtWords) ((uint32_t*)&KT.crt)[tid] = ((const uint32_t*)(P.crts + mode))[tid];
        }
        if (tid < (int)(sizeof(ChainDropTable) / 4)) ((uint32_t*)&KS)[tid] = ((const uint32_t*)(P.drops + mode))[tid];
        uint32_t pk0[kSlots], pk1[kSlots];
        tile_products(buf, ops[mode % 3], T, wave, a, kq, pk0);
        tile_products(buf, ops[mode % 3], T, wave + 8, a, kq, pk1);
        __syncthreads();  // every plane read before any is overwritten
        // the lane's entries e = 4 kq + q, fibre t, output a, stored as
        // (e, t, a): kind 0, entries contiguous; (t, e, a): kind 1, or
        // (a, e, t): kind 2, entries 16 bytes apart -- position 0 is the
        // next product's direction
        const int kind = D > 0 ? 0 : P.kind[mode];
        const int step = kind == 0 ? 0 : 16;
        auto at = [&](int t) -> int8_t* {
            return buf + (kind == 0 ? (t + 16 * a) * kChainN + 4 * kq
                                    : kind == 1 ? t + 64 * kq + 256 * a : a + 64 * kq + 256 * t);
        };
        rescale_tile<G0, G1, D == 0, CRT>(mode, P.g, pk0, T, &KS, at(wave), step);
        asm volatile("" ::: "memory");  // one tile at a time
        rescale_tile<G0, G1, D == 0, CRT>(mode, P.g, pk1, T, &KS, at(wave + 8), step);
        asm volatile("" ::: "memory");
        // operator mode + 3 into the buffer this product read (before the
        // barrier above); it is next read three products later
        if (mode + 3 < d) stage_ops(mode + 3);
        __syncthreads();
    }
    if (d >= 2) {
        // the two-block reconstruction's weights back in place of the last
        // rescaling's drop table (read after the barrier closing that product)
        if (tid < (int)(sizeof(ChainDropTable) / 4)) ((uint32_t*)&KS)[tid] = ((const uint32_t*)P.split)[tid];
        __syncthreads();
    }

    // -------------------------------------- last product and ReconstructFP64
    // (Algorithm 5), sigma = alpha Gamma.  The lane's entries 4 kq + q, its
    // fibre t and its output a run along the directions P.fin (with the
    // modes 1, 2, 3 the last product leaves them in that order).
    const double alpha = ldexp(P.Qd, -e);
    const int dir0 = D > 0 ? 0 : P.fin[0], dir1 = D > 0 ? 1 : P.fin[1], dir2 = D > 0 ? 2 : P.fin[2];
    const int64_t n2 = (int64_t)n * n;
    const int64_t st0 = dir0 == 0 ? 1 : dir0 == 1 ? n : n2;
    const int64_t st1 = dir1 == 0 ? 1 : dir1 == 1 ? n : n2;
    const int64_t st2 = dir2 == 0 ? 1 : dir2 == 1 ? n : n2;
    const int* F0 = T->fexp[dir0];
    const int* F1 = T->fexp[dir1];
    const int* F2 = T->fexp[dir2];
#pragma unroll 1
    for (int tt = 0; tt < 2; ++tt) {
        asm volatile("" ::: "memory");
        const int t = wave + 8 * tt;
        uint32_t pk[kSlots];
        tile_products(buf, ops[(d - 1) % 3], T, t, a, kq, pk);
        double V[4];
        mrc_horner_split<kChainSplit>(pk, T, &KS, V);
        // the values are complete here (the compiler would otherwise sink
        // each entry's whole digit computation into its guarded store)
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(V[q]));
        if (t < n && a < n) {
            const int f12 = F1[t] + F2[a];
            double* y = Y + t * st1 + a * st2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p0 = 4 * kq + q;
                if (p0 < n) y[p0 * st0] = ldexp(alpha, -(F0[p0] + f12)) * V[q];
            }
        }
    }
}

}  // namespace

hipError_t launch_chain(const ChainParams& P, hipStream_t st) {
    if (P.n < 1 || P.n > kChainN || P.s < kMinS || P.s > kChainMaxS || P.batch < 1 || P.batch > INT32_MAX)
        return hipErrorInvalidValue;
    if (P.d < 1 || P.d > kChainMaxD || P.g[P.d - 1] != 0) return hipErrorInvalidValue;
    for (int i = 0; i + 1 < P.d; ++i)
        if (P.g[i] < 0 || P.g[i] >= P.s || P.kind[i] < 0 || P.kind[i] > 2) return hipErrorInvalidValue;
    if (P.m0 < 0 || P.m0 > 2) return hipErrorInvalidValue;
    for (int j = 0; j < 3; ++j)
        if (P.fin[j] < 0 || P.fin[j] > 2) return hipErrorInvalidValue;
    // compile-time drop counts for the usual plans of 16^3 tensors (7 after
    // every product with 16 or 14 moduli, 6 with 12, 4 with 8; 4 then 5 for
    // a depth-3 chain with 10) and a compile-time depth for one pass over the
    // three directions; any other plan takes a guarded or run-time instance
    bool same = P.d >= 2;
    for (int i = 1; i + 1 < P.d; ++i) same = same && P.g[i] == P.g[0];
    const int g0 = same ? P.g[0] : -1;
    // the CRT form where every product with drops has the plan's margin
    bool crt = P.crts != nullptr;
    for (int i = 0; i + 1 < P.d; ++i) crt = crt && (P.g[i] == 0 || P.crt[i]);
    const dim3 grid((unsigned)P.batch), block(512);
    if (P.d == 3 && P.cyclic) {
        if (g0 == 7 && crt)
            hipLaunchKernelGGL((chain_kernel<7, 7, 3, true>), grid, block, 0, st, P);
        else if (g0 == 7)
            hipLaunchKernelGGL((chain_kernel<7, 7, 3, false>), grid, block, 0, st, P);
        else if (g0 == 6 && crt)
            hipLaunchKernelGGL((chain_kernel<6, 6, 3, true>), grid, block, 0, st, P);
        else if (g0 == 6)
            hipLaunchKernelGGL((chain_kernel<6, 6, 3, false>), grid, block, 0, st, P);
        else if (g0 == 4 && crt)
            hipLaunchKernelGGL((chain_kernel<4, 4, 3, true>), grid, block, 0, st, P);
        else if (g0 == 4)
            hipLaunchKernelGGL((chain_kernel<4, 4, 3, false>), grid, block, 0, st, P);
        else if (P.g[0] == 4 && P.g[1] == 5 && crt)
            hipLaunchKernelGGL((chain_kernel<4, 5, 3, true>), grid, block, 0, st, P);
        else if (P.g[0] == 4 && P.g[1] == 5)
            hipLaunchKernelGGL((chain_kernel<4, 5, 3, false>), grid, block, 0, st, P);
        else if (crt)
            hipLaunchKernelGGL((chain_kernel<-1, -1, 3, true>), grid, block, 0, st, P);
        else
            hipLaunchKernelGGL((chain_kernel<-1, -1, 3, false>), grid, block, 0, st, P);
    } else if (g0 == 7 && crt) {
        hipLaunchKernelGGL((chain_kernel<7, 7, 0, true>), grid, block, 0, st, P);
    } else if (g0 == 7) {
        hipLaunchKernelGGL((chain_kernel<7, 7, 0, false>), grid, block, 0, st, P);
    } else if (crt) {
        hipLaunchKernelGGL((chain_kernel<-1, -1, 0, true>), grid, block, 0, st, P);
    } else {
        hipLaunchKernelGGL((chain_kernel<-1, -1, 0, false>), grid, block, 0, st, P);
    }
    return hipGetLastError();
}

}  // namespace oz2
