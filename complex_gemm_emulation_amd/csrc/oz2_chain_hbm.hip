// oz2_chain_hbm.hip -- persistent Ozaki scheme II for chained tensor mode
// products (OzII-RescaleBE) with the residue planes in HBM between the
// products, one kernel per product: tensors too large for one block's LDS
// (n > 16), and small ones (n <= 8) that the LDS kernel would pad to 16^3.
//
// "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products":
//  - Sec. 5.2 and Algorithm 7: the tensor is encoded once with one exponent,
//    multiplied mode after mode on its residue planes, rescaled by g_i moduli
//    (Algorithm 1, Eq. 15) and base-extended (Algorithm 4, Eq. 26) after each
//    non-final product, and reconstructed once;
//  - Algorithm 5: Encode (the exponent from the tensor's largest magnitude,
//    rounding to nearest, ties to even), ToRns and ReconstructFP64 (centred
//    mixed-radix digits, FP64 Horner, scaling by alpha * Gamma, Eq. 28);
//  - Sec. 2.3 Eq. (11): centred residues.
// The chain page runs its method as batched GEMMs and elementwise kernels
// over HBM-resident residues (Sec. 5.2); here each product and its
// rescaling are one kernel.
//
// Launches for a chain of depth d: a scan (the largest |x| of each tensor),
// the encode (all s residue planes of every tensor), d - 1 rescaling
// products (planes in, planes out: two buffers in turn) and the last
// product with the reconstruction (planes in, FP64 out).
//
// Plane layout: every direction is padded to np = n rounded up to 8, and a
// tensor occupies np^3 bytes of each plane, position (p0, p1, p2) at
// p0 + np p1 + np^2 p2 with p0 the direction the next product contracts.
// Fibre f = p1 + np p2 (np^2 per tensor) is then the row of np bytes at
// f np, and a product is, per modulus, Y^T = R^T Abar^T on
// v_mfma_i32_16x16x32_i8: a tile is 16 fibres (the MFMA's rows) against 16
// operator rows (the MFMA's columns), k in pairs of 32-byte chunks of which
// each lane holds 16 consecutive bytes of its row.  The operator's residues
// are stored in that fragment order (1 KiB per wavefront and pair).  For
// padded sides below 96 a wavefront walks the operator's row tiles of one
// fibre tile, reading the fibres from memory (they stay in cache between
// the few row tiles); from 96 on a block stages its fibre tile in LDS once
// and its wavefronts share it across the row tiles; at np = 8 a tile stacks
// two sets of 16 fibres against the operator's 8 rows.  Each lane then holds
// four consecutive fibres of one output row for every modulus, and reduces,
// rescales and base-extends them in registers (oz2_chain_device.h): the g
// drops at once, by the mixed-radix digits over the dropped moduli and one
// weighted sum per kept residue (drop_extend, bitwise the repeated RnsDrop),
// the base extension in the CRT form where the plan allows it (extend_crt;
// the last template argument of the product kernels), and the
// reconstruction's digits in two blocks (mrc_horner_split).  The
// output layout puts the next product's direction at p0: with the directions
// in turn that is the fibres' p1, so the lane's four entries are four
// consecutive bytes of every output plane.
//
// Padding never reaches a result: the encode writes residues of zero there,
// the operators' columns k >= n are zero (whatever a padded position holds
// is multiplied by zero), outputs of padded fibres go to padded positions,
// operator rows beyond np are not stored, and the reconstruction stores only
// positions < n.
#include "oz2_chain_device.h"
#include "oz2_device.h"

namespace oz2 {
namespace {

using namespace chain;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef long v2l __attribute__((ext_vector_type(2)));

constexpr int kScanChunk = 4096;      // entries of one tensor per scan block
constexpr int kStepBlocksMax = 2048;  // blocks of the product kernels (8 per CU), each looping over tiles
constexpr int kStagedNp = kChainStagedNp;  // padded sides from which the fibre tiles are staged in LDS
constexpr size_t kStepLdsMax = 65536; // staged fibre tiles of one block: 16 moduli x 16 rows x 256 bytes

constexpr unsigned long long kInfBits = 0x7ff0000000000000ull;

// exponent e = b - E of a tensor whose largest |x| has the bit pattern M
// (2^(E-1) <= max|x| < 2^E), 0 for an all-zero tensor
__device__ __forceinline__ int tensor_exponent(unsigned long long M, int b) {
    if (!M) return 0;
    int E = 0;
    (void)frexp(__longlong_as_double((long long)M), &E);
    return b - E;
}

// ---------------------------------------------------------------- scan
// the largest |x| bit pattern of each tensor (positive doubles order as
// their bit patterns; non-finite entries give a pattern >= kInfBits)
// (a block takes R consecutive chunks of one tensor, so that at most 256
// blocks meet at one tensor's atomic; reduced across each wavefront by
// shuffles, then across the four wavefronts in LDS, then one atomic per
// block.  An entry past the tensor's end loads the chunk's first entry
// instead, so that every load of a chunk is unconditional and in flight
// together.)
__global__ __launch_bounds__(256) void chain_scan_kernel(const double* __restrict__ X, int64_t n3, int64_t chunks,
                                                         int R, unsigned long long* smax) {
    __shared__ unsigned long long wm[4];
    const int64_t bpt = (chunks + R - 1) / R;  // blocks per tensor
    const int64_t t = blockIdx.x / bpt, c0 = (blockIdx.x % bpt) * R;
    const double* x = X + t * n3;
    unsigned long long mx = 0;
#pragma unroll 1
    for (int64_t c = c0; c < c0 + R && c < chunks; ++c) {
#pragma unroll
        for (int j = 0; j < kScanChunk / 256; ++j) {
            const int64_t i = c * kScanChunk + j * 256 + threadIdx.x;
            const unsigned long long v =
                (unsigned long long)__double_as_longlong(x[i < n3 ? i : c * kScanChunk]) & 0x7fffffffffffffffull;
            mx = v > mx ? v : mx;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long v = __shfl_xor(mx, o, 64);
        mx = v > mx ? v : mx;
    }
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long b = wm[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) b = wm[w] > b ? wm[w] : b;
        atomicMax(&smax[t], b);
    }
}

// the same for tensors of at most kScanChunk entries: one wavefront per
// tensor, reduced across the wavefront, one store (no atomics)
__global__ __launch_bounds__(256) void chain_scan_small_kernel(const double* __restrict__ X, int64_t n3,
                                                               int64_t batch, unsigned long long* smax) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= batch) return;
    const double* x = X + t * n3;
    unsigned long long mx = 0;
    for (int64_t i = lane; i < n3; i += 64) {
        const unsigned long long v = (unsigned long long)__double_as_longlong(x[i]) & 0x7fffffffffffffffull;
        mx = v > mx ? v : mx;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long v = __shfl_xor(mx, o, 64);
        mx = v > mx ? v : mx;
    }
    if (lane == 0) smax[t] = mx;
}

// -------------------------------------------------------------- encode
// four consecutive positions p0 .. p0 + 3 of one tensor per thread, every
// modulus: x (zero at padding and for a tensor with a non-finite entry,
// whose result the reconstruction sets to NaN), xbar = rint(2^e x) split into
// byte limbs exactly (|xbar| <= 2^53), and its centred residues packed into
// one 32-bit word per plane: the low byte of xbar for m = 256, and for the
// odd moduli the byte-limb identity of the GEMM path's encoder (two
// v_dot4_u32_u8 per residue, an FP32 floor, one byte insert; exact)
__global__ __launch_bounds__(256) void chain_encode_kernel(ChainHbmParams P, ChainEncodeConsts E, int64_t bpt) {
    const int n = P.n, np = P.np;
    const int64_t np3 = (int64_t)np * np * np;
    const int64_t t = blockIdx.x / bpt;
    const int64_t i4 = ((blockIdx.x % bpt) * 256 + threadIdx.x) * 4;
    if (i4 >= np3) return;
    const int p0 = (int)(i4 % np);
    const int64_t rest = i4 / np;
    const int p1 = (int)(rest % np), p2 = (int)(rest / np);
    const unsigned long long M = P.smax[t];
    const bool finite = M < kInfBits;
    const int e = finite ? tensor_exponent(M, P.b) : 0;
    const int d0 = P.m0, d1 = (P.m0 + 1) % 3, d2 = (P.m0 + 2) % 3;
    const int64_t nn = (int64_t)n * n;
    const int64_t sd0 = d0 == 0 ? 1 : d0 == 1 ? n : nn;
    const int64_t sd1 = d1 == 0 ? 1 : d1 == 1 ? n : nn;
    const int64_t sd2 = d2 == 0 ? 1 : d2 == 1 ? n : nn;
    const double* x = P.X + t * n * nn + p1 * sd1 + p2 * sd2;
    dev::Limbs<false> L[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool in = finite && p0 + q < n && p1 < n && p2 < n;
        L[q] = dev::make_limbs<false>(in ? x[(p0 + q) * sd0] : 0.0, e, !in);
    }
    int8_t* out = P.out + t * np3 + i4;
    *(uint32_t*)out = dev::low_byte_word<false>(L);  // modulus 256 (index 0)
#pragma unroll 1
    for (int qm = 1; qm < P.s; ++qm)
        *(uint32_t*)(out + qm * P.pstride) =
            dev::residue_word<false>(L, E.K128[qm], E.c4[qm], E.mod[qm], E.frcp[qm], E.foffb[qm]);
}

// ------------------------------------------------------ product kernels
// Per-launch constants of the product kernels.
struct StepConsts {
    int n, np, first, ap;
    int64_t np2, np3, n3, opq;
    const int *F0, *F1, *F2;
    int64_t st0, st1, st2;
    __device__ explicit StepConsts(const ChainHbmParams& P) {
        n = P.n;
        np = P.np;
        first = kSlots - P.s;  // first active slot; slot u holds modulus index u - first
        ap = (np + 15) & ~15;
        np2 = (int64_t)np * np;
        np3 = np2 * np;
        n3 = (int64_t)n * n * n;
        opq = (int64_t)ap * ((np + 63) / 64) * 64;  // operator bytes per modulus
        F0 = P.fexp + P.fin[0] * np;
        F1 = P.fexp + P.fin[1] * np;
        F2 = P.fexp + P.fin[2] * np;
        st0 = P.fin[0] == 0 ? 1 : P.fin[0] == 1 ? n : (int64_t)n * n;
        st1 = P.fin[1] == 0 ? 1 : P.fin[1] == 1 ? n : (int64_t)n * n;
        st2 = P.fin[2] == 0 ? 1 : P.fin[2] == 1 ? n : (int64_t)n * n;
    }
};

// One tile: 16 fibres f0 .. f0 + 15 of tensor t against operator rows
// a0 .. a0 + 15.  The residue products of every modulus (offset by the
// MFMA's accumulator input 128, reduced and packed), then either (LAST) the
// reconstruction of the four entries of each lane, or the rescaling with
// P.g drops and the stores into the next layout (CONTIG: P.kind == 0, four
// consecutive bytes per plane).
// The contraction runs over NCP pairs of 32-byte k chunks: lane r + 16 j
// holds bytes 64 cp + 16 j .. 64 cp + 16 j + 15 of its row (fibre r of the
// tile, operator row a0 + r) for pair cp, the first 8 for one MFMA and the
// last 8 for the other.  Both operands take the same k for the same lane
// and half, so the two MFMAs of every pair sum the same products as two
// chunks of 32 consecutive k would.  xload(qm, cp) gives the fibres' 16
// bytes (zero at k >= np); the operator's come in fragment order (zero
// padded), 1 KiB per wavefront per pair, all four moduli of a slot group
// loaded before its MFMAs.
// fa = f0 + 4 kq is the lane's first fibre within the tensor (< np^2 <=
// 2^16), at positions p1 = fa mod np, p2 = fa / np (the caller's, once per
// fibre tile).
// HALF (np = 8, one pair): the operator has 8 rows, so a tile is 32 fibres
// against them: MFMA column c takes operator row c mod 8 in k group c / 8
// (the operator's fragments hold each row twice, zero elsewhere) and row i
// of the fibres' operand holds fibre f0 + i in k group 0 and fibre
// f0 + 16 + i in k group 1, so column c of the output is fibre set c / 8
// against operator row c mod 8, and every lane's entries are used: the lane
// of column c holds fibres f0 + 16 (c / 8) + 4 kq + q (the caller's fa).
// Only the pair's first MFMA carries data.
template <bool CONTIG, bool LAST, int NCP, bool HALF, bool CRT, int SPLIT, class XLoad>
__device__ __forceinline__ void step_tile(const ChainHbmParams& P, const StepConsts& K, const ChainTables* T,
                                          const ChainDropTable* DT, const ChainCrtTable* CT, int64_t t, int fa,
                                          int p1, int p2, int a0, int lane, const XLoad& xload,
                                          unsigned long long M, double alpha) {
    static_assert(!HALF || NCP == 1, "one pair of k chunks at np = 8");
    const int a = HALF ? (lane & 7) : a0 + (lane & 15);  // column of the output (operator row)
    const int8_t* opf = P.ops + ((int64_t)(a0 >> 4) * NCP * 64 + lane) * 16;
    uint32_t pk[kSlots];
#pragma unroll
    for (int u0 = 0; u0 < kSlots; u0 += 4) {
        // one slot group's operands in registers at a time: without the
        // barrier the scheduler hoists every group's loads and spills
        __builtin_amdgcn_sched_barrier(0);
        if (u0 + 3 < K.first) {  // no modulus in the group: residues of zero
#pragma unroll
            for (int v = 0; v < 4; ++v) pk[u0 + v] = 0x80808080u;
            continue;
        }
        // A slot below K.first (modulus 1) takes modulus index 0's operands:
        // its reduction modulo 1 gives the byte of a zero residue whatever
        // the products, so the group needs no branch.
        int qm[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) qm[v] = u0 + v >= K.first ? u0 + v - K.first : 0;
        v2l ob[4][NCP];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int cp = 0; cp < NCP; ++cp) ob[v][cp] = *(const v2l*)(opf + (int64_t)qm[v] * K.opq + cp * 1024);
        v4i acc[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            acc[v] = v4i{128, 128, 128, 128};
#pragma unroll
            for (int cp = 0; cp < NCP; ++cp) {
                const v2l x = xload(qm[v], cp);
                acc[v] = __builtin_amdgcn_mfma_i32_16x16x32_i8(x[0], ob[v][cp][0], acc[v], 0, 0, 0);
                if (!HALF) acc[v] = __builtin_amdgcn_mfma_i32_16x16x32_i8(x[1], ob[v][cp][1], acc[v], 0, 0, 0);
            }
        }
        // each word is pinned here, or the reductions sink below the later
        // groups and their accumulators spill
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int a4[4] = {acc[v][0], acc[v][1], acc[v][2], acc[v][3]};
            pk[u0 + v] = pack_products(a4, T, u0 + v);
            asm volatile("" : "+v"(pk[u0 + v]));
        }
    }
    if (LAST) {
        double V[4];
        mrc_horner_split<SPLIT>(pk, T, DT, V);
        if (p2 < K.n && a < K.n) {
            const int f12 = K.F1[p2] + K.F2[a];
            double* y = P.Y + t * K.n3 + p2 * K.st1 + a * K.st2;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (p1 + q < K.n)
                    y[(p1 + q) * K.st0] = M < kInfBits ? ldexp(alpha, -(K.F0[p1 + q] + f12)) * V[q] : __builtin_nan("");
        }
    } else {
        float r[4][kSlots];
        unpack_tile(pk, r);
        // the next layout: (p1, p2, a) with the four entries contiguous,
        // (p2, p1, a) or (a, p1, p2) with them np apart.  The lane's column
        // is made opaque here so that the 16 x 4 store addresses are formed
        // after the products, not hoisted above them into spilled registers.
        int ao = a;
        asm volatile("" : "+v"(ao));
        int8_t* base = P.out + t * K.np3;
        int64_t step = 0;
        if (CONTIG) {
            base += fa + K.np2 * ao;
        } else if (P.kind == 1) {
            base += p2 + (int64_t)K.np * p1 + K.np2 * ao;
            step = K.np;
        } else {
            base += ao + (int64_t)K.np * fa;
            step = K.np;
        }
        const bool ok = a < K.np;
        const int first = K.first;
        const int64_t pstride = P.pstride;
        const auto put = [=](int u, float r0, float r1, float r2, float r3) {
            if (u >= first && ok) store4<!CONTIG>(base + (int64_t)(u - first) * pstride, step, r0, r1, r2, r3);
        };
        if (P.g == 0) {
            // no drop: the residues lose their offset here and are stored
#pragma unroll
            for (int u = 0; u < kSlots; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) r[q][u] -= 128.0f;
            extend_dropped<-1>(0, r, T, put);
        } else {
            drop_extend<-1, CRT>(P.g, r, T, DT, CT, put);
        }
    }
}

// the constant tables into LDS (read per use; hoisted into registers they
// would not fit), with this product's drop weights (the last product's:
// those of the two-block reconstruction) and its CRT table if it has one
template <bool CRT>
__device__ __forceinline__ void stage_tables(const ChainHbmParams& P, ChainTables& KT, ChainDropTable& KD,
                                             ChainCrtTable& KC) {
    static_assert(sizeof(ChainTables) % 4 == 0 && sizeof(ChainDropTable) % 4 == 0 &&
                  sizeof(ChainCrtTable) % 4 == 0, "words");
    // the words of the two or three tables in one sequence, a thread's loads
    // all in flight before its stores (blocks have 256 or 512 threads); a word
    // past the end loads word 0 instead and stores nothing
    constexpr int nT = (int)(sizeof(ChainTables) / 4), nD = (int)(sizeof(ChainDropTable) / 4);
    constexpr int nW = nT + nD + (CRT ? (int)(sizeof(ChainCrtTable) / 4) : 0);
    constexpr int kPer = (nW + 255) / 256;
    uint32_t v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int x = threadIdx.x + i * blockDim.x < nW ? threadIdx.x + i * blockDim.x : 0;
        v[i] = x < nT ? ((const uint32_t*)P.tab)[x]
                      : x < nT + nD ? ((const uint32_t*)P.drop)[x - nT] : ((const uint32_t*)P.crt)[x - nT - nD];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int x = threadIdx.x + i * blockDim.x;
        if (x < nT)
            ((uint32_t*)&KT)[x] = v[i];
        else if (x < nT + nD)
            ((uint32_t*)&KD)[x - nT] = v[i];
        else if (x < nW)
            ((uint32_t*)&KC)[x - nT - nD] = v[i];
    }
    __syncthreads();
}

// Occupancy of both forms: the drop count is a run-time value (with it
// fixed at compile time the unrolled slot loops keep more table values live,
// about 200 registers, and spill hundreds of bytes at 128; the run-time form
// spills about 40) at 4 wavefronts per SIMD; the reconstruction needs about
// 250 registers and runs at 2.  NCP (pairs of k chunks, np / 64 rounded up)
// is a compile-time constant so that every operator fragment of a slot group
// is loaded before its first MFMA.
//
// Direct form (np < 96): one wavefront per tile of 16 fibres, in a
// grid-stride loop, walking the operator's rows in tiles of 16 and reading
// the fibres' operand from memory (the tile stays in cache between row
// tiles when there are few of them).
template <bool CONTIG, bool LAST, int NCP, bool HALF, bool CRT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LAST ? 2 : 4, LAST ? 2 : 4)))
void chain_step_kernel(ChainHbmParams P) {
    static_assert(!(LAST && CRT), "the last product has no base extension");
    __shared__ ChainTables KT;
    __shared__ ChainDropTable KD;
    __shared__ ChainCrtTable KC;
    stage_tables<CRT>(P, KT, KD, KC);
    const StepConsts K(P);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, kq = lane >> 4;
    constexpr int TF = HALF ? 32 : 16;  // fibres per tile
    const int64_t nft = K.np2 / TF;     // fibre tiles per tensor (np^2 is a multiple of 64)
    const int64_t tiles = P.batch * nft;
#pragma unroll 1
    for (int64_t w = (int64_t)blockIdx.x * 4 + wave; w < tiles; w += (int64_t)gridDim.x * 4) {
        const int64_t t = w / nft;
        const int f0 = (int)(w % nft) * TF;
        const int8_t* xt = P.in + t * K.np3;  // the tensor in plane 0
        // captured by value: a reference into the kernel's parameters keeps
        // them in memory and costs about 100 bytes of spills per lane
        const int64_t pstride = P.pstride;
        const int np = K.np, k0 = 16 * kq;
        const int fa = f0 + (HALF ? 16 * (r16 >> 3) : 0) + 4 * kq;
        const int p1 = fa % K.np, p2 = fa / K.np;
        const unsigned long long M = LAST ? P.smax[t] : 0ull;
        const double alpha = LAST ? ldexp(P.Qd, -tensor_exponent(M < kInfBits ? M : 0ull, P.b)) : 0.0;
#pragma unroll 1
        for (int a0 = 0; a0 < K.np; a0 += 16) {
            asm volatile("" ::: "memory");
            // the lane's fibre row (< np^3 <= 2^24), opaque in each row tile:
            // hoisted out of this loop, the 16 NCP fibre addresses would hold
            // registers across the rescaling and spill
            int xrow = (f0 + r16 + (HALF ? 16 * (kq & 1) : 0)) * np;
            asm volatile("" : "+v"(xrow));
            // bytes at k >= np (the row ends at np, a multiple of 8) are zero;
            // their loads read the row's first bytes instead, so that no load
            // is conditional.  HALF: k groups 0 and 1 hold bytes 0 .. 7 of
            // fibres f0 + r16 and f0 + 16 + r16.
            const auto xload = [=](int qm, int cp) {
                const int8_t* x = xt + (int64_t)qm * pstride + xrow;
                if (HALF) return v2l{kq < 2 ? *(const long*)x : 0l, 0l};
                const int k = k0 + 64 * cp;
                const long lo = *(const long*)(x + (k < np ? k : 0));
                const long hi = *(const long*)(x + (k + 8 < np ? k + 8 : 0));
                return v2l{k < np ? lo : 0l, k + 8 < np ? hi : 0l};
            };
            step_tile<CONTIG, LAST, NCP, HALF, CRT, kChainSplitWide>(P, K, &KT, &KD, &KC, t, fa, p1, p2, a0, lane,
                                                                     xload, M, alpha);
        }
    }
}

// Staged form (np >= 96): a block takes F fibre tiles of one tensor at a
// time (F = 1 there) and stages their rows of every plane in LDS in the
// operand order of the MFMAs, [q][F][NCP][64 lanes][16 bytes] (lane r + 16 j
// of pair cp: bytes 64 cp + 16 j .. + 15 of fibre row r, zero at k >= np),
// so that both the staging copy and every operand read are contiguous; its
// NW wavefronts take the (fibre tile, operator-row tile) pairs in turn.  The
// fibres are read from HBM once; in the direct form a fibre tile's row
// tiles re-fetch it once the tiles in flight on an XCD (about 4 MB at
// n = 256) have evicted it from L2, 36 times the planes per launch at
// n = 256, and from 96 on the staged form is faster.  NW is 8 when a block stages more than 32 KiB and the row tiles
// divide evenly (then LDS admits only two blocks per compute unit, and 4
// wavefronts each would leave 2 per SIMD to interleave the dependent
// modular steps), else 4.
template <bool CONTIG, bool LAST, int NCP, int NW, bool CRT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(LAST ? 2 : 4, LAST ? 2 : 4)))
void chain_step_staged_kernel(ChainHbmParams P, int F) {
    static_assert(!(LAST && CRT), "the last product has no base extension");
    __shared__ ChainTables KT;
    __shared__ ChainDropTable KD;
    __shared__ ChainCrtTable KC;
    extern __shared__ __attribute__((aligned(16))) int8_t xs[];  // [s][F][NCP][64 lanes][16 bytes]
    stage_tables<CRT>(P, KT, KD, KC);
    const StepConsts K(P);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int na = K.ap / 16;                // operator-row tiles
    const int64_t nft = K.np2 / 16;
    const int items = P.s * F * NCP * 64;    // 16-byte items staged per block tile
    const int64_t btiles = P.batch * (nft / F);
#pragma unroll 1
    for (int64_t bt = blockIdx.x; bt < btiles; bt += gridDim.x) {
        const int64_t t = bt / (nft / F);
        const int fb0 = (int)(bt % (nft / F)) * F * 16;  // first fibre of the block tile
        __syncthreads();  // the previous tile's operands are read
        // kStage items per thread at a time, their loads all in flight before
        // the first store (one at a time, each store waited for its loads: a
        // memory round trip per item).  An item past the end loads item x0
        // instead (in bounds, unconditional) and stores nothing.  Measured:
        // 4 at 4 wavefronts; at 8 (n > 240), 2 was faster than 4 or 8.
        constexpr int kStage = NW == 8 ? 2 : 4;
#pragma unroll 1
        for (int x0 = tid; x0 < items; x0 += kStage * 64 * NW) {
            v2l v[kStage];
#pragma unroll
            for (int i = 0; i < kStage; ++i) {
                const int x = x0 + i * 64 * NW < items ? x0 + i * 64 * NW : x0;
                const int L = x & 63, rest = x >> 6;
                const int cp = rest % NCP, rest2 = rest / NCP;
                const int f = rest2 % F, q = rest2 / F;
                const int k = 64 * cp + 16 * (L >> 4);
                const int8_t* row = P.in + q * P.pstride + t * K.np3 + (int64_t)(fb0 + 16 * f + (L & 15)) * K.np;
                // zero at k >= np; those loads read the row's first bytes
                const long lo = *(const long*)(row + (k < K.np ? k : 0));
                const long hi = *(const long*)(row + (k + 8 < K.np ? k + 8 : 0));
                v[i] = v2l{k < K.np ? lo : 0l, k + 8 < K.np ? hi : 0l};
            }
            __builtin_amdgcn_sched_barrier(0);  // every load issued before the stores
#pragma unroll
            for (int i = 0; i < kStage; ++i)
                if (x0 + i * 64 * NW < items) *(v2l*)(xs + (int64_t)(x0 + i * 64 * NW) * 16) = v[i];
        }
        __syncthreads();
#pragma unroll 1
        for (int pr = wave; pr < F * na; pr += NW) {
            asm volatile("" ::: "memory");
            const int f = pr / na;
            const int8_t* xl = xs + ((int64_t)f * NCP * 64 + lane) * 16;
            const int64_t qstride = (int64_t)F * NCP * 1024;
            const auto xload = [=](int qm, int cp) { return *(const v2l*)(xl + qm * qstride + cp * 1024); };
            const int fa = fb0 + 16 * f + 4 * (lane >> 4);
            const unsigned long long M = LAST ? P.smax[t] : 0ull;
            const double alpha = LAST ? ldexp(P.Qd, -tensor_exponent(M < kInfBits ? M : 0ull, P.b)) : 0.0;
            step_tile<CONTIG, LAST, NCP, false, CRT, kChainSplit>(P, K, &KT, &KD, &KC, t, fa, fa % K.np, fa / K.np,
                                                                  (pr % na) * 16, lane, xload, M, alpha);
        }
    }
}

template <int NCP, bool HALF>
void launch_direct(const ChainHbmParams& P, bool last, dim3 grid, hipStream_t st) {
    const bool crt = P.crt != nullptr;
    if (last)
        hipLaunchKernelGGL((chain_step_kernel<true, true, NCP, HALF, false>), grid, dim3(256), 0, st, P);
    else if (P.kind == 0 && crt)
        hipLaunchKernelGGL((chain_step_kernel<true, false, NCP, HALF, true>), grid, dim3(256), 0, st, P);
    else if (P.kind == 0)
        hipLaunchKernelGGL((chain_step_kernel<true, false, NCP, HALF, false>), grid, dim3(256), 0, st, P);
    else if (crt)
        hipLaunchKernelGGL((chain_step_kernel<false, false, NCP, HALF, true>), grid, dim3(256), 0, st, P);
    else
        hipLaunchKernelGGL((chain_step_kernel<false, false, NCP, HALF, false>), grid, dim3(256), 0, st, P);
}

template <int NCP, int NW>
void launch_staged(const ChainHbmParams& P, bool last, dim3 grid, size_t lds, int F, hipStream_t st) {
    const dim3 block(64 * NW);
    const bool crt = P.crt != nullptr;
    if (last)
        hipLaunchKernelGGL((chain_step_staged_kernel<true, true, NCP, NW, false>), grid, block, lds, st, P, F);
    else if (P.kind == 0 && crt)
        hipLaunchKernelGGL((chain_step_staged_kernel<true, false, NCP, NW, true>), grid, block, lds, st, P, F);
    else if (P.kind == 0)
        hipLaunchKernelGGL((chain_step_staged_kernel<true, false, NCP, NW, false>), grid, block, lds, st, P, F);
    else if (crt)
        hipLaunchKernelGGL((chain_step_staged_kernel<false, false, NCP, NW, true>), grid, block, lds, st, P, F);
    else
        hipLaunchKernelGGL((chain_step_staged_kernel<false, false, NCP, NW, false>), grid, block, lds, st, P, F);
}

}  // namespace

hipError_t launch_chain_scan(const ChainHbmParams& P, hipStream_t st) {
    if (P.n < 1 || P.n > kChainMaxN || P.batch < 1) return hipErrorInvalidValue;
    const int64_t n3 = (int64_t)P.n * P.n * P.n;
    const int64_t chunks = (n3 + kScanChunk - 1) / kScanChunk;
    if (P.batch * chunks > INT32_MAX) return hipErrorInvalidValue;
    if (chunks == 1) {
        hipLaunchKernelGGL(chain_scan_small_kernel, dim3((unsigned)((P.batch + 3) / 4)), dim3(256), 0, st, P.X, n3,
                           P.batch, P.smax);
    } else {
        const int R = (int)((chunks + 255) / 256);
        const int64_t bpt = (chunks + R - 1) / R;
        hipLaunchKernelGGL(chain_scan_kernel, dim3((unsigned)(P.batch * bpt)), dim3(256), 0, st, P.X, n3, chunks, R,
                           P.smax);
    }
    return hipGetLastError();
}

hipError_t launch_chain_encode(const ChainHbmParams& P, const ChainEncodeConsts& E, hipStream_t st) {
    if (P.n < 1 || P.n > kChainMaxN || P.np != ((P.n + 7) & ~7) || P.batch < 1 || P.s < kMinS || P.s > kChainMaxS ||
        P.m0 < 0 || P.m0 > 2)
        return hipErrorInvalidValue;
    const int64_t np3 = (int64_t)P.np * P.np * P.np;
    const int64_t bpt = (np3 / 4 + 255) / 256;
    if (P.batch * bpt > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chain_encode_kernel, dim3((unsigned)(P.batch * bpt)), dim3(256), 0, st, P, E, bpt);
    return hipGetLastError();
}

hipError_t launch_chain_step(const ChainHbmParams& P, bool last, hipStream_t st) {
    if (P.n < 1 || P.n > kChainMaxN || P.np != ((P.n + 7) & ~7) || P.batch < 1 || P.s < kMinS || P.s > kChainMaxS)
        return hipErrorInvalidValue;
    if (!last && (P.g < 0 || P.g >= P.s || P.kind < 0 || P.kind > 2)) return hipErrorInvalidValue;
    for (int j = 0; j < 3; ++j)
        if (P.fin[j] < 0 || P.fin[j] > 2) return hipErrorInvalidValue;
    const int ncp = (P.np + 63) / 64;
    if (P.np >= kStagedNp) {
        // F fibre tiles per block so that its wavefronts have at least 4
        // (fibre tile, operator-row tile) pairs
        const int na = ((P.np + 15) & ~15) / 16;
        const int F = na >= 4 ? 1 : na >= 2 ? 2 : 4;
        const size_t lds = (size_t)P.s * F * ncp * 1024;
        if (lds > kStepLdsMax) return hipErrorInvalidValue;
        const int64_t btiles = P.batch * ((int64_t)P.np * P.np / 16 / F);
        const dim3 grid((unsigned)(btiles < kStepBlocksMax ? btiles : kStepBlocksMax));
        // 8 wavefronts only where the row tiles divide evenly among them:
        // with more than 32 KiB staged that is np > 240 (16 row tiles),
        // four chunk pairs
        const bool nw8 = lds > 32768 && (F * na) % 8 == 0;
        switch (ncp) {
            case 2: launch_staged<2, 4>(P, last, grid, lds, F, st); break;
            case 3: launch_staged<3, 4>(P, last, grid, lds, F, st); break;
            case 4:
                if (nw8)
                    launch_staged<4, 8>(P, last, grid, lds, F, st);
                else
                    launch_staged<4, 4>(P, last, grid, lds, F, st);
                break;
            default: return hipErrorInvalidValue;
        }
    } else {
        const bool half = P.np == 8;
        const int64_t tiles = P.batch * ((int64_t)P.np * P.np / (half ? 32 : 16));
        const int64_t want = (tiles + 3) / 4;
        const dim3 grid((unsigned)(want < kStepBlocksMax ? want : kStepBlocksMax));
        if (half)
            launch_direct<1, true>(P, last, grid, st);
        else if (ncp == 1)
            launch_direct<1, false>(P, last, grid, st);
        else
            launch_direct<2, false>(P, last, grid, st);
    }
    return hipGetLastError();
}

}  // namespace oz2
