// oz2_gemm.hip -- the s exact INT8 residue products of Ozaki scheme II on the
// gfx950 INT8 matrix cores (v_mfma_i32_32x32x32_i8), with the reduction
// mod m_t fused into the epilogue.
//
// "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs:
// Ozaki Scheme II on the Xe2 Architecture", Sec. 2.3 step 3: each product
// A^(t) B^(t) is exact with INT32 accumulation while k 128^2 < 2^31; Sec. 4.3:
// longer k is split into runs of at most 131008 positions, one launch per
// run, and the residues of the runs are summed mod m_t in the reconstruction
// (bitwise the same residue as an unsplit product).  "EmuGEMM: Fused Tensor Core Kernels
// for Precision Emulation", Sec. IV-A (Eq. 14-15): reducing the INT32
// accumulator on chip and writing only one byte per entry removes the INT32
// round trip; Sec. IV-B (Eq. 16-18): the three products of the complex 3M
// form run as three k-loops over one accumulator and only Re and Im leave
// the chip.  Here T1 mod m and then T1 + T2 mod m are parked in the output
// planes between the k-loops (each lane rereads only what it wrote), so no
// registers beyond one accumulator set are held across the loops.
//
// Data layout: both operands are k-contiguous planes (rows of op(A), columns
// of op(B)), zero-padded in k to a multiple of 64 and in rows to a multiple
// of 256, so the main loop has no bounds checks.  The output plane of
// modulus t is uint8 [n][m_pad] (column-major like C) holding C^(t) mod m_t
// in [0, m_t).
//
// Kernel shape: a 256-thread block (4 wavefronts, 2 x 2) computes a BM x BN
// tile of one modulus; each wavefront owns (BM/2) x (BN/2) accumulators in
// 32x32 MFMA tiles.  k advances in steps of 64 bytes staged through LDS with
// double buffering; global loads of step k+1 are in flight while step k is
// multiplied.  LDS rows are 64 bytes of four 16-byte chunks whose position
// is XOR-swizzled by the row index so that the 16-byte MFMA operand reads of
// 8 (or 16) consecutive rows hit distinct banks.  Blocks are remapped so
// that each of the 8 XCDs (which receive blocks round-robin) works on a
// contiguous range of tiles, grouped 8 tiles tall for L2 reuse.
#include "oz2_internal.h"

namespace oz2 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KSUB = BK / 32;
    static constexpr int CH = BK / 16;
    static constexpr int A_LD = BM * CH / NT, B_LD = BN * CH / NT;
    static constexpr int LDS_A = BM * BK, LDS_B = BN * BK;
    static_assert(A_LD * NT == BM * CH && B_LD * NT == BN * CH, "tile/thread mismatch");
};

__device__ __forceinline__ int swz(int row, int ch) { return ((row >> 1) ^ (row >> 3)) & (ch - 1); }

// INT32 accumulator -> [0, m): bias makes it non-negative (a multiple of m,
// chosen for |acc| <= 2^31 - 2^20 + 255), Barrett quotient floor(u R / 2^32)
// with R = floor(2^32/m) is floor(u/m) or one less.
__device__ __forceinline__ uint32_t acc_mod(int32_t acc, uint32_t m, uint32_t R, uint32_t bias) {
    const uint32_t u = (uint32_t)acc + bias;
    const uint32_t q = __umulhi(u, R);
    const uint32_t r = u - q * m;
    const uint32_t r2 = r - m;
    return r < r2 ? r : r2;
}

template <class T, bool CPLX>
__global__ __launch_bounds__(T::NT, 1) void residue_gemm_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(16))) int8_t smem[2 * (T::LDS_A + T::LDS_B)];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % T::WM, wn = wave / T::WM;

    // block -> (modulus, tile row, tile column)
    const int nb = gridDim.x;
    const int bid = blockIdx.x;
    const int lid = (nb & 7) == 0 ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
    const int tiles = P.tiles_m * P.tiles_n;
    const int t = lid / tiles;
    const int rem = lid % tiles;
    constexpr int GROUP = 8;
    const int per_group = GROUP * P.tiles_n;
    const int first_m = (rem / per_group) * GROUP;
    const int gsz = min(P.tiles_m - first_m, GROUP);
    const int in = rem % per_group;
    const int tm = first_m + in % gsz;
    const int tn = in / gsz;

    const uint32_t m = P.mod[t], R = P.barrett[t], bias = P.bias[t];
    const int64_t kp = P.kp;
    const int nk = P.k_steps;  // this launch covers k in [k_begin, k_begin + 64 k_steps)

    v16i acc[T::FM][T::FN];

    const int row_out0 = tm * T::BM + wm * T::WTM + 4 * (lane >> 5);
    const int col_out0 = tn * T::BN + wn * T::WTN + (lane & 31);

#pragma unroll 1
    for (int pass = 0; pass < (CPLX ? 3 : 1); ++pass) {
        const int8_t* Ag = P.A + pass * P.a_set_stride + (int64_t)t * P.mp * kp +
                           (int64_t)tm * T::BM * kp + P.k_begin;
        const int8_t* Bg = P.B + pass * P.b_set_stride + (int64_t)t * P.np * kp +
                           (int64_t)tn * T::BN * kp + P.k_begin;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

        v4i ra[T::A_LD], rb[T::B_LD];
        auto gload = [&](int kt) {
#pragma unroll
            for (int q = 0; q < T::A_LD; ++q) {
                const int idx = tid + q * T::NT;
                const int row = idx / T::CH, c = idx % T::CH;
                ra[q] = *(const v4i*)(Ag + (int64_t)row * kp + (int64_t)kt * T::BK + c * 16);
            }
#pragma unroll
            for (int q = 0; q < T::B_LD; ++q) {
                const int idx = tid + q * T::NT;
                const int row = idx / T::CH, c = idx % T::CH;
                rb[q] = *(const v4i*)(Bg + (int64_t)row * kp + (int64_t)kt * T::BK + c * 16);
            }
        };
        auto sstore = [&](int buf) {
            int8_t* As = smem + buf * (T::LDS_A + T::LDS_B);
            int8_t* Bs = As + T::LDS_A;
#pragma unroll
            for (int q = 0; q < T::A_LD; ++q) {
                const int idx = tid + q * T::NT;
                const int row = idx / T::CH, c = idx % T::CH;
                *(v4i*)(As + row * T::BK + ((c ^ swz(row, T::CH)) << 4)) = ra[q];
            }
#pragma unroll
            for (int q = 0; q < T::B_LD; ++q) {
                const int idx = tid + q * T::NT;
                const int row = idx / T::CH, c = idx % T::CH;
                *(v4i*)(Bs + row * T::BK + ((c ^ swz(row, T::CH)) << 4)) = rb[q];
            }
        };
        auto compute = [&](int buf) {
            const int8_t* As = smem + buf * (T::LDS_A + T::LDS_B);
            const int8_t* Bs = As + T::LDS_A;
#pragma unroll
            for (int ks = 0; ks < T::KSUB; ++ks) {
                const int c = ks * 2 + (lane >> 5);
                v4i a[T::FM], b[T::FN];
#pragma unroll
                for (int i = 0; i < T::FM; ++i) {
                    const int row = wm * T::WTM + i * 32 + (lane & 31);
                    a[i] = *(const v4i*)(As + row * T::BK + ((c ^ swz(row, T::CH)) << 4));
                }
#pragma unroll
                for (int j = 0; j < T::FN; ++j) {
                    const int row = wn * T::WTN + j * 32 + (lane & 31);
                    b[j] = *(const v4i*)(Bs + row * T::BK + ((c ^ swz(row, T::CH)) << 4));
                }
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
#pragma unroll
                    for (int j = 0; j < T::FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        };

        gload(0);
        sstore(0);
        __syncthreads();
#pragma unroll 1
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) gload(kt + 1);
            compute(kt & 1);
            if (more) sstore((kt + 1) & 1);
            __syncthreads();
        }

        // epilogue: lane holds rows 8g + 4(lane/32) + {0..3} of column lane%32
        // of every 32x32 tile, i.e. four consecutive bytes of the output plane
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const int64_t col = col_out0 + j * 32;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t r[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = acc_mod(acc[i][j][4 * g + e], m, R, bias);
                    const int64_t row = row_out0 + i * 32 + 8 * g;
                    uint8_t* re_dst = P.C + (int64_t)t * P.n * P.mp + col * P.mp + row;
                    uint8_t* im_dst = re_dst + P.c_set_stride;
                    if (col >= P.n) continue;
                    if (!CPLX || pass == 0) {
                        // real: the result; complex pass 0: T1 mod m parked in
                        // the Re plane (each lane rereads only its own words)
                        *(uint32_t*)re_dst = r[0] | (r[1] << 8) | (r[2] << 16) | (r[3] << 24);
                    } else if (pass == 1) {
                        // Re = T1 - T2; T1 + T2 parked in the Im plane
                        const uint32_t t1w = *(const uint32_t*)re_dst;
                        uint32_t re[4], sm[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t r1 = (t1w >> (8 * e)) & 0xffu;
                            const uint32_t x = r1 + m - r[e];
                            const uint32_t x1 = x - m;
                            re[e] = x < x1 ? x : x1;
                            const uint32_t y = r1 + r[e];
                            const uint32_t y1 = y - m;
                            sm[e] = y < y1 ? y : y1;
                        }
                        *(uint32_t*)re_dst = re[0] | (re[1] << 8) | (re[2] << 16) | (re[3] << 24);
                        *(uint32_t*)im_dst = sm[0] | (sm[1] << 8) | (sm[2] << 16) | (sm[3] << 24);
                    } else {
                        // Im = T3 - (T1 + T2)
                        const uint32_t sw = *(const uint32_t*)im_dst;
                        uint32_t im[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t x = r[e] + m - ((sw >> (8 * e)) & 0xffu);
                            const uint32_t x1 = x - m;
                            im[e] = x < x1 ? x : x1;
                        }
                        *(uint32_t*)im_dst = im[0] | (im[1] << 8) | (im[2] << 16) | (im[3] << 24);
                    }
                }
            }
        }
    }
}

using BigTile = Tile<256, 256, 64, 2, 2>;
using SmallTile = Tile<128, 128, 64, 2, 2>;

template <class T>
hipError_t gemm_go(GemmParams P, bool cplx, hipStream_t st) {
    P.tiles_m = (int)(P.mp / T::BM);
    P.tiles_n = (int)(P.np / T::BN);
    const int64_t nb = (int64_t)P.tiles_m * P.tiles_n * P.s;
    if (cplx)
        hipLaunchKernelGGL((residue_gemm_kernel<T, true>), dim3((unsigned)nb), dim3(T::NT), 0, st, P);
    else
        hipLaunchKernelGGL((residue_gemm_kernel<T, false>), dim3((unsigned)nb), dim3(T::NT), 0, st, P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_residue_gemm(const GemmParams& P, bool cplx, hipStream_t st) {
    if (P.mp % kPadM || P.np % kPadM || P.kp % kPadK) return hipErrorInvalidValue;
    // large outputs: 256 x 256 tiles; otherwise 128 x 128 for more blocks
    const int64_t big_blocks = (P.mp / 256) * (P.np / 256) * P.s;
    if (big_blocks >= 1024) return gemm_go<BigTile>(P, cplx, st);
    return gemm_go<SmallTile>(P, cplx, st);
}

}  // namespace oz2
