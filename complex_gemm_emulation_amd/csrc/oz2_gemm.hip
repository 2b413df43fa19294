// oz2_gemm.hip -- the s exact INT8 residue products of Ozaki scheme II on the
// gfx950 INT8 matrix cores (v_mfma_i32_16x16x64_i8), with the reduction
// mod m_t fused into the epilogue.
//
// "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs:
// Ozaki Scheme II on the Xe2 Architecture", Sec. 2.3 step 3: each product
// A^(t) B^(t) is exact with INT32 accumulation while k 128^2 < 2^31; Sec. 4.3:
// longer k is split into runs (here of at most 130816 positions), one launch
// per run, and the residues of the runs are summed mod m_t in the
// reconstruction (bitwise the same residue as an unsplit product).
// "EmuGEMM: Fused Tensor Core Kernels for Precision Emulation", Sec. IV-A
// (Eq. 14-15): reducing the INT32 accumulator on chip and writing one byte per
// entry removes the INT32 round trip; Sec. IV-B (Eq. 16-18): the three
// products of the complex 3M form run as three k-loops of one block and only
// Re and Im leave the chip.  Between the k-loops T1 mod m and then
// (T1 + T2) mod m stay in registers as packed bytes (a quarter of an
// accumulator set), so the epilogues of the three loops read no memory.
//
// Data layout: both operands are planes of 64-position k-panels (rows of
// op(A), columns of op(B), 64 contiguous bytes per row within a panel),
// zero-padded in k to a multiple of 256 and in rows to a multiple of 256, so
// the main loop has no bounds checks and one k step of a tile is one
// contiguous run of memory.  The output plane of modulus t is uint8
// [n][m_pad] (column-major like C) holding C^(t) mod m_t in [0, m_t).
//
// Kernel shapes (CDNA4).  Large products: a 256 x 256 tile of one modulus
// per block on 8 wavefronts of 128 x 64, on v_mfma_i32_16x16x64_i8 (one
// MFMA per 16 x 16 block and 64-byte k step).  k advances one 64-byte panel
// per step through four LDS stages filled by direct global->LDS loads
// (global_load_lds_dwordx4: no VGPR staging, no ds_write) issued three steps
// ahead.  The waves form two groups of four, waves 0-3 and 4-7, one of each
// per SIMD, that alternate every half step between a memory phase (read one
// k step's fragments from LDS into registers, issue their share of the
// loads) and a compute phase (that step's 32 MFMAs from registers), with a
// block barrier between phases and the second group one phase behind: on
// every SIMD one wave issues MFMAs while the other reads LDS (a ping-pong
// schedule, measured 1.3% faster than interleaving both in every wave).
// The 16 x 16 x 64 form does the same work as 32 x 32 x 32 with the same
// LDS traffic and accumulator count, but reads and writes half the
// accumulator bytes per multiply-add; since the GEMM on residue data is
// limited by power, not by issue (it runs at 72% of the INT8 peak on
// operands whose bits do not toggle, 49% on residues), that made it 11%
// faster at 8192^3.
//
// Small grids and short k: a 128 x 128 tile on 4 wavefronts of 64 x 64, also
// on v_mfma_i32_16x16x64_i8, with two LDS stages (the loads of step k + 1
// issued at the start of step k); several blocks per CU cover each other's
// waits and epilogues (16x16x64 made the k = 256 products' GEMM 13% faster
// than the 32x32x32 form it replaced).
//
// The loads are issued from inline assembly: the compiler cannot tell the
// stages of an LDS-DMA pipeline apart and would otherwise wait for every
// load in flight before each LDS read; the kernel's own vmcnt wait before
// each barrier orders them.  LDS rows are 64 bytes of four 16-byte chunks
// whose position is XOR-ed with (row/4) mod 4: the LDS serves a
// 16-byte-per-lane read 16 lanes per clock over 64 banks, and 16 consecutive
// rows then hit distinct bank groups.  Blocks are remapped so that each of
// the 8 XCDs (which receive blocks round-robin) works on a contiguous range
// of tiles, grouped 8 tiles tall for L2 reuse.
#include "oz2_internal.h"

namespace oz2 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* global_ptr_t;

constexpr int kBK = kGemmStepK;  // k bytes per step (two 32-wide MFMA sub-steps)
constexpr int kChunks = kBK / 16;
constexpr int kMaxStages = 4;  // LDS stages of the 256 x 256 tile; 128 x 128 tiles use 2
static_assert(kBK == kPanelK, "one k step is one panel");
static_assert(kPadK % (kBK * kMaxStages) == 0, "padded k holds whole stage rounds");

// INT32 accumulator -> [0, m): r = acc - m floor((acc + 1/2) / m) in FP64.
// (acc + 1/2) / m lies at least 1 / (2m) from an integer, and
// fma(acc, fl64(1/m), fl64(1/(2m))) is within 2^-20 / m of it for
// |acc| < 2^31, so the floor and r are exact (five full-rate FP64 and
// conversion instructions instead of two quarter-rate 32-bit multiplies).
__device__ __forceinline__ uint32_t acc_mod(int32_t acc, double m, double rcp, double half_rcp) {
    const double a = (double)acc;
    return (uint32_t)(int)fma(-m, floor(fma(a, rcp, half_rcp)), a);
}

__device__ __forceinline__ uint32_t pack4(const uint32_t r[4]) {
    return r[0] | (r[1] << 8) | (r[2] << 16) | (r[3] << 24);
}

// one wave-wide 1 KiB direct load: 16 bytes per lane from base + voff into
// LDS at lds + 16 lane (M0 holds lds; one wait state before the load).  M0
// is reserved to the compiler, which warns about the clobber; these kernels
// use M0 nowhere else (a CPU test checks the generated code for that).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_1k(const int8_t* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base)
                 : "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate: vmcnt(n) (bits 3:0 and 15:14), expcnt off, lgkmcnt(0)
// or off
constexpr int waitcnt_vm(int n, bool lgkm0) {
    return (n & 15) | ((n >> 4) << 14) | 0x0070 | (lgkm0 ? 0 : 0x0F00);
}

// Block order.  Blocks start roughly in index order and are dealt
// round-robin to the 8 XCDs (bid mod 8).  When the tiles of one modulus
// split evenly over the XCDs, blocks run modulus after modulus: while one
// modulus' planes are in use, the whole chip works on them, so they stay in
// the 256 MB last-level cache.  Each XCD owns a band of tile rows (or of
// tile columns) of that modulus and walks it in groups of at most 8 tiles,
// so that its 32 resident blocks share few A and B bands in its L2.
// Otherwise each XCD takes a contiguous range of blocks, grouped 8 tiles
// tall.
__device__ __forceinline__ void block_tile(int bid, int nb, int tiles_m, int tiles_n, int& t, int& tm, int& tn) {
    constexpr int GROUP = 8;
    const int tiles = tiles_m * tiles_n;
    if (tiles % 8 == 0 && (tiles_m % 8 == 0 || tiles_n % 8 == 0)) {
        t = bid / tiles;
        const int r = bid % tiles;
        const int x = r & 7, q = r >> 3;
        const bool rows = tiles_m % 8 == 0;
        const int bm = rows ? tiles_m / 8 : tiles_m;  // this XCD's band
        const int bn = rows ? tiles_n : tiles_n / 8;
        const int g = min(bm, GROUP);                  // group height within the band
        const int per_group = g * bn;
        const int first = (q / per_group) * g;
        const int gsz = min(bm - first, g);
        const int in = q % per_group;
        tm = (rows ? x * bm : 0) + first + in % gsz;
        tn = (rows ? 0 : x * bn) + in / gsz;
        return;
    }
    const int lid = (nb & 7) == 0 ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid;
    t = lid / tiles;
    const int rem = lid % tiles;
    const int per_group = GROUP * tiles_n;
    const int first_m = (rem / per_group) * GROUP;
    const int gsz = min(tiles_m - first_m, GROUP);
    const int in = rem % per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

// The 256 x 256 tile on v_mfma_i32_16x16x64_i8: one MFMA covers a 16 x 16
// block and a whole 64-byte k step.  8 wavefronts of 128 x 64 (8 x 4 blocks,
// 32 accumulators of 4 registers each), four LDS stages, loads three steps
// ahead and the ping-pong schedule described at the top.  A fragment is 16 rows x 64 bytes:
// lane l reads row l mod 16, chunk l / 16.  Output: lane l holds column
// l mod 16, rows 4 (l / 16) + {0..3} of a block: four consecutive bytes of
// the output plane.
template <bool CPLX>
__global__ __launch_bounds__(512, 1) void residue_gemm16_kernel(GemmParams P) {
    constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NW = 8, kStages = 4;
    constexpr int WTM = BM / WM, WTN = BN / WN, GM = WTM / 16, GN = WTN / 16;
    constexpr int LOADS_A = BM * kChunks / 64 / NW, LOADS_B = BN * kChunks / 64 / NW;
    constexpr int STAGE = (BM + BN) * kBK;
    __shared__ __attribute__((aligned(1024))) int8_t sS0[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t sS1[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t sS2[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t sS3[STAGE];
    auto stage = [&](int st) -> int8_t* { return st == 0 ? sS0 : st == 1 ? sS1 : st == 2 ? sS2 : sS3; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave % WM, wn = wave / WM;
    int t, tm, tn;
    block_tile(blockIdx.x, gridDim.x, P.tiles_m, P.tiles_n, t, tm, tn);
    const uint32_t m = P.mod[t];
    const double dm = (double)m, rcp = P.rcp[t], half_rcp = 0.5 * rcp;
    const int64_t kp = P.kp;
    const int nk = P.k_steps;

    uint32_t goffA[LOADS_A], goffB[LOADS_B];
#pragma unroll
    for (int q = 0; q < LOADS_A; ++q) {
        const int piece = (wave * LOADS_A + q) * 64 + lane;
        const int row = piece / kChunks, pos = piece % kChunks;
        goffA[q] = (uint32_t)(row * kBK + ((pos ^ ((row >> 2) & 3)) << 4));
    }
#pragma unroll
    for (int q = 0; q < LOADS_B; ++q) {
        const int piece = (wave * LOADS_B + q) * 64 + lane;
        const int row = piece / kChunks, pos = piece % kChunks;
        goffB[q] = (uint32_t)(row * kBK + ((pos ^ ((row >> 2) & 3)) << 4));
    }
    const int r16 = lane & 15, c16 = lane >> 4;
    const int sw = (c16 ^ ((r16 >> 2) & 3)) << 4;  // swizzled chunk of this lane's row
    const int aoff = (wm * WTM + r16) * kBK + sw;
    const int boff = BM * kBK + (wn * WTN + r16) * kBK + sw;
    const int64_t row_out0 = (int64_t)tm * BM + wm * WTM + 4 * c16;
    const int64_t col_out0 = (int64_t)tn * BN + wn * WTN + r16;
    const int64_t panelA = P.a_rows * kBK, panelB = P.b_rows * kBK;

    v4i acc[GM][GN];
    v4i fa[GM], fb[GN];
    uint32_t park[CPLX ? GM : 1][CPLX ? GN : 1];

#pragma unroll 1
    for (int pass = 0; pass < (CPLX ? 3 : 1); ++pass) {
        const int8_t* Ag = P.A + pass * P.a_set_stride + (int64_t)t * P.a_rows * kp + (P.k_begin / kBK) * panelA +
                           (int64_t)tm * BM * kBK;
        const int8_t* Bg = P.B + pass * P.b_set_stride + (int64_t)t * P.b_rows * kp + (P.k_begin / kBK) * panelB +
                           (int64_t)tn * BN * kBK;
        auto issue = [&](int kt, int st) {
            const int8_t* Ak = Ag + (int64_t)kt * panelA;
            const int8_t* Bk = Bg + (int64_t)kt * panelB;
            const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)stage(st);
#pragma unroll
            for (int q = 0; q < LOADS_A; ++q) dma_1k(Ak, goffA[q], lds + (wave_u * LOADS_A + q) * 1024);
#pragma unroll
            for (int q = 0; q < LOADS_B; ++q) dma_1k(Bk, goffB[q], lds + BM * kBK + (wave_u * LOADS_B + q) * 1024);
        };
        constexpr int kLoadsPerStep = LOADS_A + LOADS_B;
        constexpr int kWaitPP = waitcnt_vm(2 * kLoadsPerStep, true);
        auto mem = [&](int st, int kdma, int st_dma) {
            const int8_t* S = stage(st);
#pragma unroll
            for (int i = 0; i < GM; ++i) fa[i] = *(const v4i*)(S + aoff + i * 16 * kBK);
#pragma unroll
            for (int j = 0; j < GN; ++j) fb[j] = *(const v4i*)(S + boff + j * 16 * kBK);
            issue(kdma, st_dma);
        };
        auto comp = [&]() {
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < GM; ++i)
#pragma unroll
                for (int j = 0; j < GN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        };
        auto sync = [&]() {
            __builtin_amdgcn_s_waitcnt(kWaitPP);
            __syncthreads();
        };
#pragma unroll
        for (int i = 0; i < GM; ++i)
#pragma unroll
            for (int j = 0; j < GN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
        const int grp = wave_u >> 2;
#pragma unroll
        for (int j = 0; j < 3; ++j) issue(j, j);
        sync();
        if (grp == 1) sync();
#pragma unroll 1
        for (int kt = 0; kt < nk; kt += 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mem(j, min(kt + j + 3, nk - 1), (j + 3) & 3);
                sync();
                comp();
                sync();
            }
        }
        if (grp == 0) sync();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0, false));
        __syncthreads();

#pragma unroll
        for (int i = 0; i < GM; ++i) {
#pragma unroll
            for (int j = 0; j < GN; ++j) {
                const int64_t col = col_out0 + j * 16;
                const int64_t row = row_out0 + i * 16;
                uint32_t r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = acc_mod(acc[i][j][e], dm, rcp, half_rcp);
                uint8_t* re_dst = P.C + (int64_t)t * P.n * P.mp + col * P.mp + row;
                if (!CPLX) {
                    if (col < P.n) *(uint32_t*)re_dst = pack4(r);
                } else if (pass == 0) {
                    park[i][j] = pack4(r);
                } else if (pass == 1) {
                    const uint32_t t1w = park[i][j];
                    uint32_t re[4], smv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t r1 = (t1w >> (8 * e)) & 0xffu;
                        const uint32_t x = r1 + m - r[e];
                        const uint32_t x1 = x - m;
                        re[e] = x < x1 ? x : x1;
                        const uint32_t y = r1 + r[e];
                        const uint32_t y1 = y - m;
                        smv[e] = y < y1 ? y : y1;
                    }
                    park[i][j] = pack4(smv);
                    if (col < P.n) *(uint32_t*)re_dst = pack4(re);
                } else {
                    const uint32_t swd = park[i][j];
                    uint32_t im[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t x = r[e] + m - ((swd >> (8 * e)) & 0xffu);
                        const uint32_t x1 = x - m;
                        im[e] = x < x1 ? x : x1;
                    }
                    if (col < P.n) *(uint32_t*)(re_dst + P.c_set_stride) = pack4(im);
                }
            }
        }
    }
}

// The 128 x 128 tile on v_mfma_i32_16x16x64_i8: 4 wavefronts of 64 x 64
// (4 x 4 blocks), two LDS stages, the loads of step k + 1 issued after the
// barrier that opens step k; several blocks per CU cover each other's waits.
template <bool CPLX>
__global__ __launch_bounds__(256, 2) void residue_gemm16s_kernel(GemmParams P) {
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2, NW = 4;
    constexpr int WTM = BM / WM, WTN = BN / WN, GM = WTM / 16, GN = WTN / 16;
    constexpr int LOADS_A = BM * kChunks / 64 / NW, LOADS_B = BN * kChunks / 64 / NW;
    constexpr int STAGE = (BM + BN) * kBK;
    __shared__ __attribute__((aligned(1024))) int8_t sS0[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t sS1[STAGE];
    auto stage = [&](int st) -> int8_t* { return st == 0 ? sS0 : sS1; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave % WM, wn = wave / WM;
    int t, tm, tn;
    block_tile(blockIdx.x, gridDim.x, P.tiles_m, P.tiles_n, t, tm, tn);
    const uint32_t m = P.mod[t];
    const double dm = (double)m, rcp = P.rcp[t], half_rcp = 0.5 * rcp;
    const int64_t kp = P.kp;
    const int nk = P.k_steps;

    uint32_t goffA[LOADS_A], goffB[LOADS_B];
#pragma unroll
    for (int q = 0; q < LOADS_A; ++q) {
        const int piece = (wave * LOADS_A + q) * 64 + lane;
        const int row = piece / kChunks, pos = piece % kChunks;
        goffA[q] = (uint32_t)(row * kBK + ((pos ^ ((row >> 2) & 3)) << 4));
    }
#pragma unroll
    for (int q = 0; q < LOADS_B; ++q) {
        const int piece = (wave * LOADS_B + q) * 64 + lane;
        const int row = piece / kChunks, pos = piece % kChunks;
        goffB[q] = (uint32_t)(row * kBK + ((pos ^ ((row >> 2) & 3)) << 4));
    }
    const int r16 = lane & 15, c16 = lane >> 4;
    const int sw = (c16 ^ ((r16 >> 2) & 3)) << 4;
    const int aoff = (wm * WTM + r16) * kBK + sw;
    const int boff = BM * kBK + (wn * WTN + r16) * kBK + sw;
    const int64_t row_out0 = (int64_t)tm * BM + wm * WTM + 4 * c16;
    const int64_t col_out0 = (int64_t)tn * BN + wn * WTN + r16;
    const int64_t panelA = P.a_rows * kBK, panelB = P.b_rows * kBK;

    v4i acc[GM][GN];
    v4i fa[GM], fb[GN];
    uint32_t park[CPLX ? GM : 1][CPLX ? GN : 1];

#pragma unroll 1
    for (int pass = 0; pass < (CPLX ? 3 : 1); ++pass) {
        const int8_t* Ag = P.A + pass * P.a_set_stride + (int64_t)t * P.a_rows * kp + (P.k_begin / kBK) * panelA +
                           (int64_t)tm * BM * kBK;
        const int8_t* Bg = P.B + pass * P.b_set_stride + (int64_t)t * P.b_rows * kp + (P.k_begin / kBK) * panelB +
                           (int64_t)tn * BN * kBK;
        auto issue = [&](int kt, int st) {
            const int8_t* Ak = Ag + (int64_t)kt * panelA;
            const int8_t* Bk = Bg + (int64_t)kt * panelB;
            const uint32_t lds = (uint32_t)(uintptr_t)(lds_ptr_t)stage(st);
#pragma unroll
            for (int q = 0; q < LOADS_A; ++q) dma_1k(Ak, goffA[q], lds + (wave_u * LOADS_A + q) * 1024);
#pragma unroll
            for (int q = 0; q < LOADS_B; ++q) dma_1k(Bk, goffB[q], lds + BM * kBK + (wave_u * LOADS_B + q) * 1024);
        };
#pragma unroll
        for (int i = 0; i < GM; ++i)
#pragma unroll
            for (int j = 0; j < GN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
        issue(0, 0);
        auto step = [&](int st, int kdma) {
            // this step's loads have landed and every wave is done with the
            // other stage; refill it with the next step, then read and multiply
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0, true));
            __syncthreads();
            issue(kdma, st ^ 1);
            const int8_t* S = stage(st);
#pragma unroll
            for (int i = 0; i < GM; ++i) fa[i] = *(const v4i*)(S + aoff + i * 16 * kBK);
#pragma unroll
            for (int j = 0; j < GN; ++j) fb[j] = *(const v4i*)(S + boff + j * 16 * kBK);
#pragma unroll
            for (int i = 0; i < GM; ++i)
#pragma unroll
                for (int j = 0; j < GN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        };
#pragma unroll 1
        for (int kt = 0; kt < nk; kt += 2) {
            // past the last step the loads repeat the last step (the count per step stays the same)
            step(0, min(kt + 1, nk - 1));
            step(1, min(kt + 2, nk - 1));
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0, false));
        __syncthreads();

#pragma unroll
        for (int i = 0; i < GM; ++i) {
#pragma unroll
            for (int j = 0; j < GN; ++j) {
                const int64_t col = col_out0 + j * 16;
                const int64_t row = row_out0 + i * 16;
                uint32_t r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = acc_mod(acc[i][j][e], dm, rcp, half_rcp);
                uint8_t* re_dst = P.C + (int64_t)t * P.n * P.mp + col * P.mp + row;
                if (!CPLX) {
                    if (col < P.n) *(uint32_t*)re_dst = pack4(r);
                } else if (pass == 0) {
                    park[i][j] = pack4(r);
                } else if (pass == 1) {
                    const uint32_t t1w = park[i][j];
                    uint32_t re[4], smv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t r1 = (t1w >> (8 * e)) & 0xffu;
                        const uint32_t x = r1 + m - r[e];
                        const uint32_t x1 = x - m;
                        re[e] = x < x1 ? x : x1;
                        const uint32_t y = r1 + r[e];
                        const uint32_t y1 = y - m;
                        smv[e] = y < y1 ? y : y1;
                    }
                    park[i][j] = pack4(smv);
                    if (col < P.n) *(uint32_t*)re_dst = pack4(re);
                } else {
                    const uint32_t swd = park[i][j];
                    uint32_t im[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t x = r[e] + m - ((swd >> (8 * e)) & 0xffu);
                        const uint32_t x1 = x - m;
                        im[e] = x < x1 ? x : x1;
                    }
                    if (col < P.n) *(uint32_t*)(re_dst + P.c_set_stride) = pack4(im);
                }
            }
        }
    }
}

// big: the 256 x 256 tile on 8 wavefronts; otherwise the 128 x 128 tile on 4
hipError_t gemm_go(GemmParams P, bool big, bool cplx, hipStream_t st) {
    const int T = big ? 256 : 128;
    P.tiles_m = (int)(P.mp / T);
    P.tiles_n = (int)(P.np / T);
    const int64_t nb = (int64_t)P.tiles_m * P.tiles_n * P.s;
    const dim3 grid((unsigned)nb), block(big ? 512 : 256);
    if (big && cplx)
        hipLaunchKernelGGL((residue_gemm16_kernel<true>), grid, block, 0, st, P);
    else if (big)
        hipLaunchKernelGGL((residue_gemm16_kernel<false>), grid, block, 0, st, P);
    else if (cplx)
        hipLaunchKernelGGL((residue_gemm16s_kernel<true>), grid, block, 0, st, P);
    else
        hipLaunchKernelGGL((residue_gemm16s_kernel<false>), grid, block, 0, st, P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_residue_gemm(const GemmParams& P, bool cplx, hipStream_t st) {
    if (P.mp % kPadM || P.np % kPadM || P.kp % kPadK || P.k_begin % (kBK * kMaxStages))
        return hipErrorInvalidValue;
    if (P.a_rows < P.mp || P.b_rows < P.np || P.a_rows % kPadM || P.b_rows % kPadM) return hipErrorInvalidValue;
    if (P.k_steps <= 0 || P.k_steps % kMaxStages || P.k_begin + (int64_t)P.k_steps * kBK > P.kp)
        return hipErrorInvalidValue;
    // 256 x 256 tiles on 8 wavefronts with four stages unless the grid is
    // small or the k-loop very short.  Otherwise 128 x 128 tiles on 4
    // wavefronts with two stages (32 KiB of LDS, several blocks per CU, whose
    // epilogues overlap the others' MFMAs).  Measured at 8192 x k x 8192,
    // s = 8: faster at k = 256, even at k = 1024, and slower at
    // 16384 x 2048 x 16384 (twice the L2->LDS bytes per MAC).
    const int64_t big_blocks = (P.mp / 256) * (P.np / 256) * P.s;
    return gemm_go(P, big_blocks >= 512 && (int64_t)P.k_steps * kBK > 512, cplx, st);
}

}  // namespace oz2
