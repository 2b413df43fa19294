// oz2_internal.h -- kernel parameter blocks and launchers shared by the
// C-ABI layer (oz2_api.cpp) and the device code (oz2_kernels.hip,
// oz2_gemm.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "oz2_plan.h"

namespace oz2 {

// Residue planes of op(A) and op(B) are int8 [sets][s][k_pad/64][rows_pad][64]:
// k-panels of 64 positions, each panel holding every row (a row of op(A) or a
// column of op(B)) as 64 contiguous bytes, zero-padded in rows and k; sets = 1
// (real) or 3 (complex: re, im, re+im).  One GEMM k step of a 256-row tile is
// then 16 KiB of contiguous memory.
// Product residues are uint8 [outs][s][n][m_pad] holding values in [0, m_t)
// (outs = 1 real, 2 complex: Re, Im), i.e. column-major like C.
constexpr int kPadM = 256;   // row padding of the A planes / product planes
constexpr int kPadK = 256;   // k padding of the planes (four GEMM k steps)
constexpr int kPanelK = 64;  // k positions per panel of the residue planes
constexpr int kGemmStepK = 64;   // k bytes per GEMM k step (one panel)

// Vector layout of an operand as seen by scan/encode: vector v (a row of
// op(A) or a column of op(B)) has element p at X[v*ld + p] when contiguous,
// at X[v + p*ld] otherwise (complex: in units of complex128).
struct ScanParams {
    const double* X;
    int64_t ld;
    int64_t nvec;
    int64_t k;
    int64_t pchunk;     // strided scan: p-range per block
    uint64_t* amax;     // bit pattern of max |x| (sign cleared) per vector
};

struct EncodeParams {
    const double* X;
    int64_t ld;
    int64_t nvec, k;         // logical sizes
    int64_t vpad, kpad;      // plane row count and row length
    int64_t set_stride;      // bytes between the sets of planes
    const uint64_t* amax;
    int8_t* planes;
    int conj;                // negate imaginary parts (op = 'C')
    int t, s;
    uint32_t mod[kMaxS], K[kMaxS];
    uint32_t c[kMaxS][kExtWords];     // byte-limb constants (see oz2_device.h)
    float frcp[kMaxS];                // fl32(1 / m)
    float foffb[kMaxS];               // fl32((hb + 1/2 - 128) / m) (oz2_plan.h)
};

struct GemmParams {
    const int8_t* A;   // planes of op(A): [sets][s][kp/64][a_rows][64], from row 0 of this product
    const int8_t* B;   // planes of op(B): [sets][s][kp/64][b_rows][64], from column 0 of this product
    uint8_t* C;        // [outs][s][n][mp]
    int64_t mp, np, kp, n;     // this product's padded rows, columns and k; n columns of C
    int64_t a_rows, b_rows;    // rows per k-panel of the planes (>= mp, np; larger for a block of bigger planes)
    int64_t a_set_stride, b_set_stride, c_set_stride;  // bytes
    int s;
    int tiles_m, tiles_n;
    int64_t k_begin;   // first k position of this launch (multiple of 256)
    int k_steps;       // 64-wide k steps of this launch (multiple of 4): <= 2044 keeps INT32 exact
    uint32_t mod[kMaxS];
    double rcp[kMaxS];   // fl64(1 / m)
};

struct ReconParams {
    const uint8_t* R;       // product residues [chunks][outs][s][n][mp]
    int64_t mp, m, n;
    int64_t r_set_stride;   // bytes between Re and Im residues
    int64_t r_chunk_stride; // bytes between the residues of successive k runs
    int chunks;             // k runs whose residues are summed mod m_t
    const uint64_t* amaxA;
    const uint64_t* amaxB;
    double* C;
    int64_t ldc;
    double alpha[2], beta[2];
    int t, s;
    uint32_t* chat;         // optional debug copy of c_hat words [outs][n][mp][NL]
    uint32_t Y2[kMaxS / 2]; // round(2^16 y_t / m_t) of moduli 2u and 2u+1 in 16-bit halves
    uint32_t W2[kMaxS / 2][kMaxLimb16];  // 16-bit limbs of W_(2u) | W_(2u+1) << 16
    uint32_t M16[kMaxLimb16];
    uint32_t mod[kMaxS];
};

// Fused path for a short inner dimension (oz2_small.hip): every step of the
// method for a 16 x 16 output tile in one wavefront, batched with strides.
constexpr int64_t kSmallMaxK = 32;
struct SmallParams {
    const double* A;
    int64_t lda, strideA;      // strides in doubles; 0 shares the operand
    const double* B;
    int64_t ldb, strideB;
    double* C;
    int64_t ldc, strideC;
    int64_t m, n, k, batch;
    int transa, transb;        // 1 = transposed ('T' or 'C')
    int tiles_m, tiles_n;      // filled by the launcher
    int64_t tiles_total;
    int tiles_per_wave;
    double alpha, beta;
    int t, s;
    uint32_t mod[kMaxS], K[kMaxS];
    double rcp[kMaxS];                // fl64(1 / m)
    uint32_t c[kMaxS][kExtWords];     // byte-limb constants (see oz2_device.h)
    float frcp[kMaxS];                // fl32(1 / m)
    float foffb[kMaxS];               // fl32((hb + 1/2 - 128) / m) (oz2_plan.h)
    uint32_t Y2[kMaxS / 2];           // round(2^16 y_t / m_t), pairs as in ReconParams
    uint32_t W2[kMaxS / 2][kMaxLimb16];  // 16-bit limbs of W_(2u) | W_(2u+1) << 16
    uint32_t M16[kMaxLimb16];
};

// Persistent tensor-mode chain, OzII-RescaleBE ("You Only Convert Twice:
// Ozaki Scheme II for Chained Tensor Mode Products", Sec. 5.2 and
// Algorithm 7): Y = X x_{m1} A1 x_{m2} A2 ... for a batch of n x n x n
// tensors, d operators, by default along the directions in turn.  For
// n <= kChainN one block per tensor keeps the residues in LDS for the whole
// chain (oz2_chain.hip); larger tensors keep them in HBM between one kernel
// per product (oz2_chain_hbm.hip).
constexpr int kChainN = 16;      // tensor side of the LDS kernel's tiles (n <= 16 is zero padded)
constexpr int kChainMaxN = 256;  // tensor side of the HBM-resident kernels
constexpr int kChainMaxS = 16;   // moduli: one LDS buffer of 16 residue planes (64 KiB)
constexpr int kChainMaxD = 8;    // chain depth: operators
// The residue constants of the chain's moduli (by modulus index) for the
// chain kernels' encode, from the GEMM path's moduli plan (oz2_plan.h): the
// byte-limb identity of the encoder with the standard width.
struct ChainEncodeConsts {
    uint32_t K128[kChainMaxS];            // ((-2^62) mod m) + 128
    uint32_t c4[kChainMaxS][kStdWords];   // byte j of word p: 2^(32p + 8j) mod m
    float mod[kChainMaxS], frcp[kChainMaxS], foffb[kChainMaxS];
};
struct ChainDropTable;
struct ChainCrtTable;

struct ChainParams {
    const double* X;             // [batch][n^3] column-major tensors
    double* Y;
    int64_t batch;
    int n, s, b, d;
    int g[kChainMaxD];           // moduli dropped after product i (g[d - 1] = 0)
    int crt[kChainMaxD];         // 1: 1 <= g[i] <= 14 and after product i's drops |X_g| <= (1/2 - 2^-13) M
                                 // (M: the kept moduli), so that its base extension may take the CRT form
    const ChainCrtTable* crts;   // device [d] per-product CRT tables (chain_crt_table), or null: the
                                 // mixed-radix base extension everywhere
    // residue layout: position 0 of a plane row is the contracted direction.
    // m0: direction at position 0 before the first product (positions hold
    // m0, m0 + 1, m0 + 2 mod 3); kind[i]: how product i's output is stored
    // (0: the lane's four entries contiguous, 1 and 2: 16 bytes apart, see
    // oz2_chain.hip); fin: directions of the last product's entry, fibre
    // and output indices; cyclic: the modes are 0, 1, 2, 0, ...
    int m0, cyclic;
    int kind[kChainMaxD];
    int fin[3];
    double Qd;                   // fl64 product of the dropped moduli, in drop order
    const int8_t* ops;           // device [d][kChainMaxS][16][16] centred residues of the integer operators, by modulus index
    const float* tab;            // device ChainTables (below)
    const ChainDropTable* split; // device: the two-block reconstruction's table (chain_split_table)
    const ChainDropTable* drops; // device [d]: product i's drop table (chain_drop_table; the last: split)
    ChainEncodeConsts enc;       // the encode's residue constants
};

// Per non-final product with 1 <= g <= 14 drops: the base extension of X_g
// from its kept slots 0 .. keep = 15 - g (M the product of their moduli) to
// the dropped slots by the Chinese remainder theorem instead of mixed-radix
// digits.  With xi_i = [r_i cinv_i]_{m_i}, cinv_i = [(M / m_i)^{-1}]_{m_i},
// sum_i xi_i M / m_i = X_g + alpha M for the integer
// alpha = round(sum_i xi_i / m_i), so that
// [X_g]_p = [sum_i xi_i [M / m_i]_{m_p} - alpha [M]_{m_p}]_{m_p}.
// Packed in one 16 x 16 block, centred values: w[0][i] = cinv_i (kept i),
// w[1][p] = [M]_{m_p} (dropped p), w[p][i] = [M / m_i]_{m_p} (dropped p,
// kept i); rows 0 and 1 are kept slots since keep >= 1.  Zero elsewhere and
// for slots of modulus 1.  Used only where the plan bounds |X_g| by
// (1/2 - 2^-13) M (ChainParams::crt), which keeps the rounding of alpha away
// from a tie.
struct ChainCrtTable {
    float w[kChainMaxS][kChainMaxS];
};

// Constant tables of the chain kernel, in slot order (the s moduli
// right-aligned in kChainMaxS slots, descending; unused slots hold 1)
struct ChainTables {
    float inv[kChainMaxS][kChainMaxS];    // m_i^{-1} mod m_j (i != j), in [0, m_j)
    union {
        float omega[kChainMaxS][kChainMaxS];  // [prod_{l<i} m_l]_{m_j}, centred
        ChainCrtTable crt;  // in the LDS kernel's CRT instances: the current product's CRT table
    };
    float mod[kChainMaxS];                // m_u
    float rmod[kChainMaxS];               // fl32(1 / m_u)
    float ohalf[kChainMaxS];              // fl32(1/2 - 128 rmod[u]): reduction of an accumulator offset by 128
    int fexp[3][kChainN];                 // row exponents left pending on each direction (0 for padding)
};

// Per non-final product with g >= 1 drops (slots 15, 14, .. 15 - g + 1 in
// that order, q_j = the modulus of slot 15 - j, Q = prod_{j<g} q_j): the
// weights that take the kept residues of X to those of X_g = (X - D) / Q in
// one sum (D from the mixed-radix digits d_j of X over q_0, q_1, ..):
// [X_g]_p = [r_p qinv[p] + sum_{j<g} d_j nw[j][p]]_{m_p}.  Centred values,
// zero for j >= g, for the dropped slots and for slots of modulus 1.
struct ChainDropTable {
    float qinv[kChainMaxS];                 // [Q^{-1}]_{m_p}
    float nw[kChainMaxS - 1][kChainMaxS];   // -[prod_{l<j} q_l Q^{-1}]_{m_p}
};
void chain_drop_table(const ChainTables& T, int g, ChainDropTable* D);
void chain_crt_table(const ChainTables& T, int g, ChainCrtTable* C);
// The last product's table for the reconstruction's digits in blocks of
// `split` slots (16 / split blocks): after block b (slots lo .. lo + split
// - 1, M_b their moduli's product) the later slots p get the residues of
// (X_b - A_b) / M_b, with the weights in rows b (split + 1) .. b (split + 1)
// + split of the table (row 0 is qinv, row r > 0 is nw[r - 1]): first
// [M_b^{-1}]_{m_p}, then -[prod_{lo <= l < lo + i} m_l M_b^{-1}]_{m_p} for
// i = 0 .. split - 1; centred, zero elsewhere and for slots of modulus 1.
// Needs (16 / split - 1)(split + 1) <= 16 rows: split = 4 or 8.
void chain_split_table(const ChainTables& T, int split, ChainDropTable* D);
constexpr int kChainSplit = 4;      // slots per block of the reconstruction: the LDS kernel, the staged HBM one
constexpr int kChainSplitWide = 8;  // the direct HBM kernel (fewer registers; 4 spills there)
constexpr int kChainStagedNp = 96;  // padded sides from which the HBM product kernels stage their fibre tiles

// Host planning of the chain (Algorithms 2, 3 and 5 of the chain page, with
// the pending row scales of a direction folded into the next operator on
// it, Sec. 5.2): the significand bits b, the drop counts g, the effective
// integer operators' residues and the residue layout of every product.
// ops: d HOST n x n column-major operators; modes: d directions in
// {0, 1, 2}; 1 <= n <= kChainMaxN.  Writes P (all but the device pointers
// and the per-call fields), T (T->fexp only for n <= kChainN), ops_res
// [d][s][n][n] (operator i, modulus index q, row a, column k: the centred
// residue of the integer operator) and fexp [3][n] (the row exponents left
// pending on each direction).  Returns 0, -(i + 1) for a non-finite entry in
// operator i, or OZ2_STATUS_RANGE when no b in [1, 53] passes.
int chain_plan(int s, int n, int d, const double* const* ops, const int* modes, ChainParams* P,
               ChainTables* T, int8_t* ops_res, int* fexp);

// One launch of the HBM-resident chain (oz2_chain_hbm.hip).  Every residue
// plane holds each tensor as np^3 bytes, np = n rounded up to a multiple of
// 8 in every direction: position (p0, p1, p2) at p0 + np p1 + np^2 p2, p0 the
// direction the next product contracts; fibre f = p1 + np p2 is the row of
// np bytes at f np.  Padding positions hold residues too (of zero, or of
// products of padding) and never reach a result: the operators' columns
// k >= n are zero, and rows, fibres and outputs beyond n are not stored.
struct ChainHbmParams {
    const double* X;             // [batch][n^3] column-major tensors
    double* Y;
    int64_t batch;
    int n, np, s, b;
    int m0;                      // direction at position 0 of the encoded planes
    int g;                       // moduli dropped after this product
    int kind;                    // this product's output layout (as ChainParams::kind)
    int fin[3];                  // the last product's entry, fibre and output directions
    double Qd;                   // as ChainParams::Qd
    const int8_t* ops;           // [s][ap / 16][ncp][64][16] this product's operator residues in MFMA fragment
                                 // order (ap = np rounded up to 16, ncp = np / 64 rounded up)
    const float* tab;            // ChainTables
    const ChainDropTable* drop;  // this product's drop weights (g >= 1; the last product: chain_split_table)
    const ChainCrtTable* crt;    // this product's CRT base extension, or null: the mixed-radix form
    const int* fexp;             // [3][np] row exponents left pending on each direction
    unsigned long long* smax;    // [batch] max |x| bit pattern of each tensor (0 before the scan)
    const int8_t* in;            // planes [s][batch][np^3] read by this product
    int8_t* out;                 // planes written by the encode or a non-final product
    int64_t pstride;             // bytes between planes: batch np^3
};

struct CrtTestParams {
    const uint8_t* R;  // [s][count]
    int64_t count;
    uint32_t* words;   // [count][NL]
    int s;
    uint32_t Y2[kMaxS / 2];
    uint32_t W2[kMaxS / 2][kMaxLimb16];  // 16-bit limbs of W_(2u) | W_(2u+1) << 16
    uint32_t M16[kMaxLimb16];
};

// The fixed device scratch of oz2_dgemm_noalloc (oz2_scratch.hip): one array
// of kScratchBytes per GPU.  scratch_address gives its device address on
// `device`, which must be the current device; 0 or an OZ2_STATUS_* code.
constexpr size_t kScratchBytes = size_t(128) << 20;
int scratch_address(int device, void** out);

// launchers (return hipError_t of the launch)
hipError_t launch_fill_u64(uint64_t* p, int64_t n, uint64_t value, hipStream_t st);
hipError_t launch_scan(const ScanParams& P, bool contiguous, bool cplx, hipStream_t st);
hipError_t launch_encode(const EncodeParams& P, bool contiguous, bool cplx, bool ext,
                         hipStream_t st);
hipError_t launch_residue_gemm(const GemmParams& P, bool cplx, hipStream_t st);
hipError_t launch_reconstruct(const ReconParams& P, int NL, bool cplx, bool beta_nonzero,
                              hipStream_t st);
hipError_t launch_scale_c(double* C, int64_t m, int64_t n, int64_t ldc, const double beta[2],
                          bool cplx, hipStream_t st);
hipError_t launch_crt_test(const CrtTestParams& P, int NL, hipStream_t st);
hipError_t launch_small_gemm(SmallParams P, int NL, bool beta_nonzero, hipStream_t st);
hipError_t launch_chain(const ChainParams& P, hipStream_t st);
hipError_t launch_chain_scan(const ChainHbmParams& P, hipStream_t st);
hipError_t launch_chain_encode(const ChainHbmParams& P, const ChainEncodeConsts& E, hipStream_t st);
hipError_t launch_chain_step(const ChainHbmParams& P, bool last, hipStream_t st);

}  // namespace oz2
