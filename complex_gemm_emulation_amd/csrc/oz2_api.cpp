// oz2_api.cpp -- the C ABI declared in include/oz2.h: argument checking,
// BLAS quick returns, the per-call plan (scaling width, padding, workspace
// layout) and the launch sequence scan -> encode -> residue GEMM ->
// reconstruct on the handle's stream.
//
// "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs:
// Ozaki Scheme II on the Xe2 Architecture": Sec. 4 (the pipeline runs
// entirely on the device; the host only computes O(s) tables), Sec. 6 (one
// in-order queue, asynchronous submission; workspace reused across calls and
// capped by a resident-memory hint), Sec. 9.1 (interface = dgemm/zgemm plus
// the number of moduli; default precision policy).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "oz2.h"
#include "oz2_internal.h"

using namespace oz2;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }

// a run of at most this many k-positions keeps |INT32 accumulator| <= 2^31 - 2^22
// (Arc page Sec. 2.3 step 3: exact while k 128^2 < 2^31); a multiple of kPadK
constexpr int64_t kMaxRunK = 130816;
static_assert(kMaxRunK % kPadK == 0, "runs must be whole pairs of GEMM k steps");

struct Layout {
    int sets = 1, outs = 1, s = 0, NL = 0, t = 0, chunks = 1;
    int64_t m = 0, n = 0, k = 0, mp = 0, np = 0, kp = 0;
    size_t off_amaxA = 0, off_amaxB = 0, off_pa = 0, off_pb = 0, off_res = 0, off_chat = 0;
    size_t bytes_pa = 0, bytes_pb = 0, bytes_res = 0, bytes_chat = 0, total = 0;
    bool valid = false;
    bool prepared = false;  // operands came from oz2_operand objects (not in the workspace)
};

}  // namespace

struct oz2_context {
    int device = 0;
    hipStream_t stream = nullptr;
    void* ws = nullptr;
    size_t ws_size = 0;
    size_t mem_limit = 0;
    int timing = 0;
    int debug = 0;
    bool timed = false;
    hipEvent_t ev[5] = {};
    hipEvent_t order_ev = nullptr;  // orders a stream switch after the old stream's work
    Layout last;
    void* last_ws = nullptr;        // the workspace `last` refers to
    // the fixed device scratch (oz2_dgemm_noalloc), its address on this
    // handle's device; noalloc is set for the duration of such a call
    void* scratch = nullptr;
    bool noalloc = false;
    // blocking of the last product: block rows and columns of C, and which
    // operand's encoded block was kept across the other's blocks
    int64_t tile_mb = 0, tile_nb = 0;
    int tile_held = OZ2_TILE_UNTILED;
    // which kernels run a persistent chain (OZ2_CHAIN_KERNEL_*)
    int chain_kernel = OZ2_CHAIN_KERNEL_AUTO;
    int chain_crt = 1;  // base extension in the CRT form where the plan allows it
};

// a scanned and encoded operand kept on the device between products
struct oz2_operand {
    int device = 0;
    bool cplx = false, is_a = true, ext = false;
    char trans = 'N';
    int64_t rows = 0, k = 0, rows_pad = 0, kp = 0;
    int s = 0, t = 0, sets = 1;
    void* mem = nullptr;
    uint64_t* amax = nullptr;  // [rows_pad] bit patterns of the row (column) maxima
    int8_t* planes = nullptr;  // [sets][s][kp/64][rows_pad][64]
};

// a planned persistent tensor-mode chain: the kernels' tables and the
// operator residues on the device, in the layouts of both chain kernels
// (the LDS kernel's only for n <= 16)
struct oz2_chain_plan {
    ChainParams params;        // b, g, Qd and device pointers; X, Y, batch per call
    void* mem = nullptr;       // device: ChainTables, LDS-kernel residues, fexp, HBM-kernel residues
    int np = 0, ap = 0;        // n rounded up to 8 (plane padding) and to 16 (operator rows)
    int ncp = 0;               // pairs of 32-byte MFMA k chunks covering np
    const int* fexp = nullptr;     // device [3][np] row exponents left pending on each direction
    const ChainDropTable* drop = nullptr;  // device [d] drop weights of each product (HBM kernels)
    const ChainCrtTable* crt = nullptr;    // device [d] CRT base-extension tables (used where params.crt)
    const int8_t* hops = nullptr;  // device [d][s][ap / 16][ncp][64][16] operator residues of the HBM kernels
};

namespace {

bool valid_op(char c) {
    return c == 'N' || c == 'n' || c == 'T' || c == 't' || c == 'C' || c == 'c';
}
bool is_trans(char c) { return !(c == 'N' || c == 'n'); }
bool is_conj(char c) { return c == 'C' || c == 'c'; }

// the workspace of the call in progress: the handle's own, or the fixed
// scratch during oz2_dgemm_noalloc
char* workspace(const oz2_context* h) { return (char*)(h->noalloc ? h->scratch : h->ws); }

int ensure_workspace(oz2_context* h, size_t bytes) {
    if (h->noalloc) return bytes <= kScratchBytes ? OZ2_STATUS_SUCCESS : OZ2_STATUS_WORKSPACE_LIMIT;
    if (bytes <= h->ws_size) return OZ2_STATUS_SUCCESS;
    size_t cap = h->mem_limit;
    if (cap == 0) {
        size_t free_b = 0, total_b = 0;
        if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) return OZ2_STATUS_HIP_ERROR;
        cap = free_b + h->ws_size;
    }
    if (bytes > cap) return OZ2_STATUS_WORKSPACE_LIMIT;
    if (h->ws) {
        if (hipStreamSynchronize(h->stream) != hipSuccess) return OZ2_STATUS_HIP_ERROR;
        (void)hipFree(h->ws);
        h->ws = nullptr;
        h->ws_size = 0;
    }
    if (hipMalloc(&h->ws, bytes) != hipSuccess) {
        h->ws = nullptr;
        (void)hipGetLastError();
        return OZ2_STATUS_ALLOC_FAILED;
    }
    h->ws_size = bytes;
    return OZ2_STATUS_SUCCESS;
}

#define OZ2_LAUNCH(expr)                                  \
    do {                                                  \
        if ((expr) != hipSuccess) return OZ2_STATUS_HIP_ERROR; \
    } while (0)

void fill_mod_tables(const ModuliPlan& pl, EncodeParams* E, bool ext) {
    for (int q = 0; q < pl.s; ++q) {
        E->mod[q] = (uint32_t)pl.mod[q];
        E->K[q] = ext ? pl.Kext[q] : pl.Kstd[q];
        E->frcp[q] = pl.frcp[q];
        E->foffb[q] = pl.foffb[q];
        for (int l = 0; l < kExtWords; ++l) E->c[q][l] = pl.c4[q][l];
    }
}

template <class P>
void fill_crt_tables(const ModuliPlan& pl, P* R) {
    for (int u = 0; u < (pl.s + 1) / 2; ++u) R->Y2[u] = pl.Y2[u];  // high half 0 past the last modulus
    for (int u = 0; u < (pl.s + 1) / 2; ++u)
        for (int l = 0; l < 2 * pl.NL; ++l) R->W2[u][l] = pl.W2[u][l];
    for (int l = 0; l < 2 * pl.NL; ++l) R->M16[l] = pl.M16[l];
}

// the fused short-k path applies when k fits one wavefront's registers and
// one of the output dimensions is small, so that the operand tile re-encoded
// per output tile is the small one
bool small_path(const oz2_context* h, int64_t m, int64_t n, int64_t k) {
    return !h->debug && k >= 1 && k <= kSmallMaxK && (m <= 64 || n <= 64);
}

int small_impl(oz2_context* h, const ModuliPlan& pl, int t, char transa, char transb, int64_t m,
               int64_t n, int64_t k, double alpha, const double* A, int64_t lda, int64_t strideA,
               const double* B, int64_t ldb, int64_t strideB, double beta, double* C, int64_t ldc,
               int64_t strideC, int64_t batch, int s) {
    if (pl.NL <= 4 && t > kMaxStdT) return OZ2_STATUS_INTERNAL;
    SmallParams P{};
    P.A = A; P.lda = lda; P.strideA = strideA;
    P.B = B; P.ldb = ldb; P.strideB = strideB;
    P.C = C; P.ldc = ldc; P.strideC = strideC;
    P.m = m; P.n = n; P.k = k; P.batch = batch;
    P.transa = is_trans(transa) ? 1 : 0;
    P.transb = is_trans(transb) ? 1 : 0;
    P.alpha = alpha; P.beta = beta;
    P.t = t; P.s = s;
    const bool ext = pl.NL >= 5;
    for (int q = 0; q < s; ++q) {
        P.mod[q] = (uint32_t)pl.mod[q];
        P.K[q] = ext ? pl.Kext[q] : pl.Kstd[q];
        P.rcp[q] = pl.drcp[q];
        P.frcp[q] = pl.frcp[q];
        P.foffb[q] = pl.foffb[q];
        for (int l = 0; l < kExtWords; ++l) P.c[q][l] = pl.c4[q][l];
    }
    fill_crt_tables(pl, &P);
    hipStream_t stm = h->stream;
    h->last.valid = false;
    if (h->timing)
        for (int e = 0; e < 3; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], stm));
    OZ2_LAUNCH(launch_small_gemm(P, pl.NL, beta != 0.0, stm));
    if (h->timing) {
        OZ2_LAUNCH(hipEventRecord(h->ev[3], stm));
        OZ2_LAUNCH(hipEventRecord(h->ev[4], stm));
        h->timed = true;
    }
    return OZ2_STATUS_SUCCESS;
}

// workspace layout of the four-phase path for one m x n x k product
Layout plan_layout(const oz2_context* h, bool cplx, int s, const ModuliPlan& plan, int t, int64_t m, int64_t n,
                   int64_t k, bool with_operands = true) {
    const ModuliPlan* pl = &plan;
    Layout L;
    L.sets = cplx ? 3 : 1;
    L.outs = cplx ? 2 : 1;
    L.s = s;
    L.NL = pl->NL;
    L.t = t;
    L.m = m; L.n = n; L.k = k;
    L.mp = round_up(m, kPadM);
    L.np = round_up(n, kPadM);
    L.kp = round_up(k, kPadK);
    size_t off = 0;
    if (with_operands) {
        L.off_amaxA = off; off = align_up(off + 8 * (size_t)L.mp);
        L.off_amaxB = off; off = align_up(off + 8 * (size_t)L.np);
        L.bytes_pa = (size_t)L.sets * s * L.mp * L.kp;
        L.off_pa = off; off = align_up(off + L.bytes_pa);
        L.bytes_pb = (size_t)L.sets * s * L.np * L.kp;
        L.off_pb = off; off = align_up(off + L.bytes_pb);
    } else {
        L.prepared = true;
    }
    L.chunks = (int)((L.kp + kMaxRunK - 1) / kMaxRunK);
    L.bytes_res = (size_t)L.chunks * L.outs * s * L.n * L.mp;
    L.off_res = off; off = align_up(off + L.bytes_res);
    L.bytes_chat = h->debug ? (size_t)L.outs * L.n * L.mp * L.NL * 4 : 0;
    L.off_chat = off; off = align_up(off + L.bytes_chat);
    L.total = off;
    return L;
}

// whether a workspace of `bytes` is allowed: under the memory limit when one
// is set, else within the free device memory (plus the current workspace);
// *cap receives the bound
bool fits(oz2_context* h, size_t bytes, size_t* cap) {
    if (h->noalloc) {
        *cap = kScratchBytes;
        return bytes <= kScratchBytes;
    }
    if (h->mem_limit) {
        *cap = h->mem_limit;
        return bytes <= h->mem_limit;
    }
    if (bytes <= h->ws_size) {
        *cap = h->ws_size;
        return true;
    }
    size_t free_b = 0, total_b = 0;
    if (hipMemGetInfo(&free_b, &total_b) != hipSuccess) {
        (void)hipGetLastError();
        *cap = h->ws_size;
        return false;
    }
    *cap = free_b + h->ws_size;
    return bytes <= *cap;
}

// phase 1 for one operand: the row maxima of op(A) (is_a) or the column
// maxima of op(B).  Row i of op(A) is column i of A when transposed; column
// j of op(B) is column j of B when not.
bool operand_contiguous(bool is_a, char trans) { return is_a ? is_trans(trans) : !is_trans(trans); }

int scan_operand(oz2_context* h, bool cplx, bool is_a, char trans, int64_t rows, int64_t k, const double* X,
                 int64_t ld, uint64_t* amax, int64_t rows_pad) {
    hipStream_t stm = h->stream;
    OZ2_LAUNCH(launch_fill_u64(amax, rows_pad, 0, stm));
    ScanParams S{};
    S.X = X; S.ld = ld; S.nvec = rows; S.k = k; S.amax = amax;
    const int64_t vb = (rows + 255) / 256;
    int64_t chunks = 2048 / (vb > 0 ? vb : 1);
    if (chunks < 1) chunks = 1;
    S.pchunk = (k + chunks - 1) / chunks;
    OZ2_LAUNCH(launch_scan(S, operand_contiguous(is_a, trans), cplx, stm));
    return OZ2_STATUS_SUCCESS;
}

// phase 2 for one operand: integerize with the scan's exponents and write the
// residue planes [sets][s][kp/64][rows_pad][64]
int encode_operand(oz2_context* h, bool cplx, bool is_a, char trans, int64_t rows, int64_t k, const double* X,
                   int64_t ld, int s, const ModuliPlan* pl, int t, bool ext, const uint64_t* amax,
                   int8_t* planes, int64_t rows_pad, int64_t kp) {
    EncodeParams E{};
    fill_mod_tables(*pl, &E, ext);
    E.t = t; E.s = s;
    E.X = X; E.ld = ld; E.nvec = rows; E.k = k; E.vpad = rows_pad; E.kpad = kp;
    E.set_stride = (int64_t)s * rows_pad * kp;
    E.amax = amax; E.planes = planes; E.conj = cplx && is_conj(trans);
    OZ2_LAUNCH(launch_encode(E, operand_contiguous(is_a, trans), cplx, ext, h->stream));
    return OZ2_STATUS_SUCCESS;
}

// phases 3 and 4: s exact INT8 products reduced mod m_t on chip (one launch
// per k run of at most kMaxRunK positions), then CRT, rounding, scale back
// and alpha/beta.  L gives the padded sizes and the workspace offsets of the
// product residues (and c_hat).
int product(oz2_context* h, bool cplx, const Layout& L, const int8_t* pa, int64_t a_rows, const uint64_t* amaxA,
            const int8_t* pb, int64_t b_rows, const uint64_t* amaxB, const double alpha[2], const double beta[2],
            double* C, int64_t ldc, const ModuliPlan* pl, bool record) {
    const bool beta_zero = beta[0] == 0.0 && beta[1] == 0.0;
    const int s = L.s;
    char* ws = workspace(h);
    uint8_t* res = (uint8_t*)(ws + L.off_res);
    uint32_t* chat = h->debug ? (uint32_t*)(ws + L.off_chat) : nullptr;
    hipStream_t stm = h->stream;
    const int64_t chunk_stride = (int64_t)L.outs * s * L.n * L.mp;
    {
        GemmParams G{};
        G.A = pa; G.B = pb;
        G.mp = L.mp; G.np = L.np; G.kp = L.kp; G.n = L.n;
        G.a_rows = a_rows; G.b_rows = b_rows;
        G.a_set_stride = (int64_t)s * a_rows * L.kp;
        G.b_set_stride = (int64_t)s * b_rows * L.kp;
        G.c_set_stride = (int64_t)s * L.n * L.mp;
        G.s = s;
        for (int q = 0; q < s; ++q) {
            G.mod[q] = (uint32_t)pl->mod[q];
            G.rcp[q] = pl->drcp[q];
        }
        for (int c = 0; c < L.chunks; ++c) {
            G.C = res + c * chunk_stride;
            G.k_begin = c * kMaxRunK;
            const int64_t k_end = (c + 1) * kMaxRunK < L.kp ? (c + 1) * kMaxRunK : L.kp;
            G.k_steps = (int)((k_end - G.k_begin) / kGemmStepK);
            OZ2_LAUNCH(launch_residue_gemm(G, cplx, stm));
        }
    }
    if (record) OZ2_LAUNCH(hipEventRecord(h->ev[3], stm));
    {
        ReconParams R{};
        fill_crt_tables(*pl, &R);
        R.R = res; R.mp = L.mp; R.m = L.m; R.n = L.n;
        R.r_set_stride = (int64_t)s * L.n * L.mp;
        R.r_chunk_stride = chunk_stride;
        R.chunks = L.chunks;
        for (int q = 0; q < s; ++q) R.mod[q] = (uint32_t)pl->mod[q];
        R.amaxA = amaxA; R.amaxB = amaxB;
        R.C = C; R.ldc = ldc;
        R.alpha[0] = alpha[0]; R.alpha[1] = alpha[1];
        R.beta[0] = beta[0]; R.beta[1] = beta[1];
        R.t = L.t; R.s = s; R.chat = chat;
        OZ2_LAUNCH(launch_reconstruct(R, pl->NL, cplx, !beta_zero, stm));
    }
    if (record) {
        OZ2_LAUNCH(hipEventRecord(h->ev[4], stm));
        h->timed = true;
    }
    return OZ2_STATUS_SUCCESS;
}

// the four phases for one block (the whole product when untiled); record:
// phase events of this call
int core(oz2_context* h, bool cplx, char transa, char transb, int64_t m, int64_t n, int64_t k,
         const double alpha[2], const double* A, int64_t lda, const double* B, int64_t ldb,
         const double beta[2], double* C, int64_t ldc, int s, const ModuliPlan* pl, int t, bool ext,
         bool record) {
    Layout L = plan_layout(h, cplx, s, *pl, t, m, n, k);
    int st = ensure_workspace(h, L.total);
    if (st) return st;
    char* ws = workspace(h);
    uint64_t* amaxA = (uint64_t*)(ws + L.off_amaxA);
    uint64_t* amaxB = (uint64_t*)(ws + L.off_amaxB);
    int8_t* pa = (int8_t*)(ws + L.off_pa);
    int8_t* pb = (int8_t*)(ws + L.off_pb);
    hipStream_t stm = h->stream;
    if (record) OZ2_LAUNCH(hipEventRecord(h->ev[0], stm));
    if ((st = scan_operand(h, cplx, true, transa, m, k, A, lda, amaxA, L.mp))) return st;
    if ((st = scan_operand(h, cplx, false, transb, n, k, B, ldb, amaxB, L.np))) return st;
    if (record) OZ2_LAUNCH(hipEventRecord(h->ev[1], stm));
    if ((st = encode_operand(h, cplx, true, transa, m, k, A, lda, s, pl, t, ext, amaxA, pa, L.mp, L.kp))) return st;
    if ((st = encode_operand(h, cplx, false, transb, n, k, B, ldb, s, pl, t, ext, amaxB, pb, L.np, L.kp)))
        return st;
    if (record) OZ2_LAUNCH(hipEventRecord(h->ev[2], stm));
    st = product(h, cplx, L, pa, L.mp, amaxA, pb, L.np, amaxB, alpha, beta, C, ldc, pl, record);
    if (st) return st;
    L.valid = true;
    h->last = L;
    h->last_ws = ws;
    return OZ2_STATUS_SUCCESS;
}

// ------------------------------------------------------------------------
// Memory-aware tiling (Arc page Sec. 6, memory-aware tiling, and Table 16's
// power-of-two tiles; Sec. 9.2 for the shape of the cost model).  When the
// workspace of the whole product exceeds the cap, C is computed in blocks of
// mb x nb entries, each with all of k, so that every block has the full row
// and column exponents and the result is bitwise that of the untiled call.
// One operand's encoded block is kept while the other's blocks go by, so
// that operand is scanned and encoded once in total.
// ------------------------------------------------------------------------
struct TilePlan {
    int64_t mb = 0, nb = 0;
    bool hold_a = true;  // block rows outer (op(A) block kept); else block columns outer
    double cost_us = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Time of one block's residue products (us): the per-block model fitted to
// measured DGEMMs on this GPU (N = 1024 .. 8192, s = 8, 16, 24), about 19 us
// fixed plus 0.62 us per 64-position k step for a 256 x 256 tile with one
// block per CU, over waves of 256 CUs; for the 128 x 128 tile (small grids
// or short k) about 2.5 us per step per wave of 1024 blocks.  Complex
// products run three k-loops per block.
double gemm_block_us(int64_t mb, int64_t nb, int64_t kp, int s, bool cplx) {
    const double steps = (double)kp / kGemmStepK;
    const int64_t mp = round_up(mb, kPadM), np = round_up(nb, kPadM);
    const double passes = cplx ? 3.0 : 1.0;
    const int64_t big = (mp / 256) * (np / 256) * s;
    if (big >= 512 && kp > 512) return (double)ceil_div(big, 256) * (19.0 + 0.62 * steps * passes);
    const int64_t small = (mp / 128) * (np / 128) * s;
    return (double)ceil_div(small, 1024) * (0.16 + 2.53 * steps * passes);
}

// Modelled time of the whole product under a blocking (us): residue products
// of every block, the scans and encodes (each operand block read once and
// its planes written once) and the reconstructions (the same for every
// blocking) at the fitted 4.6 TB/s, and about 7 us per kernel launch.
double tile_cost_us(bool cplx, int s, int64_t m, int64_t n, int64_t k, int64_t mb, int64_t nb, bool hold_a,
                    bool prepared) {
    const int64_t kp = round_up(k, kPadK);
    const int64_t br = ceil_div(m, mb), bc = ceil_div(n, nb);
    const int64_t mlast = m - (br - 1) * mb, nlast = n - (bc - 1) * nb;
    double gemm = 0;
    gemm += (double)(br - 1) * (bc - 1) * gemm_block_us(mb, nb, kp, s, cplx);
    gemm += (double)(br - 1) * gemm_block_us(mb, nlast, kp, s, cplx);
    gemm += (double)(bc - 1) * gemm_block_us(mlast, nb, kp, s, cplx);
    gemm += gemm_block_us(mlast, nlast, kp, s, cplx);
    const double w = cplx ? 2.0 : 1.0, sets = cplx ? 3.0 : 1.0, outs = cplx ? 2.0 : 1.0;
    const double per_elem = 16.0 * w + sets * s;  // scan reads 8w, encode reads 8w and writes sets * s
    double enc_bytes = 0;
    int64_t launches = br * bc * (kp > 130816 ? 3 : 2);
    if (!prepared) {
        const double a_times = hold_a ? 1.0 : (double)bc, b_times = hold_a ? (double)br : 1.0;
        enc_bytes = per_elem * ((double)m * k * a_times + (double)n * k * b_times);
        launches += 4 * (hold_a ? br + br * bc : bc + br * bc);
    }
    const double crt_bytes = (outs * s + 8.0 * w) * (double)m * n;
    return gemm + enc_bytes / 4.6e6 + crt_bytes / 4.6e6 + 7.0 * (double)launches;
}

// Cheapest blocking whose workspace fits `cap`: block sides are the whole
// dimension or a power-of-two multiple of 256 below it, non-square allowed,
// with either operand held.  Returns false when no 256 x 256 block fits.
bool choose_tiles(const oz2_context* h, bool cplx, int s, const ModuliPlan& pl, int t, int64_t m, int64_t n,
                  int64_t k, size_t cap, bool prepared, TilePlan* best) {
    int64_t cm[40], cn[40];
    int nm = 0, nn = 0;
    for (int64_t T = kPadM; T < m && nm < 39; T *= 2) cm[nm++] = T;
    cm[nm++] = m;
    for (int64_t T = kPadM; T < n && nn < 39; T *= 2) cn[nn++] = T;
    cn[nn++] = n;
    bool found = false;
    for (int a = 0; a < nm; ++a) {
        for (int b = 0; b < nn; ++b) {
            const int64_t mb = cm[a], nb = cn[b];
            if (plan_layout(h, cplx, s, pl, t, mb, nb, k, !prepared).total > cap) continue;
            for (int held = 0; held < (prepared ? 1 : 2); ++held) {
                const double c = tile_cost_us(cplx, s, m, n, k, mb, nb, held == 0, prepared);
                // ties go to the larger block (fewer launches)
                if (!found || c < best->cost_us || (c == best->cost_us && mb * nb > best->mb * best->nb)) {
                    best->mb = mb; best->nb = nb; best->hold_a = held == 0; best->cost_us = c;
                    found = true;
                }
            }
        }
    }
    return found;
}

// the four phases over the blocks of a plan; the workspace is laid out for
// the largest block, and each block's planes use its own padded sizes
int tiled_impl(oz2_context* h, bool cplx, char transa, char transb, int64_t m, int64_t n, int64_t k,
               const double alpha[2], const double* A, int64_t lda, const double* B, int64_t ldb,
               const double beta[2], double* C, int64_t ldc, int s, const ModuliPlan* pl, int t, bool ext,
               const TilePlan& tp) {
    const int64_t mb = tp.mb < m ? tp.mb : m, nb = tp.nb < n ? tp.nb : n;
    const Layout Lmax = plan_layout(h, cplx, s, *pl, t, mb, nb, k);
    int st = ensure_workspace(h, Lmax.total);
    if (st) return st;
    char* ws = workspace(h);
    uint64_t* amaxA = (uint64_t*)(ws + Lmax.off_amaxA);
    uint64_t* amaxB = (uint64_t*)(ws + Lmax.off_amaxB);
    int8_t* pa = (int8_t*)(ws + Lmax.off_pa);
    int8_t* pb = (int8_t*)(ws + Lmax.off_pb);
    const int64_t w = cplx ? 2 : 1;  // doubles per element
    hipStream_t stm = h->stream;
    const bool rec = h->timing != 0;
    if (rec)
        for (int e = 0; e < 3; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], stm));
    auto encode_a = [&](int64_t i0, int64_t rows) -> int {
        const double* Ab = A + w * (is_trans(transa) ? i0 * lda : i0);
        const int64_t rp = round_up(rows, kPadM);
        int r = scan_operand(h, cplx, true, transa, rows, k, Ab, lda, amaxA, rp);
        if (!r) r = encode_operand(h, cplx, true, transa, rows, k, Ab, lda, s, pl, t, ext, amaxA, pa, rp, Lmax.kp);
        return r;
    };
    auto encode_b = [&](int64_t j0, int64_t cols) -> int {
        const double* Bb = B + w * (is_trans(transb) ? j0 : j0 * ldb);
        const int64_t cp = round_up(cols, kPadM);
        int r = scan_operand(h, cplx, false, transb, cols, k, Bb, ldb, amaxB, cp);
        if (!r) r = encode_operand(h, cplx, false, transb, cols, k, Bb, ldb, s, pl, t, ext, amaxB, pb, cp, Lmax.kp);
        return r;
    };
    auto block = [&](int64_t i0, int64_t rows, int64_t j0, int64_t cols) -> int {
        Layout Lb = plan_layout(h, cplx, s, *pl, t, rows, cols, k);
        Lb.off_amaxA = Lmax.off_amaxA; Lb.off_amaxB = Lmax.off_amaxB;
        Lb.off_pa = Lmax.off_pa; Lb.off_pb = Lmax.off_pb;
        Lb.off_res = Lmax.off_res; Lb.off_chat = Lmax.off_chat;
        double* Cb = C + w * (i0 + j0 * ldc);
        const int r = product(h, cplx, Lb, pa, Lb.mp, amaxA, pb, Lb.np, amaxB, alpha, beta, Cb, ldc, pl, false);
        if (!r) {
            Lb.valid = true;
            h->last = Lb;
            h->last_ws = ws;
        }
        return r;
    };
    if (tp.hold_a) {
        for (int64_t i0 = 0; i0 < m; i0 += mb) {
            const int64_t rows = m - i0 < mb ? m - i0 : mb;
            if ((st = encode_a(i0, rows))) return st;
            for (int64_t j0 = 0; j0 < n; j0 += nb) {
                const int64_t cols = n - j0 < nb ? n - j0 : nb;
                if ((st = encode_b(j0, cols))) return st;
                if ((st = block(i0, rows, j0, cols))) return st;
            }
        }
    } else {
        for (int64_t j0 = 0; j0 < n; j0 += nb) {
            const int64_t cols = n - j0 < nb ? n - j0 : nb;
            if ((st = encode_b(j0, cols))) return st;
            for (int64_t i0 = 0; i0 < m; i0 += mb) {
                const int64_t rows = m - i0 < mb ? m - i0 : mb;
                if ((st = encode_a(i0, rows))) return st;
                if ((st = block(i0, rows, j0, cols))) return st;
            }
        }
    }
    if (rec) {
        for (int e = 3; e < 5; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], stm));
        h->timed = true;
    }
    h->tile_mb = mb;
    h->tile_nb = nb;
    h->tile_held = tp.hold_a ? OZ2_TILE_HOLD_A : OZ2_TILE_HOLD_B;
    return OZ2_STATUS_SUCCESS;
}

int gemm_impl(oz2_context* h, bool cplx, char transa, char transb, int64_t m, int64_t n,
              int64_t k, const double alpha[2], const double* A, int64_t lda, const double* B,
              int64_t ldb, const double beta[2], double* C, int64_t ldc, int s) {
    if (!h) return -1;
    if (!valid_op(transa)) return -2;
    if (!valid_op(transb)) return -3;
    if (m < 0) return -4;
    if (n < 0) return -5;
    if (k < 0) return -6;
    const int64_t rows_a = is_trans(transa) ? k : m;
    const int64_t rows_b = is_trans(transb) ? n : k;
    if (lda < (rows_a > 1 ? rows_a : 1)) return -9;
    if (ldb < (rows_b > 1 ? rows_b : 1)) return -11;
    if (ldc < (m > 1 ? m : 1)) return -14;
    if (s < kMinS || s > kMaxS) return -15;
    if (m == 0 || n == 0) return OZ2_STATUS_SUCCESS;
    if (!C) return -13;
    const bool alpha_zero = alpha[0] == 0.0 && alpha[1] == 0.0;
    h->timed = false;
    if (alpha_zero || k == 0) {
        OZ2_LAUNCH(launch_scale_c(C, m, n, ldc, beta, cplx, h->stream));
        return OZ2_STATUS_SUCCESS;
    }
    if (!A) return -8;
    if (!B) return -10;

    const ModuliPlan* pl = moduli_plan(s);
    if (!pl) return OZ2_STATUS_INTERNAL;
    const int t = scaling_width(*pl, k, cplx);
    if (t < 1) return OZ2_STATUS_RANGE;
    const bool ext = t > kMaxStdT;
    if (!cplx && small_path(h, m, n, k)) {
        h->tile_mb = m;
        h->tile_nb = n;
        h->tile_held = OZ2_TILE_UNTILED;
        return small_impl(h, *pl, t, transa, transb, m, n, k, alpha[0], A, lda, 0, B, ldb, 0, beta[0], C,
                          ldc, 0, 1, s);
    }

    // memory-aware tiling when the whole product's workspace exceeds the cap
    const Layout full = plan_layout(h, cplx, s, *pl, t, m, n, k);
    size_t cap = 0;
    if (!fits(h, full.total, &cap)) {
        TilePlan tp;
        if (!choose_tiles(h, cplx, s, *pl, t, m, n, k, cap, false, &tp)) return OZ2_STATUS_WORKSPACE_LIMIT;
        return tiled_impl(h, cplx, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s, pl, t, ext,
                          tp);
    }
    h->tile_mb = m;
    h->tile_nb = n;
    h->tile_held = OZ2_TILE_UNTILED;
    return core(h, cplx, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s, pl, t, ext,
                h->timing != 0);
}

}  // namespace

extern "C" {

int oz2_create(oz2_handle_t* out) {
    if (!out) return -1;
    *out = nullptr;
    oz2_context* h = new (std::nothrow) oz2_context();
    if (!h) return OZ2_STATUS_ALLOC_FAILED;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return OZ2_STATUS_HIP_ERROR;
    }
    for (auto& e : h->ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            delete h;
            return OZ2_STATUS_HIP_ERROR;
        }
    }
    if (hipEventCreateWithFlags(&h->order_ev, hipEventDisableTiming) != hipSuccess) {
        delete h;
        return OZ2_STATUS_HIP_ERROR;
    }
    // the fixed scratch's address on this device, taken once per device here
    // at set-up; without it only oz2_dgemm_noalloc fails (HIP_ERROR)
    if (scratch_address(h->device, &h->scratch) != OZ2_STATUS_SUCCESS) h->scratch = nullptr;
    *out = h;
    return OZ2_STATUS_SUCCESS;
}

int oz2_destroy(oz2_handle_t h) {
    if (!h) return -1;
    (void)hipStreamSynchronize(h->stream);
    if (h->ws) (void)hipFree(h->ws);
    for (auto& e : h->ev)
        if (e) (void)hipEventDestroy(e);
    if (h->order_ev) (void)hipEventDestroy(h->order_ev);
    delete h;
    return OZ2_STATUS_SUCCESS;
}

int oz2_set_stream(oz2_handle_t h, void* stream) {
    if (!h) return -1;
    hipStream_t next = (hipStream_t)stream;
    if (next == h->stream) return OZ2_STATUS_SUCCESS;
    // Every call on a handle uses the same workspace, so the new stream waits
    // for all work already queued on the old one.  Work on any earlier stream
    // is then ordered before the current stream's, and synchronising the
    // current stream (destroy, workspace growth) covers it too.
    if (hipEventRecord(h->order_ev, h->stream) != hipSuccess) return OZ2_STATUS_HIP_ERROR;
    if (hipStreamWaitEvent(next, h->order_ev, 0) != hipSuccess) return OZ2_STATUS_HIP_ERROR;
    h->stream = next;
    return OZ2_STATUS_SUCCESS;
}

int oz2_set_memory_limit(oz2_handle_t h, size_t bytes) {
    if (!h) return -1;
    h->mem_limit = bytes;
    return OZ2_STATUS_SUCCESS;
}

int oz2_get_workspace_size(oz2_handle_t h, size_t* bytes) {
    if (!h) return -1;
    if (!bytes) return -2;
    *bytes = h->ws_size;
    return OZ2_STATUS_SUCCESS;
}

int oz2_set_timing(oz2_handle_t h, int enable) {
    if (!h) return -1;
    h->timing = enable ? 1 : 0;
    return OZ2_STATUS_SUCCESS;
}

int oz2_get_phase_times(oz2_handle_t h, float ms[4]) {
    if (!h) return -1;
    if (!ms) return -2;
    if (!h->timed) {
        for (int i = 0; i < 4; ++i) ms[i] = 0.0f;
        return OZ2_STATUS_SUCCESS;
    }
    if (hipEventSynchronize(h->ev[4]) != hipSuccess) return OZ2_STATUS_HIP_ERROR;
    for (int i = 0; i < 4; ++i)
        if (hipEventElapsedTime(&ms[i], h->ev[i], h->ev[i + 1]) != hipSuccess)
            return OZ2_STATUS_HIP_ERROR;
    return OZ2_STATUS_SUCCESS;
}

int oz2_get_tile_plan(oz2_handle_t h, int64_t* mb, int64_t* nb, int* held) {
    if (!h) return -1;
    if (mb) *mb = h->tile_mb;
    if (nb) *nb = h->tile_nb;
    if (held) *held = h->tile_held;
    return OZ2_STATUS_SUCCESS;
}

int oz2_moduli_for_bits(int64_t k, int bits, int is_complex) {
    for (int s = kMinS; s <= kMaxS; ++s) {
        const ModuliPlan* pl = moduli_plan(s);
        if (!pl) continue;
        if (scaling_width(*pl, k, is_complex != 0) >= bits) return s;
    }
    return kMaxS;
}

int oz2_plan_info(int num_moduli, int64_t k, int is_complex, int32_t* moduli_out, int* t_out,
                  int* nl_out, double* log2M_out) {
    const ModuliPlan* pl = moduli_plan(num_moduli);
    if (!pl) return -1;
    if (moduli_out)
        for (int q = 0; q < kMaxS; ++q) moduli_out[q] = q < pl->s ? pl->mod[q] : 0;
    if (t_out) *t_out = scaling_width(*pl, k, is_complex != 0);
    if (nl_out) *nl_out = pl->NL;
    if (log2M_out) *log2M_out = pl->log2M;
    return OZ2_STATUS_SUCCESS;
}

int oz2_dgemm(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n, int64_t k,
              double alpha, const double* A, int64_t lda, const double* B, int64_t ldb,
              double beta, double* C, int64_t ldc, int num_moduli) {
    const double al[2] = {alpha, 0.0}, be[2] = {beta, 0.0};
    return gemm_impl(h, false, transa, transb, m, n, k, al, A, lda, B, ldb, be, C, ldc, num_moduli);
}

int oz2_dgemm_noalloc(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n, int64_t k,
                      double alpha, const double* A, int64_t lda, const double* B, int64_t ldb,
                      double beta, double* C, int64_t ldc, int num_moduli) {
    if (!h) return -1;
    if (!h->scratch) return OZ2_STATUS_HIP_ERROR;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != h->device) return OZ2_STATUS_HIP_ERROR;
    // the same path as oz2_dgemm with the fixed scratch as its workspace; a
    // product larger than the scratch runs in blocks of C that fit it
    struct Scope {
        oz2_context* h;
        explicit Scope(oz2_context* c) : h(c) { h->noalloc = true; }
        ~Scope() { h->noalloc = false; }
    } scope(h);
    const double al[2] = {alpha, 0.0}, be[2] = {beta, 0.0};
    const int st = gemm_impl(h, false, transa, transb, m, n, k, al, A, lda, B, ldb, be, C, ldc, num_moduli);
    return st == OZ2_STATUS_WORKSPACE_LIMIT ? OZ2_STATUS_SCRATCH_LIMIT : st;
}

int oz2_zgemm(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n, int64_t k,
              const double* alpha, const double* A, int64_t lda, const double* B, int64_t ldb,
              const double* beta, double* C, int64_t ldc, int num_moduli) {
    if (!alpha) return -7;
    if (!beta) return -12;
    return gemm_impl(h, true, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                     num_moduli);
}

int oz2_dgemm_strided_batched(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n,
                              int64_t k, double alpha, const double* A, int64_t lda,
                              int64_t strideA, const double* B, int64_t ldb, int64_t strideB,
                              double beta, double* C, int64_t ldc, int64_t strideC,
                              int64_t batch, int num_moduli) {
    if (!h) return -1;
    if (!valid_op(transa)) return -2;
    if (!valid_op(transb)) return -3;
    if (m < 0) return -4;
    if (n < 0) return -5;
    if (k < 0) return -6;
    const int64_t rows_a = is_trans(transa) ? k : m;
    const int64_t rows_b = is_trans(transb) ? n : k;
    if (lda < (rows_a > 1 ? rows_a : 1)) return -9;
    if (strideA < 0) return -10;
    if (ldb < (rows_b > 1 ? rows_b : 1)) return -12;
    if (strideB < 0) return -13;
    if (ldc < (m > 1 ? m : 1)) return -16;
    if (strideC < 0) return -17;
    if (batch < 0) return -18;
    if (num_moduli < kMinS || num_moduli > kMaxS) return -19;
    if (m == 0 || n == 0 || batch == 0) return OZ2_STATUS_SUCCESS;
    if (!C) return -15;
    if (alpha != 0.0 && k > 0 && small_path(h, m, n, k)) {
        if (!A) return -8;
        if (!B) return -11;
        const ModuliPlan* pl = moduli_plan(num_moduli);
        if (!pl) return OZ2_STATUS_INTERNAL;
        const int t = scaling_width(*pl, k, false);
        if (t < 1) return OZ2_STATUS_RANGE;
        h->timed = false;
        return small_impl(h, *pl, t, transa, transb, m, n, k, alpha, A, lda, strideA, B, ldb, strideB,
                          beta, C, ldc, strideC, batch, num_moduli);
    }
    // otherwise one call of the four-phase path per product
    const double al[2] = {alpha, 0.0}, be[2] = {beta, 0.0};
    for (int64_t b = 0; b < batch; ++b) {
        int st = gemm_impl(h, false, transa, transb, m, n, k, al, A ? A + b * strideA : nullptr,
                           lda, B ? B + b * strideB : nullptr, ldb, be,
                           C ? C + b * strideC : nullptr, ldc, num_moduli);
        if (st) return st;
    }
    return OZ2_STATUS_SUCCESS;
}

const char* oz2_status_string(int status) {
    switch (status) {
        case OZ2_STATUS_SUCCESS: return "success";
        case OZ2_STATUS_ALLOC_FAILED: return "device workspace allocation failed";
        case OZ2_STATUS_HIP_ERROR: return "HIP runtime error";
        case OZ2_STATUS_RANGE: return "no scaling width t >= 1 for this number of moduli and k";
        case OZ2_STATUS_WORKSPACE_LIMIT: return "workspace would exceed the memory limit";
        case OZ2_STATUS_NOT_SUPPORTED: return "not supported on this device";
        case OZ2_STATUS_SCRATCH_LIMIT:
            return "oz2_dgemm_noalloc: one 256 x 256 block of C with all of k does not fit the fixed 128 MiB scratch";
        case OZ2_STATUS_INTERNAL: return "internal error";
        default: return status < 0 ? "invalid argument" : "unknown status";
    }
}

int oz2_operand_create(oz2_handle_t h, char side, int is_complex, char trans, int64_t rows, int64_t k,
                       const double* X, int64_t ld, int num_moduli, oz2_operand_t* out) {
    if (!h) return -1;
    const bool is_a = side == 'A' || side == 'a';
    if (!is_a && !(side == 'B' || side == 'b')) return -2;
    if (!valid_op(trans)) return -4;
    if (rows < 1) return -5;
    if (k < 1) return -6;
    if (!X) return -7;
    // stored rows: A is m x k (N) or k x m (T/C); B is k x n (N) or n x k (T/C)
    const int64_t stored = is_a ? (is_trans(trans) ? k : rows) : (is_trans(trans) ? rows : k);
    if (ld < stored) return -8;
    if (num_moduli < kMinS || num_moduli > kMaxS) return -9;
    if (!out) return -10;
    *out = nullptr;
    const bool cplx = is_complex != 0;
    const ModuliPlan* pl = moduli_plan(num_moduli);
    if (!pl) return OZ2_STATUS_INTERNAL;
    const int t = scaling_width(*pl, k, cplx);
    if (t < 1) return OZ2_STATUS_RANGE;
    oz2_operand* op = new (std::nothrow) oz2_operand();
    if (!op) return OZ2_STATUS_ALLOC_FAILED;
    op->device = h->device;
    op->cplx = cplx; op->is_a = is_a; op->trans = trans;
    op->rows = rows; op->k = k;
    op->rows_pad = round_up(rows, kPadM);
    op->kp = round_up(k, kPadK);
    op->s = num_moduli; op->t = t; op->ext = t > kMaxStdT;
    op->sets = cplx ? 3 : 1;
    const size_t off_planes = align_up(8 * (size_t)op->rows_pad);
    const size_t bytes = off_planes + (size_t)op->sets * op->s * op->rows_pad * op->kp;
    if (hipMalloc(&op->mem, bytes) != hipSuccess) {
        (void)hipGetLastError();
        delete op;
        return OZ2_STATUS_ALLOC_FAILED;
    }
    op->amax = (uint64_t*)op->mem;
    op->planes = (int8_t*)op->mem + off_planes;
    int st = scan_operand(h, cplx, is_a, trans, rows, k, X, ld, op->amax, op->rows_pad);
    if (!st) st = encode_operand(h, cplx, is_a, trans, rows, k, X, ld, op->s, pl, t, op->ext, op->amax, op->planes,
                                 op->rows_pad, op->kp);
    if (st) {
        (void)hipStreamSynchronize(h->stream);
        (void)hipFree(op->mem);
        delete op;
        return st;
    }
    *out = op;
    return OZ2_STATUS_SUCCESS;
}

int oz2_operand_update(oz2_handle_t h, oz2_operand_t op, const double* X, int64_t ld) {
    if (!h) return -1;
    if (!op) return -2;
    if (!X) return -3;
    const int64_t stored = op->is_a ? (is_trans(op->trans) ? op->k : op->rows) : (is_trans(op->trans) ? op->rows : op->k);
    if (ld < stored) return -4;
    const ModuliPlan* pl = moduli_plan(op->s);
    if (!pl) return OZ2_STATUS_INTERNAL;
    int st = scan_operand(h, op->cplx, op->is_a, op->trans, op->rows, op->k, X, ld, op->amax, op->rows_pad);
    if (st) return st;
    return encode_operand(h, op->cplx, op->is_a, op->trans, op->rows, op->k, X, ld, op->s, pl, op->t, op->ext,
                          op->amax, op->planes, op->rows_pad, op->kp);
}

int oz2_operand_destroy(oz2_operand_t op) {
    if (!op) return -1;
    if (op->mem && hipFree(op->mem) != hipSuccess) {
        (void)hipGetLastError();
        delete op;
        return OZ2_STATUS_HIP_ERROR;
    }
    delete op;
    return OZ2_STATUS_SUCCESS;
}

int oz2_gemm_prepared(oz2_handle_t h, oz2_operand_t pa, oz2_operand_t pb, const double* alpha,
                      const double* beta, double* C, int64_t ldc) {
    if (!h) return -1;
    if (!pa || !pa->is_a) return -2;
    if (!pb || pb->is_a || pb->cplx != pa->cplx || pb->s != pa->s || pb->k != pa->k) return -3;
    if (!alpha) return -4;
    if (!beta) return -5;
    if (!C) return -6;
    const int64_t m = pa->rows, n = pb->rows, k = pa->k;
    if (ldc < m) return -7;
    const bool cplx = pa->cplx;
    const double al[2] = {alpha[0], cplx ? alpha[1] : 0.0};
    const double be[2] = {beta[0], cplx ? beta[1] : 0.0};
    h->timed = false;
    if (al[0] == 0.0 && al[1] == 0.0) {
        OZ2_LAUNCH(launch_scale_c(C, m, n, ldc, be, cplx, h->stream));
        return OZ2_STATUS_SUCCESS;
    }
    const ModuliPlan* pl = moduli_plan(pa->s);
    if (!pl) return OZ2_STATUS_INTERNAL;
    const int sm = pa->s;
    Layout L = plan_layout(h, cplx, sm, *pl, pa->t, m, n, k, false);
    size_t cap = 0;
    TilePlan tp;
    tp.mb = m;
    tp.nb = n;
    if (!fits(h, L.total, &cap)) {
        // blocks of C over sub-blocks of the prepared planes: a block's rows
        // start at a multiple of 256, so they are a run of whole GEMM tiles
        // inside every k-panel of the operand
        if (!choose_tiles(h, cplx, sm, *pl, pa->t, m, n, k, cap, true, &tp)) return OZ2_STATUS_WORKSPACE_LIMIT;
        L = plan_layout(h, cplx, sm, *pl, pa->t, tp.mb < m ? tp.mb : m, tp.nb < n ? tp.nb : n, k, false);
    }
    int st = ensure_workspace(h, L.total);
    if (st) return st;
    const int64_t mb = tp.mb < m ? tp.mb : m, nb = tp.nb < n ? tp.nb : n;
    const int64_t w = cplx ? 2 : 1;
    const bool rec = h->timing != 0;
    if (rec)
        for (int e = 0; e < 3; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], h->stream));
    const bool tiled = mb < m || nb < n;
    for (int64_t j0 = 0; j0 < n; j0 += nb) {
        const int64_t cols = n - j0 < nb ? n - j0 : nb;
        for (int64_t i0 = 0; i0 < m; i0 += mb) {
            const int64_t rows = m - i0 < mb ? m - i0 : mb;
            Layout Lb = plan_layout(h, cplx, sm, *pl, pa->t, rows, cols, k, false);
            Lb.off_res = L.off_res;
            Lb.off_chat = L.off_chat;
            st = product(h, cplx, Lb, pa->planes + i0 * kPanelK, pa->rows_pad, pa->amax + i0,
                         pb->planes + j0 * kPanelK, pb->rows_pad, pb->amax + j0, al, be, C + w * (i0 + j0 * ldc), ldc,
                         pl, rec && !tiled);
            if (st) return st;
            Lb.valid = true;
            h->last = Lb;
            h->last_ws = workspace(h);
        }
    }
    if (rec && tiled) {
        for (int e = 3; e < 5; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], h->stream));
        h->timed = true;
    }
    h->tile_mb = mb;
    h->tile_nb = nb;
    h->tile_held = tiled ? OZ2_TILE_PREPARED : OZ2_TILE_UNTILED;
    return OZ2_STATUS_SUCCESS;
}

int oz2_chain_plan_create(oz2_handle_t h, int64_t n, int depth, const double* const* ops, const int* modes,
                          int num_moduli, oz2_chain_plan_t* out) {
    if (!h) return -1;
    if (n < 1 || n > kChainMaxN) return -2;
    if (depth < 1 || depth > kChainMaxD) return -3;
    if (!ops) return -4;
    for (int i = 0; i < depth; ++i)
        if (!ops[i]) return -4;
    int dirs[kChainMaxD];
    for (int i = 0; i < depth; ++i) {
        dirs[i] = modes ? modes[i] - 1 : i % 3;  // 1-based directions in the interface
        if (dirs[i] < 0 || dirs[i] > 2) return -5;
    }
    if (num_moduli < kMinS || num_moduli > kChainMaxS) return -6;
    if (!out) return -7;
    *out = nullptr;
    const int nn = (int)n, s = num_moduli;
    oz2_chain_plan* plan = new (std::nothrow) oz2_chain_plan();
    if (!plan) return OZ2_STATUS_ALLOC_FAILED;
    plan->np = (nn + 7) & ~7;
    plan->ap = (plan->np + 15) & ~15;
    plan->ncp = (plan->np + 63) / 64;
    const int np = plan->np, ap = plan->ap, ncp = plan->ncp;
    const bool lds = nn <= kChainN;
    const size_t lds_bytes = lds ? (size_t)depth * kChainMaxS * kChainN * kChainN : 0;
    const size_t hops_bytes = (size_t)depth * s * ap * ncp * 64;
    const size_t off_lds = align_up(sizeof(ChainTables));
    const size_t off_fexp = align_up(off_lds + lds_bytes);
    const size_t off_hops = align_up(off_fexp + sizeof(int) * 3 * np);
    const size_t off_drop = align_up(off_hops + hops_bytes);
    const size_t off_crt = align_up(off_drop + sizeof(ChainDropTable) * depth);
    const size_t off_split = align_up(off_crt + sizeof(ChainCrtTable) * depth);  // the LDS kernel's reconstruction
    const size_t total = off_split + sizeof(ChainDropTable);
    std::vector<char> host;
    std::vector<int8_t> res;
    std::vector<int> fexp;
    int st = OZ2_STATUS_SUCCESS;
    try {
        host.assign(total, 0);
        res.resize((size_t)depth * s * nn * nn);
        fexp.resize((size_t)3 * nn);
    } catch (...) {
        st = OZ2_STATUS_ALLOC_FAILED;
    }
    if (!st) {
        ChainTables* tab = (ChainTables*)host.data();
        st = chain_plan(s, nn, depth, ops, dirs, &plan->params, tab, res.data(), fexp.data());
        if (st < 0) st = -4;  // a non-finite operator entry
    }
    if (!st) {
        // the LDS kernel: [d][kChainMaxS][16][16] by modulus index, zero padded
        int8_t* lo = (int8_t*)(host.data() + off_lds);
        int* fe = (int*)(host.data() + off_fexp);
        int8_t* ho = (int8_t*)(host.data() + off_hops);
        for (int i = 0; i < depth; ++i)
            for (int q = 0; q < s; ++q)
                for (int a = 0; a < nn; ++a)
                    for (int k = 0; k < nn; ++k) {
                        const int8_t v = res[(((size_t)i * s + q) * nn + a) * nn + k];
                        if (lds) lo[(((size_t)i * kChainMaxS + q) * kChainN + a) * kChainN + k] = v;
                        // fragment order, zero padded: row a = 16 at + r, byte k = 64 cp + 16 j + e at
                        // [i][q][at][cp][r + 16 j][e], the 16 bytes lane r + 16 j of a wavefront loads for
                        // the two MFMA k chunks of pair cp.  np = 8 (8 rows, 32 fibres per tile): row a
                        // at lanes a (k group 0) and a + 8 + 16 (k group 1), only the first chunk used
                        const size_t mq = (((size_t)i * s + q) * (ap / 16)) * ncp * 64;
                        if (np == 8) {
                            ho[(mq + a) * 16 + k] = v;
                            ho[(mq + a + 8 + 16) * 16 + k] = v;
                        } else {
                            const int at = a >> 4, r = a & 15, cp = k >> 6, j = (k >> 4) & 3, e = k & 15;
                            ho[(mq + ((size_t)at * ncp + cp) * 64 + r + 16 * j) * 16 + e] = v;
                        }
                    }
        for (int m = 0; m < 3; ++m)
            for (int a = 0; a < nn; ++a) fe[m * np + a] = fexp[(size_t)m * nn + a];
        ChainDropTable* dt = (ChainDropTable*)(host.data() + off_drop);
        const ChainTables& tabs = *(const ChainTables*)host.data();
        for (int i = 0; i + 1 < depth; ++i) chain_drop_table(tabs, plan->params.g[i], dt + i);
        // the last product's reconstruction: on the HBM kernels in blocks of
        // 4 slots when staged, 8 when direct; on the LDS kernel in blocks of 4
        chain_split_table(tabs, np >= kChainStagedNp ? kChainSplit : kChainSplitWide, dt + depth - 1);
        chain_split_table(tabs, kChainSplit, (ChainDropTable*)(host.data() + off_split));
        ChainCrtTable* ct = (ChainCrtTable*)(host.data() + off_crt);
        for (int i = 0; i < depth; ++i) chain_crt_table(tabs, i + 1 < depth ? plan->params.g[i] : 0, ct + i);
    }
    if (!st && hipMalloc(&plan->mem, total) != hipSuccess) {
        (void)hipGetLastError();
        plan->mem = nullptr;
        st = OZ2_STATUS_ALLOC_FAILED;
    }
    if (!st && hipMemcpy(plan->mem, host.data(), total, hipMemcpyHostToDevice) != hipSuccess) st = OZ2_STATUS_HIP_ERROR;
    if (st) {
        if (plan->mem) (void)hipFree(plan->mem);
        delete plan;
        return st;
    }
    plan->params.tab = (const float*)plan->mem;
    plan->params.ops = lds ? (const int8_t*)((char*)plan->mem + off_lds) : nullptr;
    plan->fexp = (const int*)((char*)plan->mem + off_fexp);
    plan->hops = (const int8_t*)((char*)plan->mem + off_hops);
    plan->drop = (const ChainDropTable*)((char*)plan->mem + off_drop);
    plan->crt = (const ChainCrtTable*)((char*)plan->mem + off_crt);
    plan->params.crts = plan->crt;
    plan->params.split = (const ChainDropTable*)((char*)plan->mem + off_split);
    plan->params.drops = plan->drop;
    {
        // the encode's residue constants of the chain's moduli (index q = slot - first);
        // moduli_plan(s) is non-null here: chain_plan above succeeded with this s
        const ModuliPlan* mpl = moduli_plan(s);
        ChainEncodeConsts& E = plan->params.enc;
        for (int q = 0; q < s; ++q) {
            E.K128[q] = mpl->Kstd[q] + 128u;
            for (int l = 0; l < kStdWords; ++l) E.c4[q][l] = mpl->c4[q][l];
            E.mod[q] = (float)mpl->mod[q];
            E.frcp[q] = mpl->frcp[q];
            E.foffb[q] = mpl->foffb[q];
        }
    }
    *out = plan;
    return OZ2_STATUS_SUCCESS;
}

int oz2_chain_plan_info(oz2_chain_plan_t plan, int* depth, int* b, int* g) {
    if (!plan) return -1;
    if (depth) *depth = plan->params.d;
    if (b) *b = plan->params.b;
    if (g)
        for (int i = 0; i < plan->params.d; ++i) g[i] = plan->params.g[i];
    return OZ2_STATUS_SUCCESS;
}

namespace {

// The chain on HBM-resident residue planes (oz2_chain_hbm.hip): per batch
// of tensors that fits the workspace, a scan, the encode, one kernel per
// product.  Phase times: scan, encode, the rescaling products, the last
// product with the reconstruction (with several batches: all in the third).
int chain_hbm(oz2_context* h, const oz2_chain_plan* plan, const double* X, double* Y, int64_t batch) {
    const ChainParams& C = plan->params;
    const int n = C.n, np = plan->np, s = C.s;
    const int64_t np3 = (int64_t)np * np * np, n3 = (int64_t)n * n * n;
    const size_t per_tensor = 2 * (size_t)s * np3 + sizeof(unsigned long long);
    const size_t fixed = 3 * 256;  // alignment of the three parts
    int64_t chunk = batch;
    size_t cap = 0;
    if (!fits(h, fixed + per_tensor * (size_t)batch, &cap)) {
        chunk = cap > fixed ? (int64_t)((cap - fixed) / per_tensor) : 0;
        if (chunk < 1) return OZ2_STATUS_WORKSPACE_LIMIT;
        // equal batches
        const int64_t parts = (batch + chunk - 1) / chunk;
        chunk = (batch + parts - 1) / parts;
    }
    const size_t off_b0 = align_up(sizeof(unsigned long long) * (size_t)chunk);
    const size_t off_b1 = align_up(off_b0 + (size_t)s * chunk * np3);
    const size_t bytes = off_b1 + (size_t)s * chunk * np3;
    const ChainEncodeConsts& E = plan->params.enc;
    int st = ensure_workspace(h, bytes);
    if (st) return st;
    char* ws = workspace(h);
    hipStream_t stm = h->stream;
    const bool timed = h->timing && chunk == batch;
    if (h->timing && !timed)
        for (int e = 0; e < 3; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], stm));
    for (int64_t t0 = 0; t0 < batch; t0 += chunk) {
        const int64_t nb = batch - t0 < chunk ? batch - t0 : chunk;
        ChainHbmParams P{};
        P.X = X + t0 * n3;
        P.Y = Y + t0 * n3;
        P.batch = nb;
        P.n = n;
        P.np = np;
        P.s = s;
        P.b = C.b;
        P.m0 = C.m0;
        for (int j = 0; j < 3; ++j) P.fin[j] = C.fin[j];
        P.Qd = C.Qd;
        P.tab = C.tab;
        P.fexp = plan->fexp;
        P.smax = (unsigned long long*)ws;
        P.pstride = nb * np3;
        int8_t* buf[2] = {(int8_t*)(ws + off_b0), (int8_t*)(ws + off_b1)};
        if (timed) OZ2_LAUNCH(hipEventRecord(h->ev[0], stm));
        OZ2_LAUNCH(launch_fill_u64((uint64_t*)P.smax, nb, 0, stm));
        OZ2_LAUNCH(launch_chain_scan(P, stm));
        if (timed) OZ2_LAUNCH(hipEventRecord(h->ev[1], stm));
        P.out = buf[0];
        OZ2_LAUNCH(launch_chain_encode(P, E, stm));
        if (timed) OZ2_LAUNCH(hipEventRecord(h->ev[2], stm));
        for (int i = 0; i < C.d; ++i) {
            const bool last = i == C.d - 1;
            if (last && timed) OZ2_LAUNCH(hipEventRecord(h->ev[3], stm));
            P.in = buf[i & 1];
            P.out = last ? nullptr : buf[(i + 1) & 1];
            P.g = C.g[i];
            P.kind = C.kind[i];
            P.ops = plan->hops + (size_t)i * s * plan->ap * plan->ncp * 64;
            P.drop = plan->drop + i;
            // the CRT base extension where the plan's bound allows it
            const bool crt = h->chain_crt && C.crt[i];
            P.crt = !last && C.g[i] > 0 && crt ? plan->crt + i : nullptr;
            OZ2_LAUNCH(launch_chain_step(P, last, stm));
        }
        if (timed) OZ2_LAUNCH(hipEventRecord(h->ev[4], stm));
    }
    if (h->timing && !timed) {
        OZ2_LAUNCH(hipEventRecord(h->ev[3], stm));
        OZ2_LAUNCH(hipEventRecord(h->ev[4], stm));
    }
    h->timed = h->timing != 0;
    return OZ2_STATUS_SUCCESS;
}

}  // namespace

int oz2_chain_rescale_be(oz2_handle_t h, oz2_chain_plan_t plan, const double* X, double* Y, int64_t batch) {
    if (!h) return -1;
    if (!plan) return -2;
    if (batch < 0 || batch > INT32_MAX) return -5;
    h->timed = false;
    if (batch == 0) return OZ2_STATUS_SUCCESS;
    if (!X) return -3;
    if (!Y) return -4;
    // automatic choice: the LDS kernel pads every tensor to 16^3, so it
    // serves 8 < n <= 16; smaller tensors (padded to 8^3) and larger ones
    // run on the HBM kernels
    const bool lds = h->chain_kernel == OZ2_CHAIN_KERNEL_LDS ||
                     (h->chain_kernel == OZ2_CHAIN_KERNEL_AUTO && plan->params.n > 8 && plan->params.n <= kChainN);
    if (lds && plan->params.n > kChainN) return OZ2_STATUS_NOT_SUPPORTED;
    h->last.valid = false;
    if (!lds) return chain_hbm(h, plan, X, Y, batch);
    ChainParams P = plan->params;
    P.X = X;
    P.Y = Y;
    P.batch = batch;
    if (!h->chain_crt) P.crts = nullptr;  // the mixed-radix form everywhere
    hipStream_t stm = h->stream;
    if (h->timing)
        for (int e = 0; e < 3; ++e) OZ2_LAUNCH(hipEventRecord(h->ev[e], stm));
    OZ2_LAUNCH(launch_chain(P, stm));
    if (h->timing) {
        OZ2_LAUNCH(hipEventRecord(h->ev[3], stm));
        OZ2_LAUNCH(hipEventRecord(h->ev[4], stm));
        h->timed = true;
    }
    return OZ2_STATUS_SUCCESS;
}

int oz2_set_chain_crt(oz2_handle_t h, int enable) {
    if (!h) return -1;
    if (enable != 0 && enable != 1) return -2;
    h->chain_crt = enable;
    return OZ2_STATUS_SUCCESS;
}

int oz2_set_chain_kernel(oz2_handle_t h, int kernel) {
    if (!h) return -1;
    if (kernel < OZ2_CHAIN_KERNEL_AUTO || kernel > OZ2_CHAIN_KERNEL_HBM) return -2;
    h->chain_kernel = kernel;
    return OZ2_STATUS_SUCCESS;
}

int oz2_chain_plan_destroy(oz2_chain_plan_t plan) {
    if (!plan) return -1;
    int st = OZ2_STATUS_SUCCESS;
    if (plan->mem && hipFree(plan->mem) != hipSuccess) {
        (void)hipGetLastError();
        st = OZ2_STATUS_HIP_ERROR;
    }
    delete plan;
    return st;
}

int oz2_set_debug(oz2_handle_t h, int debug) {
    if (!h) return -1;
    h->debug = debug ? 1 : 0;
    return OZ2_STATUS_SUCCESS;
}

int oz2_debug_copy(oz2_handle_t h, int which, void* dst, size_t capacity, size_t* bytes,
                   int64_t dims[5]) {
    if (!h) return -1;
    const Layout& L = h->last;
    if (!L.valid) return OZ2_STATUS_INTERNAL;
    size_t off = 0, nbytes = 0;
    int64_t d[5] = {1, 1, 1, 1, 1};
    if (L.prepared && which >= 0 && which <= 3) return OZ2_STATUS_NOT_SUPPORTED;
    switch (which) {
        case 0: off = L.off_amaxA; nbytes = 8 * (size_t)L.mp; d[2] = L.mp; break;
        case 1: off = L.off_amaxB; nbytes = 8 * (size_t)L.np; d[2] = L.np; break;
        case 2: off = L.off_pa; nbytes = L.bytes_pa;
            d[0] = L.sets; d[1] = L.s; d[2] = L.kp / kPanelK; d[3] = L.mp; d[4] = kPanelK; break;
        case 3: off = L.off_pb; nbytes = L.bytes_pb;
            d[0] = L.sets; d[1] = L.s; d[2] = L.kp / kPanelK; d[3] = L.np; d[4] = kPanelK; break;
        case 4: off = L.off_res; nbytes = L.bytes_res;
            d[0] = L.outs; d[1] = L.s; d[2] = L.n; d[3] = L.mp; d[4] = L.chunks; break;
        case 5: off = L.off_chat; nbytes = L.bytes_chat;
            d[0] = L.outs; d[2] = L.n; d[3] = L.mp; d[4] = L.NL; break;
        default: return -2;
    }
    if (bytes) *bytes = nbytes;
    if (dims)
        for (int i = 0; i < 5; ++i) dims[i] = d[i];
    if (!dst) return OZ2_STATUS_SUCCESS;
    if (capacity < nbytes) return -4;
    if (hipStreamSynchronize(h->stream) != hipSuccess) return OZ2_STATUS_HIP_ERROR;
    if (nbytes && hipMemcpy(dst, (char*)h->last_ws + off, nbytes, hipMemcpyDeviceToHost) != hipSuccess)
        return OZ2_STATUS_HIP_ERROR;
    return OZ2_STATUS_SUCCESS;
}

int oz2_test_crt(oz2_handle_t h, int64_t count, int num_moduli, const uint8_t* residues,
                 uint32_t* words) {
    if (!h) return -1;
    if (count < 0) return -2;
    const ModuliPlan* pl = moduli_plan(num_moduli);
    if (!pl) return -3;
    if (count == 0) return OZ2_STATUS_SUCCESS;
    if (!residues) return -4;
    if (!words) return -5;
    CrtTestParams P{};
    fill_crt_tables(*pl, &P);
    P.R = residues; P.count = count; P.words = words; P.s = num_moduli;
    OZ2_LAUNCH(launch_crt_test(P, pl->NL, h->stream));
    return OZ2_STATUS_SUCCESS;
}

}  // extern "C"
