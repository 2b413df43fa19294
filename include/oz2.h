/*
 * oz2.h -- C ABI of the oz2 library: FP64 real and complex matrix products
 * (DGEMM / ZGEMM) emulated with Ozaki scheme II on the INT8 matrix cores of
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the BLAS one, C <- alpha op(A) op(B) + beta C, with
 * column-major storage, op in {N, T, C} and leading dimensions ("Emulating
 * DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs: Ozaki Scheme II
 * on the Xe2 Architecture", Sec. 1 contributions and Sec. 2.1 notation).
 * The interface mirrors dgemm/zgemm with one extra argument, the number of
 * moduli s (same page, Sec. 9.1).  How a call is computed (same page, Sec. 2.3
 * and Sec. 4): every row of op(A) and column of op(B) is scaled by a power of
 * two and rounded to integers with at most t+1 bits (Sec. 4.1), the integers
 * are reduced to signed INT8 residues modulo s pairwise-coprime moduli <= 256
 * (Sec. 2.3 step 2, Sec. 4.2), s exact INT8 products with INT32 accumulation
 * are formed (Sec. 2.3 step 3, Sec. 4.3), and the integer product is recovered
 * by the Chinese remainder theorem, rounded once to double and scaled back
 * (Sec. 4.4).  ZGEMM uses the exact integer 3M (Karatsuba) form, 3s INT8
 * products (Sec. 5).
 *
 * Conventions shared by every entry point
 *  - Pointers to matrices are DEVICE pointers (hipMalloc / torch CUDA
 *    tensors) owned by the caller; the library never frees them.  Complex
 *    matrices are interleaved (re, im) pairs of doubles (complex128).
 *  - Work is enqueued asynchronously, in order, on the handle's stream;
 *    calls return without synchronizing.  Device-side faults surface at the
 *    caller's next synchronization.
 *  - Return value: 0 on success; -i when argument i (1-based, the handle is
 *    argument 1) is invalid, LAPACK "info" style; a positive OZ2_STATUS_*
 *    code for run-time failures (see oz2_status_string()).
 *  - A handle is not thread-safe; use one handle per host thread.
 *  - Quick returns follow reference BLAS: m = 0 or n = 0 does nothing;
 *    alpha = 0 or k = 0 sets C <- beta C (C is not read when beta = 0) and
 *    A and B are not read.  When beta = 0, C is never read, so NaN in C does
 *    not propagate.
 *  - An Inf or NaN anywhere in a row of op(A) (column of op(B)) makes the
 *    whole row (column) of the result NaN (Arc page Sec. 8.1 and Sec. 9.3).
 *  - Results are deterministic and independent of the launch configuration:
 *    all accumulation is exact integer arithmetic (Arc page Sec. 9.1).
 *    Normal results are the correctly rounded value of
 *    2^(-D_i-E_j) * c_hat_ij; subnormal results may be rounded twice
 *    (Arc page Sec. 4.4, Sec. 9.3).  alpha/beta are then applied as
 *    t1 = alpha*x; t2 = beta*c; C = t1 + t2 (complex:
 *    re = (ar*xr - ai*xi) + (br*cr - bi*ci), im = (ar*xi + ai*xr) + (br*ci + bi*cr)),
 *    each operation rounded separately.
 */
#ifndef OZ2_H
#define OZ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oz2_context* oz2_handle_t;

enum {
    OZ2_STATUS_SUCCESS = 0,
    OZ2_STATUS_ALLOC_FAILED = 1,     /* device workspace allocation failed */
    OZ2_STATUS_HIP_ERROR = 2,        /* a HIP runtime call or launch failed */
    OZ2_STATUS_RANGE = 3,            /* no scaling width t >= 1 for this (s, k) */
    OZ2_STATUS_WORKSPACE_LIMIT = 4,  /* workspace would exceed the memory limit */
    OZ2_STATUS_NOT_SUPPORTED = 5,    /* e.g. no gfx950 device */
    OZ2_STATUS_INTERNAL = 6,
    OZ2_STATUS_SCRATCH_LIMIT = 7     /* oz2_dgemm_noalloc: too large for the fixed scratch */
};

/* Create a handle bound to the current HIP device; its stream is the null
 * stream until oz2_set_stream().  *h receives the handle. */
int oz2_create(oz2_handle_t* h);

/* Free the handle and its workspace (waits for the handle's stream first).
 * The stream itself is not destroyed. */
int oz2_destroy(oz2_handle_t h);

/* All later work of this handle is enqueued on `stream` (a hipStream_t,
 * NULL for the null stream).  The handle's calls share one workspace, so on a
 * change of stream the new stream is made to wait (an event, no host wait)
 * for everything already queued on the old one: calls issued on different
 * streams through one handle run in issue order.  Returns OZ2_STATUS_HIP_ERROR
 * if the event cannot be recorded or waited on. */
int oz2_set_stream(oz2_handle_t h, void* stream);

/* Cap on the workspace in bytes; 0 (the default) means the free device
 * memory reported by hipMemGetInfo at the call.  A product whose workspace
 * would exceed the cap is computed in blocks of C, each with all of k: every
 * block has the full row and column exponents, so the result is bitwise
 * that of the untiled call (the resident-memory hint and memory-aware tiling
 * of Arc page Sec. 6).  The blocking is the cheapest one that fits under a
 * cost model (the shape of Arc page Sec. 9.2): block sides are the whole
 * dimension or a power-of-two multiple of 256 below it (Table 16's 2^j
 * tiles), rows and columns chosen separately; the model sums the residue
 * products of every block (a per-block time measured on this GPU, over
 * waves of 256 CUs), the scans and encodes, the reconstruction and the
 * launches.  One operand's encoded block is kept while the other's blocks
 * go by, so that operand is encoded once in total; the model picks which.
 * OZ2_STATUS_WORKSPACE_LIMIT is returned only when not even a 256 x 256 block
 * fits.  A tiled call reports its whole duration in ms[2] of
 * oz2_get_phase_times, oz2_get_tile_plan reports its blocking, and
 * oz2_debug_copy sees its last block. */
int oz2_set_memory_limit(oz2_handle_t h, size_t bytes);

/* Current workspace size in bytes (0 before the first call). */
int oz2_get_workspace_size(oz2_handle_t h, size_t* bytes);

/* Enable (1) or disable (0) per-phase hipEvent timing of later calls. */
int oz2_set_timing(oz2_handle_t h, int enable);

/* Phase times in milliseconds of the last timed call: ms[0] scan (row/column
 * exponents), ms[1] encode (integerize + residues), ms[2] residue GEMM,
 * ms[3] reconstruct (CRT + alpha/beta).  A call that took the fused short-k
 * path (see oz2_dgemm) reports its single kernel in ms[2] and 0 elsewhere.
 * Synchronizes with the last call. */
int oz2_get_phase_times(oz2_handle_t h, float ms[4]);

/* Blocking of the last product on this handle (oz2_set_memory_limit):
 * *mb x *nb entries of C per block (the whole m x n when untiled) and
 * *held, one of OZ2_TILE_*: which operand's encoded block stayed in the
 * workspace across the other's blocks.  Any output pointer may be NULL. */
enum {
    OZ2_TILE_UNTILED = 0,   /* one block: the whole product */
    OZ2_TILE_HOLD_A = 1,    /* block rows outer: each op(A) block encoded once */
    OZ2_TILE_HOLD_B = 2,    /* block columns outer: each op(B) block encoded once */
    OZ2_TILE_PREPARED = 3   /* oz2_gemm_prepared in blocks of the prepared planes */
};
int oz2_get_tile_plan(oz2_handle_t h, int64_t* mb, int64_t* nb, int* held);

/* Default precision policy (Arc page Sec. 9.1): the smallest s in [2, 24]
 * whose scaling width t(s, k) reaches `bits`; 24 when none does. */
int oz2_moduli_for_bits(int64_t k, int bits, int is_complex);

/* Host-side plan of the method for (s, k): moduli in descending order
 * (moduli_out[24], first s entries used), the scaling width t (<= 0 when
 * none exists), N_L = number of 32-bit words of c_hat, and log2 M.  Any
 * output pointer may be NULL.  Returns -1 for s outside [2, 24]. */
int oz2_plan_info(int num_moduli, int64_t k, int is_complex, int32_t* moduli_out,
                  int* t_out, int* nl_out, double* log2M_out);

/* C <- alpha op(A) op(B) + beta C.  op(A) is m x k, op(B) is k x n, C is
 * m x n; lda >= max(1, rows of A as stored), likewise ldb, ldc >= max(1, m).
 * transa/transb in {'N','T','C'} (upper or lower case; 'C' = 'T' here).
 * 2 <= num_moduli <= 24; k may exceed 131071 (the INT32 accumulation is
 * split internally, Arc page Sec. 4.3).  Returns OZ2_STATUS_RANGE when no
 * scaling width exists for (num_moduli, k).
 * Products with 1 <= k <= 32 and m <= 64 or n <= 64 take a fused path (one
 * kernel, every step of the method per 16 x 16 output tile in registers)
 * that gives bit-identical results to the four-phase path and needs no
 * workspace. */
int oz2_dgemm(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n, int64_t k,
              double alpha, const double* A, int64_t lda, const double* B, int64_t ldb,
              double beta, double* C, int64_t ldc, int num_moduli);

/* For callers that cannot allocate device memory during a call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * oz2_dgemm with the same arguments, results and status codes, that calls
 * no hipMalloc, hipFree or other allocating routine.  Its workspace is a
 * fixed 128 MiB device array per GPU, held from the library's load on that
 * GPU until the process ends; oz2_create takes its address for the handle's
 * device.  A product whose workspace exceeds 128 MiB runs in blocks of C
 * that fit it, bitwise equal to the untiled result (as under
 * oz2_set_memory_limit); OZ2_STATUS_SCRATCH_LIMIT when not even one
 * 256 x 256 block with all of k fits (about k > 16000 at s = 16), with
 * nothing enqueued.  Every call on one GPU, from any handle, shares that
 * GPU's array and finds the previous call's contents in it (nothing here
 * needs it cleared): calls that overlap on one GPU race, so issue them on
 * one stream or order them.  OZ2_STATUS_HIP_ERROR if the current device is
 * not the handle's or the array's address could not be taken.  The
 * handle's own workspace is not used or grown. */
int oz2_dgemm_noalloc(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n, int64_t k,
                      double alpha, const double* A, int64_t lda, const double* B, int64_t ldb,
                      double beta, double* C, int64_t ldc, int num_moduli);

/* Complex version (Arc page Sec. 5): A, B, C are interleaved complex128;
 * alpha[2] and beta[2] are HOST arrays (re, im); 'C' conjugates.  Uses one
 * exponent per row/column shared by the real and imaginary parts and the
 * scaling width of a 2k-term product. */
int oz2_zgemm(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n, int64_t k,
              const double* alpha, const double* A, int64_t lda, const double* B, int64_t ldb,
              const double* beta, double* C, int64_t ldc, int num_moduli);

/* batch independent products C_b <- alpha op(A_b) op(B_b) + beta C_b with
 * A_b = A + b*strideA (in doubles), likewise B and C.  A stride of 0 shares
 * one operand across the batch (the shared operators of a tensor mode
 * product: "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode
 * Products", Sec. 2.1 Eq. (5) and Sec. 5.1).  Every product uses its own
 * row/column exponents, as separate oz2_dgemm calls would (bit-identical
 * results).  With 1 <= k <= 32 and m <= 64 or n <= 64 the whole batch is one
 * launch of the fused path; otherwise the products run one after another on
 * the four-phase path.  Argument numbers of the -i codes: h 1, transa 2,
 * transb 3, m 4, n 5, k 6, alpha 7, A 8, lda 9, strideA 10, B 11, ldb 12,
 * strideB 13, beta 14, C 15, ldc 16, strideC 17, batch 18, num_moduli 19. */
int oz2_dgemm_strided_batched(oz2_handle_t h, char transa, char transb, int64_t m, int64_t n,
                              int64_t k, double alpha, const double* A, int64_t lda,
                              int64_t strideA, const double* B, int64_t ldb, int64_t strideB,
                              double beta, double* C, int64_t ldc, int64_t strideC,
                              int64_t batch, int num_moduli);

/* ---------------------------------------------------------------------
 * Prepared operands: the row exponents and residue planes of op(A), or the
 * column exponents and residue planes of op(B), computed once and kept on
 * the device, so that products which reuse an operand skip its scan and
 * encode phases.  The Arc page names reuse of the residues of A across
 * calls as future work (Sec. 10); the chain page caches the operators'
 * residues the same way ("You Only Convert Twice", Sec. 5, Algorithm 6 and
 * Fig. 4).  A prepared operand depends on (side, complex, op, rows, k, s):
 * every product that uses it has the same k and num_moduli, and therefore
 * the same scaling width t, so results are bitwise those of oz2_dgemm /
 * oz2_zgemm on the same data.
 * ------------------------------------------------------------------- */
typedef struct oz2_operand* oz2_operand_t;

/* Allocate DEVICE memory for a prepared operand (owned by the returned
 * object; rows_pad * k_pad * s * sets bytes plus 8 * rows_pad, with
 * rows_pad = rows rounded up to 256, k_pad = k rounded up to 256, sets = 1
 * real or 3 complex) and enqueue its scan and encode on h's stream.
 * side 'A': X is A, op(A) = op(X) is rows x k (rows = m), X stored m x k
 * (trans 'N') or k x m (trans 'T' or 'C'); side 'B': X is B, op(B) is
 * k x rows (rows = n), X stored k x n ('N') or n x k ('T' / 'C').  X is a
 * DEVICE pointer (complex128 when is_complex), read only by the enqueued
 * work: it may be changed or freed once h's stream has passed this call.
 * Argument numbers of the -i codes: h 1, side 2, trans 4, rows 5, k 6,
 * X 7, ld 8, num_moduli 9, out 10.  OZ2_STATUS_RANGE when no scaling width
 * exists for (num_moduli, k); OZ2_STATUS_ALLOC_FAILED when the device
 * memory cannot be allocated.  *out is NULL on any failure. */
int oz2_operand_create(oz2_handle_t h, char side, int is_complex, char trans, int64_t rows, int64_t k,
                       const double* X, int64_t ld, int num_moduli, oz2_operand_t* out);

/* Re-encode new data of the same shape into `op` (scan and encode enqueued
 * on h's stream): -1 h, -2 op, -3 X, -4 ld.  Work already enqueued that
 * reads `op` uses the old data (stream order). */
int oz2_operand_update(oz2_handle_t h, oz2_operand_t op, const double* X, int64_t ld);

/* Free a prepared operand's device memory (hipFree waits for the device, so
 * enqueued work that reads it completes first). */
int oz2_operand_destroy(oz2_operand_t op);

/* C <- alpha op(A) op(B) + beta C from a prepared op(A) (side 'A') and a
 * prepared op(B) (side 'B') with the same is_complex, k and num_moduli: the
 * residue GEMM and reconstruct phases only.  m = rows of pa, n = rows of pb.
 * alpha[2], beta[2]: HOST arrays (re, im); the imaginary parts are ignored
 * for real operands.  C is a DEVICE pointer, ldc >= m.  The workspace holds
 * only the product residues; when they exceed the memory limit, C is
 * computed in blocks whose residues fit (sides a power-of-two multiple of
 * 256 or the whole dimension, chosen by the cost model of oz2_set_memory_limit),
 * each reading its rows and columns of the prepared planes in place: bitwise
 * the untiled result.  OZ2_STATUS_WORKSPACE_LIMIT only when not even a
 * 256 x 256 block fits.  Phase times: ms[0] = ms[1] = 0 (a tiled call reports
 * its whole duration in ms[2]).  Argument numbers of the -i codes: h 1, pa 2, pb 3
 * (also when it does not match pa), alpha 4, beta 5, C 6, ldc 7.
 * oz2_debug_copy of buffers 0-3 after such a call returns
 * OZ2_STATUS_NOT_SUPPORTED (they live in the operand objects). */
int oz2_gemm_prepared(oz2_handle_t h, oz2_operand_t pa, oz2_operand_t pb, const double* alpha,
                      const double* beta, double* C, int64_t ldc);

/* ---------------------------------------------------------------------
 * Persistent tensor-mode chains (OzII-RescaleBE, "You Only Convert Twice:
 * Ozaki Scheme II for Chained Tensor Mode Products", Sec. 5.2, Algorithm 7):
 * Y = X x_{m1} A1 x_{m2} A2 ... x_{md} Ad for a batch of n x n x n tensors
 * (column-major X[i + n j + n^2 k], tensor t at X + t n^3) with shared
 * n x n operators; x_m contracts direction m in {1, 2, 3} with the
 * operator's second index.  By default m_i = ((i - 1) mod 3) + 1, so depth 3
 * is Y_abc = sum A1_ai A2_bj A3_ck X_ijk and longer chains revisit the
 * directions in turn (Sec. 6); Algorithm 7 takes any sequence, and so does
 * this interface (other sequences take slower byte-wise residue stores).  The tensor is encoded once with one
 * power-of-two exponent (b significand bits), stays in residue form through
 * all d mode products -- after every product but the last the g_i smallest
 * moduli are dropped by rounded division (Sec. 2.3.1 Eq. 15, Algorithm 1)
 * and restored by base extension (Sec. 4.4 Eq. 26, Algorithm 4; the
 * kernels may take the CRT form of it, oz2_set_chain_crt, with the same
 * residues) -- and is reconstructed once (Algorithm 5).  Row scales still
 * pending on a direction are folded into the columns of the next operator
 * on it before that operator is encoded (Sec. 5.2, after Eq. 28).  The
 * residue basis is the max-product modulus set for num_moduli, descending.
 * Limits of this implementation: 1 <= n <= OZ2_CHAIN_MAX_N,
 * 1 <= depth <= OZ2_CHAIN_MAX_DEPTH, 2 <= num_moduli <= OZ2_CHAIN_MAX_MODULI.
 * Two kernels run it, with identical results: for 8 < n <= 16 one kernel
 * per batch keeps each tensor's residues (padded to 16^3) in LDS; for other
 * n (or when oz2_set_chain_kernel asks for it) the residues (padded to a
 * multiple of 8 in each direction) stay in HBM, in the handle's workspace,
 * between one kernel per product.  Results are deterministic;
 * parity with the CPU oracle is bitwise.
 * ------------------------------------------------------------------- */
#define OZ2_CHAIN_MAX_N 256
#define OZ2_CHAIN_MAX_DEPTH 8
#define OZ2_CHAIN_MAX_MODULI 16
typedef struct oz2_chain_plan* oz2_chain_plan_t;

/* Plan a chain (Algorithms 2, 3; host work): the largest b <= 53 whose
 * greedy drop schedule passes every range check for the effective
 * operators, the drop counts g, and the effective operators' residues and
 * the row exponents left pending on each direction, which are copied to
 * DEVICE memory owned by the plan (about 3.5 KiB + 12 np + depth * (2 KiB +
 * s * np * (np rounded up to 16)) bytes, plus depth * 4 KiB for n <= 16).  ops: HOST
 * array of depth pointers to HOST n x n column-major operators (finite).
 * modes: HOST array of depth directions in {1, 2, 3}, or NULL for the
 * directions in turn.  Argument numbers: h 1, n 2, depth 3, ops 4 (also a
 * NULL entry or a non-finite operator entry), modes 5, num_moduli 6, out 7.
 * OZ2_STATUS_RANGE when no b in [1, 53] passes.  The plan can be reused for
 * any number of tensors and calls. */
int oz2_chain_plan_create(oz2_handle_t h, int64_t n, int depth, const double* const* ops, const int* modes,
                          int num_moduli, oz2_chain_plan_t* out);

/* The plan's depth, significand bits b and drop counts g[0 .. depth - 1]
 * (g[depth - 1] = 0); any pointer may be NULL, g must hold depth ints. */
int oz2_chain_plan_info(oz2_chain_plan_t plan, int* depth, int* b, int* g);

/* Run the planned chain on `batch` tensors: X and Y are DEVICE arrays of
 * batch * n^3 doubles that must not overlap.  Asynchronous on h's stream.
 * The LDS kernel is one launch (phase times: the whole chain in ms[2]).  The
 * HBM kernels use 2 s np^3 + 8 bytes of workspace per tensor (np = n rounded
 * up to a multiple of 8), under the memory limit in as many equal batches as
 * needed, OZ2_STATUS_WORKSPACE_LIMIT when not even one tensor fits; phase
 * times: scan ms[0], encode ms[1], the rescaling products ms[2], the last
 * product and the reconstruction ms[3] (everything in ms[2] when the call
 * ran in several batches).  A tensor with a non-finite entry gives an
 * all-NaN result tensor.  Argument numbers: h 1, plan 2, X 3, Y 4, batch 5.
 * OZ2_STATUS_NOT_SUPPORTED when the LDS kernel is asked for and n > 16. */
int oz2_chain_rescale_be(oz2_handle_t h, oz2_chain_plan_t plan, const double* X, double* Y,
                         int64_t batch);

/* Which kernels oz2_chain_rescale_be uses on this handle: AUTO (the
 * default: LDS for 8 < n <= 16, else HBM), LDS (n <= 16), or HBM (any n).  Argument
 * numbers: h 1, kernel 2. */
enum {
    OZ2_CHAIN_KERNEL_AUTO = 0,
    OZ2_CHAIN_KERNEL_LDS = 1,
    OZ2_CHAIN_KERNEL_HBM = 2
};
int oz2_set_chain_kernel(oz2_handle_t h, int kernel);

/* After a product's drops the chain kernels extend the kept residues to the
 * dropped moduli by the Chinese remainder theorem where the plan's bound
 * leaves the kept moduli's product M a margin (|X| <= (1/2 - 2^-13) M; in
 * the LDS kernel when every product with drops has it), else by mixed-radix
 * digits (Algorithm 4, Eq. 26); both give the same residues.
 * enable = 0 takes the mixed-radix form everywhere on this handle (a test
 * hook), 1 (the default) the CRT form where allowed.  Argument numbers:
 * h 1, enable 2. */
int oz2_set_chain_crt(oz2_handle_t h, int enable);

/* Free a plan and its device memory. */
int oz2_chain_plan_destroy(oz2_chain_plan_t plan);

/* Human-readable text of a status code (static storage). */
const char* oz2_status_string(int status);

/* ---------------------------------------------------------------------
 * Test hooks (the GPU analogues of the split and CRT unit tests of the Arc
 * page, Sec. 8.1).  Not needed for normal use.
 * ------------------------------------------------------------------- */

/* debug = 1: later calls take the four-phase path (never the fused short-k
 * one) and also keep c_hat (N_L 32-bit two's-complement words per entry,
 * entry-major, column-major entry order) in the workspace, so that every
 * intermediate buffer can be copied out with oz2_debug_copy. */
int oz2_set_debug(oz2_handle_t h, int debug);

/* Copy an intermediate buffer of the handle's LAST call to HOST memory
 * `dst` (at most `capacity` bytes; synchronizes first).  `which`:
 *   0 row maxima |op(A)| as IEEE bit patterns, uint64[m_pad]
 *   1 column maxima |op(B)|, uint64[n_pad]
 *   2 residue planes of op(A) in k-panels: int8[sets][s][k_pad/64][m_pad][64]
 *     (sets = 1 real, 3 complex: re, im, re+im): panel p holds k positions
 *     64p .. 64p+63 of every row as 64 contiguous bytes
 *   3 residue planes of op(B): int8[sets][s][k_pad/64][n_pad][64]
 *   4 product residues in [0, m_t): uint8[outs][s][n][m_pad] (outs = 1 real,
 *     2 complex: Re, Im)
 *   5 c_hat words (only when debug was enabled): uint32[outs][n][m_pad][N_L]
 * dims[0..4] receive the buffer's extents: (sets, s, k_pad/64, rows_pad, 64)
 * for 2 and 3; (outs, s, n, m_pad, runs) for 4; (outs, 1, n, m_pad, N_L)
 * for 5; (1, 1, rows_pad, 1, 1) for 0 and 1.
 * Returns the byte size in *bytes.  -2 for an unknown `which`. */
int oz2_debug_copy(oz2_handle_t h, int which, void* dst, size_t capacity, size_t* bytes,
                   int64_t dims[5]);

/* CRT reconstruction only: from residues r[t][q] in [0, m_t) (DEVICE
 * uint8[num_moduli][count]) compute c = the integer in (-M/2, M/2] that is
 * congruent to r_t mod m_t for every t, valid when |c| <= M/4, as N_L
 * two's-complement 32-bit words per entry (DEVICE uint32[count][N_L]). */
int oz2_test_crt(oz2_handle_t h, int64_t count, int num_moduli, const uint8_t* residues,
                 uint32_t* words);

#ifdef __cplusplus
}
#endif

#endif /* OZ2_H */
