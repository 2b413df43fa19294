/*
 * oz2_oracle.c -- plain, slow CPU oracle for Ozaki scheme II DGEMM/ZGEMM
 * emulation.  TEST INFRASTRUCTURE ONLY: called by the tests, by
 * __graft_entry__.smoke() and by the cpu_baseline leg of bench.py, never by
 * the product.  It shares no code, header or table with the GPU library.
 *
 * It follows the method of "Emulating DGEMM and ZGEMM with INT8 Matrix
 * Engines on Intel Arc GPUs: Ozaki Scheme II on the Xe2 Architecture":
 *   Sec. 4.1  D_i = t - e(max_p |a_ip|), E_j = t - e(max_p |b_pj|)
 *   Sec. 2.3  a_hat = rint(a * 2^D) (ties to even), b_hat likewise
 *   Sec. 2.3  c_hat = a_hat . b_hat, here computed EXACTLY in wide integers
 *             (no residues, no CRT: that is what makes it an oracle)
 *   Sec. 4.4  output = c_hat * 2^(-D_i-E_j) rounded once to double
 *   Sec. 5    ZGEMM: Re = sum(ar br - ai bi), Im = sum(ar bi + ai br), the
 *             plain 4M form (the 3M form of the product must equal it)
 *   Sec. 8.1  a non-finite entry makes its whole row/column of C NaN
 * The BLAS operation is C <- alpha op(A) op(B) + beta C with column-major
 * storage (Sec. 2.1, Sec. 1).  The alpha/beta evaluation order is not given
 * by the pages; the one used is: t1 = alpha*x; t2 = beta*c; out = t1 + t2,
 * every operation rounded separately (compile with -ffp-contract=off).  The
 * tests pin it order-free, against the rounding bound of the exact rational
 * alpha*x + beta*c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef __int128 i128;
typedef unsigned __int128 u128;
typedef struct { uint64_t w[4]; } i256; /* two's complement, w[0] lowest */

/* ------------------------------------------------------------------ */
/* 256-bit integer helpers                                              */
/* ------------------------------------------------------------------ */
static i256 i256_from_i128(i128 x) {
    i256 r;
    u128 u = (u128)x;
    uint64_t ext = (x < 0) ? ~0ull : 0ull;
    r.w[0] = (uint64_t)u;
    r.w[1] = (uint64_t)(u >> 64);
    r.w[2] = ext;
    r.w[3] = ext;
    return r;
}

static i256 i256_add(i256 a, i256 b) {
    i256 r;
    u128 carry = 0;
    for (int q = 0; q < 4; ++q) {
        u128 s = (u128)a.w[q] + b.w[q] + carry;
        r.w[q] = (uint64_t)s;
        carry = s >> 64;
    }
    return r;
}

static i256 i256_neg(i256 a) {
    i256 one = {{1, 0, 0, 0}};
    for (int q = 0; q < 4; ++q) a.w[q] = ~a.w[q];
    return i256_add(a, one);
}

static i256 i256_sub(i256 a, i256 b) { return i256_add(a, i256_neg(b)); }

static int i256_is_neg(i256 a) { return (int64_t)a.w[3] < 0; }

static int i256_bitlen(i256 a) { /* of a non-negative value */
    for (int q = 3; q >= 0; --q)
        if (a.w[q]) return 64 * q + 64 - __builtin_clzll(a.w[q]);
    return 0;
}

static int i256_bit(i256 a, int b) {
    if (b < 0 || b >= 256) return 0;
    return (int)((a.w[b >> 6] >> (b & 63)) & 1u);
}

/* exact product of two signed integers of magnitude < 2^127 */
static i256 mul_i128(i128 a, i128 b) {
    int neg = (a < 0) != (b < 0);
    u128 ua = a < 0 ? (u128)0 - (u128)a : (u128)a;
    u128 ub = b < 0 ? (u128)0 - (u128)b : (u128)b;
    uint64_t a0 = (uint64_t)ua, a1 = (uint64_t)(ua >> 64);
    uint64_t b0 = (uint64_t)ub, b1 = (uint64_t)(ub >> 64);
    u128 p00 = (u128)a0 * b0, p01 = (u128)a0 * b1, p10 = (u128)a1 * b0, p11 = (u128)a1 * b1;
    i256 r;
    r.w[0] = (uint64_t)p00;
    u128 mid = (p00 >> 64) + (uint64_t)p01 + (uint64_t)p10;
    r.w[1] = (uint64_t)mid;
    u128 hi = (mid >> 64) + (p01 >> 64) + (p10 >> 64) + (uint64_t)p11;
    r.w[2] = (uint64_t)hi;
    r.w[3] = (uint64_t)(hi >> 64) + (uint64_t)(p11 >> 64);
    return neg ? i256_neg(r) : r;
}

/* ------------------------------------------------------------------ */
/* Scaling and integerization (P1 Sec. 2.3 step 1, Sec. 4.1)            */
/* ------------------------------------------------------------------ */
static int e_of(double x) { /* 2^(e-1) <= |x| < 2^e */
    int e;
    frexp(x, &e);
    return e;
}

/* rint(a * 2^D): ldexp is exact whenever the scaled value is >= 2^-1022,
 * and anything smaller rounds to zero anyway; nearbyint rounds to nearest
 * with ties to even (the default rounding mode). */
static i128 integerize(double a, int D) {
    double v = nearbyint(ldexp(a, D));
    return (i128)v;
}

/* element p of vector v of op(X): a row of op(A) (is_b = 0) or a column of
 * op(B) (is_b = 1); op in {N, T, C}; column-major storage with leading
 * dimension ld; complex data interleaved (re, im). */
static void load_elem(int cplx, char op, int is_b, const double* X, int64_t ld, int64_t v,
                      int64_t p, double* re, double* im) {
    int trans = (op == 'T' || op == 't' || op == 'C' || op == 'c');
    int64_t idx;
    if (!is_b)
        idx = trans ? p + v * ld : v + p * ld;
    else
        idx = trans ? v + p * ld : p + v * ld;
    if (cplx) {
        *re = X[2 * idx];
        *im = X[2 * idx + 1];
        if (op == 'C' || op == 'c') *im = -*im;
    } else {
        *re = X[idx];
        *im = 0.0;
    }
}

/* Scan and integerize one vector: D, non-finite flag, a_hat (re, im). */
static void prepare_vector(int cplx, char op, int is_b, int64_t k, const double* X, int64_t ld,
                           int64_t v, int t, int32_t* D, uint8_t* flag, i128* hre, i128* him) {
    double amax = 0.0;
    int bad = 0;
    for (int64_t p = 0; p < k; ++p) {
        double re, im;
        load_elem(cplx, op, is_b, X, ld, v, p, &re, &im);
        if (!isfinite(re) || !isfinite(im)) bad = 1;
        if (fabs(re) > amax) amax = fabs(re);
        if (fabs(im) > amax) amax = fabs(im);
    }
    int d = (bad || amax == 0.0) ? 0 : t - e_of(amax);
    *D = d;
    *flag = (uint8_t)bad;
    for (int64_t p = 0; p < k; ++p) {
        double re, im;
        load_elem(cplx, op, is_b, X, ld, v, p, &re, &im);
        hre[p] = bad ? 0 : integerize(re, d);
        if (him) him[p] = bad ? 0 : integerize(im, d);
    }
}

/* ------------------------------------------------------------------ */
/* Correctly rounded output (P1 Sec. 4.4)                               */
/* ------------------------------------------------------------------ */
/* q = RNE(mag / 2^n) for 0 < n; the caller guarantees q < 2^64 */
static uint64_t shr_rne(i256 mag, int n) {
    uint64_t q = 0;
    for (int b = 0; b < 64; ++b) q |= (uint64_t)i256_bit(mag, n + b) << b;
    int half = i256_bit(mag, n - 1);
    int sticky = 0;
    for (int b = 0; b < n - 1 && b < 256; ++b)
        if (i256_bit(mag, b)) { sticky = 1; break; }
    if (half && (sticky || (q & 1u))) q += 1;
    return q;
}

/* RN(c * 2^-S), c an exact integer; integer zero gives +0 */
static double round_scaled(i256 c, int S) {
    int neg = i256_is_neg(c);
    i256 mag = neg ? i256_neg(c) : c;
    int L = i256_bitlen(mag);
    if (L == 0) return 0.0;
    int expo = L - 1 - S;                            /* exponent of the leading bit */
    int p = (expo >= -1022) ? 53 : 53 - (-1022 - expo); /* significant bits available */
    int n = L - p;                                   /* bits to drop */
    double r;
    if (n <= 0) {
        /* mag has at most 53 bits and the value is representable */
        r = ldexp((double)mag.w[0], -S); /* exact: at most 53 bits, representable */
    } else if (n > L) {
        r = 0.0; /* below half of the smallest subnormal */
    } else {
        uint64_t q = shr_rne(mag, n);
        r = ldexp((double)q, n - S);
    }
    return neg ? -r : r;
}

/* ------------------------------------------------------------------ */
/* Entry point: selected entries of C <- alpha op(A) op(B) + beta C      */
/* ------------------------------------------------------------------ */
static void put_chat(uint64_t* dst, i256 v) { memcpy(dst, v.w, sizeof v.w); }

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int orc_gemm_entries(int cplx, char transa, char transb, int64_t m, int64_t n, int64_t k,
                     const double* alpha, const double* A, int64_t lda, const double* B,
                     int64_t ldb, const double* beta, const double* C, int64_t ldc, int t,
                     int64_t ns, const int64_t* si, const int64_t* sj, double* out,
                     uint64_t* chat, int32_t* Dout, int32_t* Eout, uint8_t* flags, int nthreads) {
    if (m < 0 || n < 0 || k < 0 || ns < 0) return 1;
    const int nc = cplx ? 2 : 1;
    const double ar = alpha[0], ai = cplx ? alpha[1] : 0.0;
    const double br = beta[0], bi = cplx ? beta[1] : 0.0;
    const int beta_zero = (br == 0.0 && bi == 0.0);
    const int alpha_zero = (ar == 0.0 && ai == 0.0);
    memset(chat, 0, sizeof(uint64_t) * 4 * nc * (size_t)ns);
    memset(Dout, 0, sizeof(int32_t) * ns);
    memset(Eout, 0, sizeof(int32_t) * ns);
    memset(flags, 0, ns);

    /* BLAS quick return: alpha = 0 or k = 0 leaves C <- beta C */
    if (alpha_zero || k == 0) {
        for (int64_t q = 0; q < ns; ++q) {
            int64_t idx = si[q] + sj[q] * ldc;
            if (!cplx) {
                out[q] = beta_zero ? 0.0 : br * C[idx];
            } else if (beta_zero) {
                out[2 * q] = 0.0;
                out[2 * q + 1] = 0.0;
            } else {
                double cr = C[2 * idx], ci = C[2 * idx + 1];
                double t3 = br * cr, t4 = bi * ci;
                out[2 * q] = t3 - t4;
                double t5 = br * ci, t6 = bi * cr;
                out[2 * q + 1] = t5 + t6;
            }
        }
        return 0;
    }
    if (t < 1) return 3; /* no admissible scaling width */

    /* distinct rows of op(A) and columns of op(B) that are needed */
    int64_t* rmap = (int64_t*)malloc(sizeof(int64_t) * (m ? m : 1));
    int64_t* cmap = (int64_t*)malloc(sizeof(int64_t) * (n ? n : 1));
    for (int64_t i = 0; i < m; ++i) rmap[i] = -1;
    for (int64_t j = 0; j < n; ++j) cmap[j] = -1;
    int64_t nr = 0, ncol = 0;
    for (int64_t q = 0; q < ns; ++q) {
        if (si[q] < 0 || si[q] >= m || sj[q] < 0 || sj[q] >= n) {
            free(rmap);
            free(cmap);
            return 2;
        }
        if (rmap[si[q]] < 0) rmap[si[q]] = nr++;
        if (cmap[sj[q]] < 0) cmap[sj[q]] = ncol++;
    }
    int64_t* rlist = (int64_t*)malloc(sizeof(int64_t) * (nr ? nr : 1));
    int64_t* clist = (int64_t*)malloc(sizeof(int64_t) * (ncol ? ncol : 1));
    for (int64_t i = 0; i < m; ++i)
        if (rmap[i] >= 0) rlist[rmap[i]] = i;
    for (int64_t j = 0; j < n; ++j)
        if (cmap[j] >= 0) clist[cmap[j]] = j;

    i128* ahr = (i128*)malloc(sizeof(i128) * (size_t)(nr * k));
    i128* ahi = cplx ? (i128*)malloc(sizeof(i128) * (size_t)(nr * k)) : NULL;
    i128* bhr = (i128*)malloc(sizeof(i128) * (size_t)(ncol * k));
    i128* bhi = cplx ? (i128*)malloc(sizeof(i128) * (size_t)(ncol * k)) : NULL;
    int32_t* Dr = (int32_t*)malloc(sizeof(int32_t) * (nr ? nr : 1));
    int32_t* Ec = (int32_t*)malloc(sizeof(int32_t) * (ncol ? ncol : 1));
    uint8_t* fr = (uint8_t*)malloc(nr ? nr : 1);
    uint8_t* fc = (uint8_t*)malloc(ncol ? ncol : 1);
    int nt = nthreads > 0 ? nthreads : orc_max_threads();

#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t r = 0; r < nr; ++r)
        prepare_vector(cplx, transa, 0, k, A, lda, rlist[r], t, &Dr[r], &fr[r], ahr + r * k,
                       cplx ? ahi + r * k : NULL);
#pragma omp parallel for schedule(dynamic, 4) num_threads(nt)
    for (int64_t c = 0; c < ncol; ++c)
        prepare_vector(cplx, transb, 1, k, B, ldb, clist[c], t, &Ec[c], &fc[c], bhr + c * k,
                       cplx ? bhi + c * k : NULL);

#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t q = 0; q < ns; ++q) {
        int64_t r = rmap[si[q]], c = cmap[sj[q]];
        const i128* a_r = ahr + r * k;
        const i128* b_r = bhr + c * k;
        i256 acc_re = i256_from_i128(0), acc_im = i256_from_i128(0);
        if (!cplx) {
            for (int64_t p = 0; p < k; ++p) acc_re = i256_add(acc_re, mul_i128(a_r[p], b_r[p]));
        } else {
            const i128* a_i = ahi + r * k;
            const i128* b_i = bhi + c * k;
            for (int64_t p = 0; p < k; ++p) {
                acc_re = i256_add(acc_re, mul_i128(a_r[p], b_r[p]));
                acc_re = i256_sub(acc_re, mul_i128(a_i[p], b_i[p]));
                acc_im = i256_add(acc_im, mul_i128(a_r[p], b_i[p]));
                acc_im = i256_add(acc_im, mul_i128(a_i[p], b_r[p]));
            }
        }
        int bad = fr[r] | fc[c];
        int S = Dr[r] + Ec[c];
        Dout[q] = Dr[r];
        Eout[q] = Ec[c];
        flags[q] = (uint8_t)(fr[r] | (fc[c] << 1));
        put_chat(chat + (size_t)q * 4 * nc, acc_re);
        if (cplx) put_chat(chat + (size_t)q * 4 * nc + 4, acc_im);
        double xr = bad ? NAN : round_scaled(acc_re, S);
        double xi = bad ? NAN : (cplx ? round_scaled(acc_im, S) : 0.0);
        int64_t idx = si[q] + sj[q] * ldc;
        if (!cplx) {
            double t1 = ar * xr;
            if (beta_zero) {
                out[q] = t1;
            } else {
                double t2 = br * C[idx];
                out[q] = t1 + t2;
            }
        } else {
            double t1 = ar * xr, t2 = ai * xi;
            double u_re = t1 - t2;
            double t3 = ar * xi, t4 = ai * xr;
            double u_im = t3 + t4;
            if (beta_zero) {
                out[2 * q] = u_re;
                out[2 * q + 1] = u_im;
            } else {
                double cr = C[2 * idx], ci = C[2 * idx + 1];
                double t5 = br * cr, t6 = bi * ci;
                double v_re = t5 - t6;
                double t7 = br * ci, t8 = bi * cr;
                double v_im = t7 + t8;
                out[2 * q] = u_re + v_re;
                out[2 * q + 1] = u_im + v_im;
            }
        }
    }
    free(rmap); free(cmap); free(rlist); free(clist);
    free(ahr); free(ahi); free(bhr); free(bhi);
    free(Dr); free(Ec); free(fr); free(fc);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Residues for comparing the product's intermediate planes             */
/* ------------------------------------------------------------------ */
/* sym_m(v) in [-h, m-1-h], h = floor((m-1)/2), stored as a signed byte
 * (128, only possible for m = 256, wraps to -128). */
static int8_t sym_byte(i128 v, int m) {
    int h = (m - 1) / 2;
    i128 r = v % m;
    if (r < 0) r += m;
    if (r > m - 1 - h) r -= m;
    return (int8_t)(int)r;
}

/* D, flags, a_hat and the residue bytes of nvec vectors: sets (re) or
 * (re, im, re+im).  hat is [ncomp][nvec][k] of (lo, hi) int64 pairs;
 * planes is [nsets][s][nvec][k]. */
int orc_encode_vectors(int cplx, char op, int is_b, int64_t k, int64_t nvec, const double* X,
                       int64_t ld, int t, int s, const int32_t* moduli, int32_t* D,
                       uint8_t* flags, int64_t* hat, int8_t* planes, void* unused) {
    (void)unused;
    if (t < 1) return 3;
    i128* hre = (i128*)malloc(sizeof(i128) * (k ? k : 1));
    i128* him = (i128*)malloc(sizeof(i128) * (k ? k : 1));
    for (int64_t v = 0; v < nvec; ++v) {
        prepare_vector(cplx, op, is_b, k, X, ld, v, t, &D[v], &flags[v], hre, cplx ? him : NULL);
        for (int64_t p = 0; p < k; ++p) {
            int64_t* h0 = hat + 2 * (v * k + p);
            h0[0] = (int64_t)(uint64_t)(u128)hre[p];
            h0[1] = (int64_t)(hre[p] >> 64);
            if (cplx) {
                int64_t* h1 = hat + 2 * (nvec * k + v * k + p);
                h1[0] = (int64_t)(uint64_t)(u128)him[p];
                h1[1] = (int64_t)(him[p] >> 64);
            }
            for (int q = 0; q < s; ++q) {
                int m = moduli[q];
                planes[((size_t)(0 * s + q) * nvec + v) * k + p] = sym_byte(hre[p], m);
                if (cplx) {
                    planes[((size_t)(1 * s + q) * nvec + v) * k + p] = sym_byte(him[p], m);
                    planes[((size_t)(2 * s + q) * nvec + v) * k + p] = sym_byte(hre[p] + him[p], m);
                }
            }
        }
    }
    free(hre);
    free(him);
    return 0;
}

/* value mod m in [0, m) for count two's complement 256-bit integers */
void orc_residues_i256(int64_t count, const uint64_t* vals, int s, const int32_t* moduli,
                       uint8_t* out) {
    for (int64_t c = 0; c < count; ++c) {
        i256 v;
        memcpy(v.w, vals + 4 * c, sizeof v.w);
        int neg = i256_is_neg(v);
        i256 mag = neg ? i256_neg(v) : v;
        for (int q = 0; q < s; ++q) {
            uint64_t m = (uint64_t)moduli[q], r = 0;
            for (int w = 3; w >= 0; --w) {
                r = ((r << 32) | (mag.w[w] >> 32)) % m;
                r = ((r << 32) | (mag.w[w] & 0xffffffffull)) % m;
            }
            if (neg) r = (m - r) % m;
            out[(size_t)q * count + c] = (uint8_t)r;
        }
    }
}
