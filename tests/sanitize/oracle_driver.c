/* Host sanitizer driver for the oracle's C part (oracle/oz2_oracle.c), built
 * with -fsanitize=address,undefined by tests/test_sanitizers.py.  It calls
 * every exported routine on small inputs that reach the 128- and 256-bit
 * paths: real and complex, op N/T/C, scaling widths 1..100, zeros,
 * subnormals, huge and non-finite values, sampled and full entry lists. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_gemm_entries(int cplx, char transa, char transb, int64_t m, int64_t n, int64_t k, const double* alpha,
                     const double* A, int64_t lda, const double* B, int64_t ldb, const double* beta,
                     const double* C, int64_t ldc, int t, int64_t ns, const int64_t* rows, const int64_t* cols,
                     double* out, uint64_t* chat, int32_t* D, int32_t* E, uint8_t* flags, int nthreads);
int orc_encode_vectors(int cplx, char op, int is_b, int64_t k, int64_t nvec, const double* X, int64_t ld, int t,
                       int s, const int32_t* moduli, int32_t* D, uint8_t* flags, int64_t* hat, int8_t* planes,
                       void* unused);
void orc_residues_i256(int64_t count, const uint64_t* vals, int s, const int32_t* moduli, uint8_t* out);

static uint64_t state = 88172645463325252ull;
static uint64_t next_u64(void) { /* xorshift64 */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1.0p-53 * 2.0 - 1.0; }

static double value(int kind) {
    switch (kind % 8) {
        case 0: return 0.0;
        case 1: return -0.0;
        case 2: return uniform() * 0x1.0p-1060;         /* subnormal */
        case 3: return uniform() * 0x1.0p+1000;         /* huge */
        case 4: return uniform() * 0x1.0p-1000;         /* tiny normal */
        default: return uniform() * exp(6.0 * uniform());
    }
}

int main(void) {
    static const int32_t mods[24] = {256, 253, 251, 249, 247, 245, 241, 239, 233, 229, 227, 223,
                                     217, 211, 199, 197, 193, 191, 181, 179, 173, 167, 163, 157};
    const int ts[] = {1, 20, 55, 61, 62, 85, 100};
    const char ops[] = {'N', 'T', 'C'};
    int fails = 0;
    for (int rep = 0; rep < 60; ++rep) {
        const int cplx = rep % 3 == 2;
        const int64_t m = 1 + (int64_t)(next_u64() % 7), n = 1 + (int64_t)(next_u64() % 6),
                      k = 1 + (int64_t)(next_u64() % 9);
        const char ta = ops[next_u64() % (cplx ? 3 : 2)], tb = ops[next_u64() % (cplx ? 3 : 2)];
        const int t = ts[rep % 7];
        const int w = cplx ? 2 : 1;
        const int64_t ra = ta == 'N' ? m : k, ca = ta == 'N' ? k : m;
        const int64_t rb = tb == 'N' ? k : n, cb = tb == 'N' ? n : k;
        const int64_t lda = ra + rep % 3, ldb = rb + rep % 2, ldc = m + 1;
        double* A = malloc(sizeof(double) * w * lda * ca);
        double* B = malloc(sizeof(double) * w * ldb * cb);
        double* C = malloc(sizeof(double) * w * ldc * n);
        for (int64_t x = 0; x < w * lda * ca; ++x) A[x] = rep % 5 == 0 ? value((int)(next_u64() % 8)) : uniform();
        for (int64_t x = 0; x < w * ldb * cb; ++x) B[x] = rep % 5 == 1 ? value((int)(next_u64() % 8)) : uniform();
        for (int64_t x = 0; x < w * ldc * n; ++x) C[x] = uniform();
        if (rep % 11 == 3) A[0] = INFINITY;
        if (rep % 13 == 4) B[w * ldb * cb - 1] = NAN;
        const double al[2] = {uniform(), uniform()}, be[2] = {rep % 4 ? uniform() : 0.0, uniform()};
        /* every entry, then a sampled list with repeats */
        const int64_t ns = m * n;
        int64_t* rows = malloc(sizeof(int64_t) * (ns + 5));
        int64_t* cols = malloc(sizeof(int64_t) * (ns + 5));
        for (int64_t q = 0; q < ns; ++q) rows[q] = q % m, cols[q] = q / m;
        for (int64_t q = ns; q < ns + 5; ++q) rows[q] = (int64_t)(next_u64() % m), cols[q] = (int64_t)(next_u64() % n);
        double* out = malloc(sizeof(double) * w * (ns + 5));
        uint64_t* chat = malloc(sizeof(uint64_t) * 4 * w * (ns + 5));
        int32_t* D = malloc(sizeof(int32_t) * (ns + 5));
        int32_t* E = malloc(sizeof(int32_t) * (ns + 5));
        uint8_t* fl = malloc(ns + 5);
        fails += orc_gemm_entries(cplx, ta, tb, m, n, k, al, A, lda, B, ldb, be, C, ldc, t, ns + 5, rows, cols, out,
                                  chat, D, E, fl, 1) != 0;
        /* residues of the exact products, and encoded vectors */
        const int s = 2 + rep % 23;
        uint8_t* res = malloc((size_t)s * (ns + 5) * w);
        orc_residues_i256((ns + 5) * w, chat, s, mods, res);
        const int64_t nvec = m;
        int32_t* Dv = malloc(sizeof(int32_t) * nvec);
        uint8_t* fv = malloc(nvec);
        int64_t* hat = malloc(sizeof(int64_t) * 2 * 2 * nvec * k);
        int8_t* planes = malloc((size_t)(cplx ? 3 : 1) * s * nvec * k);
        fails += orc_encode_vectors(cplx, ta, 0, k, nvec, A, lda, t, s, mods, Dv, fv, hat, planes, NULL) != 0;
        free(A), free(B), free(C), free(rows), free(cols), free(out), free(chat), free(D), free(E), free(fl);
        free(res), free(Dv), free(fv), free(hat), free(planes);
    }
    printf("oracle driver: %d failing calls\n", fails);
    return fails != 0;
}
