// oz2_kernels.hip -- memory-bound phases of Ozaki scheme II on gfx950:
// row/column exponent scan, exact residue encoder, CRT reconstruction with
// the alpha/beta epilogue.
//
// Method: "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc
// GPUs: Ozaki Scheme II on the Xe2 Architecture":
//   Sec. 4.1  D_i = t - e(max_p |a_ip|)            -> scan + scale_of()
//   Sec. 2.3  a_hat = rint(a 2^D), ties to even     -> make_limbs()
//   Sec. 4.2  residues from the byte limbs of a_hat + 2^62 (the page uses
//             21-bit limbs) with precomputed 2^(8 l) mod m and
//             K_m = (h_m - 2^62) mod m, four limbs per v_dot4_u32_u8; no
//             FP64 and no branches in the loop over the moduli (a_hat itself
//             is formed once per element by exact full-rate FP64 operations)
//                                                  -> encode_kernel
//   Sec. 4.4  q = rint(sum r_t y_t/m_t), estimated in 16.16 fixed point
//             (sum r_t round(2^16 y_t/m_t) by v_dot2, within 0.05 of Z/M;
//             the page sums FP32 products, either is exact under its 1/4
//             margin), c_hat = sum r_t W_t - q M in 16-bit limbs, one carry
//             pass, top 64 bits + sticky rounded once to double, times
//             2^(-D_i-E_j)                         -> reconstruct_kernel
//   Sec. 5    ZGEMM: residues of re, im and re+im; Re and Im reconstructed
//   Sec. 8.1  non-finite row/column -> NaN row/column
// Compiled with -ffp-contract=off: the alpha/beta epilogue is evaluated
// exactly as written, every operation rounded separately.
#include "oz2_device.h"
#include "oz2_internal.h"

namespace oz2 {
namespace {

using namespace dev;

// ------------------------------------------------------------------ fill
__global__ void fill_u64_kernel(uint64_t* p, int64_t n, uint64_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ------------------------------------------------------------------ scan
// |x| as the bit pattern of a double (monotone in |x|, Inf < NaN) of both
// halves of a 16-byte pair
__device__ __forceinline__ uint64_t abs_bits2(double2 v) { return max(abs_bits(v.x), abs_bits(v.y)); }

typedef double nd2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ double2 load_stream(const double2* p) {
    const nd2 v = __builtin_nontemporal_load((const nd2*)p);
    return double2(v.x, v.y);
}

// One wavefront per vector whose elements are contiguous.  VEC: the vector
// starts 16-byte aligned (wave-uniform: the host checks the base and the
// leading dimension), so lanes read 16-byte pairs, four in flight each.
template <bool CPLX, bool VEC>
__global__ __launch_bounds__(256) void scan_contig_kernel(ScanParams P) {
    const int lane = threadIdx.x & 63;
    const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (v >= P.nvec) return;
    constexpr int W = CPLX ? 2 : 1;
    const int64_t len = P.k * W;
    const double* x = P.X + v * P.ld * W;
    uint64_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    if (VEC) {
        const double2* x2 = (const double2*)x;
        const int64_t len2 = len >> 1;
        int64_t p = lane;
        for (; p + 192 < len2; p += 256) {
            const double2 a = load_stream(x2 + p), b = load_stream(x2 + p + 64);
            const double2 c = load_stream(x2 + p + 128), d = load_stream(x2 + p + 192);
            m0 = max(m0, abs_bits2(a));
            m1 = max(m1, abs_bits2(b));
            m2 = max(m2, abs_bits2(c));
            m3 = max(m3, abs_bits2(d));
        }
        for (; p < len2; p += 64) m0 = max(m0, abs_bits2(load_stream(x2 + p)));
        if ((len & 1) && lane == 0) m1 = max(m1, abs_bits(x[len - 1]));
    } else {
        int64_t p = lane;
        for (; p + 192 < len; p += 256) {
            m0 = max(m0, abs_bits(x[p]));
            m1 = max(m1, abs_bits(x[p + 64]));
            m2 = max(m2, abs_bits(x[p + 128]));
            m3 = max(m3, abs_bits(x[p + 192]));
        }
        for (; p < len; p += 64) m0 = max(m0, abs_bits(x[p]));
    }
    unsigned long long mx = max(max(m0, m1), max(m2, m3));
    for (int off = 32; off >= 1; off >>= 1) {
        unsigned long long o = __shfl_xor(mx, off);
        mx = mx > o ? mx : o;
    }
    if (lane == 0) P.amax[v] = mx;
}

// Vectors whose elements are strided: a wavefront reads consecutive vectors
// at one position p, coalesced.  Real data with an even leading dimension
// and a 16-byte aligned base (VEC) gives each thread two neighbouring
// vectors as one 16-byte pair; otherwise one vector (complex: one 16-byte
// element).  The p range is split across blocks and combined with an atomic
// max on the zero-filled output; four positions are loaded per trip.
template <bool CPLX, bool VEC>
__global__ __launch_bounds__(256) void scan_strided_kernel(ScanParams P) {
    constexpr int VPT = (VEC && !CPLX) ? 2 : 1;  // vectors per thread
    const int64_t v = ((int64_t)blockIdx.x * 256 + threadIdx.x) * VPT;
    if (v >= P.nvec) return;
    const int64_t p0 = (int64_t)blockIdx.y * P.pchunk;
    const int64_t p1 = min(P.k, p0 + P.pchunk);
    uint64_t mx = 0, my = 0;
    if (CPLX && VEC) {
        // one complex element per load: 16 bytes, aligned with the base
        const double2* z = (const double2*)P.X + v;
        int64_t p = p0;
        for (; p + 3 < p1; p += 4) {
            const double2 a = z[p * P.ld], b = z[(p + 1) * P.ld], c = z[(p + 2) * P.ld], d = z[(p + 3) * P.ld];
            mx = max(mx, max(max(abs_bits2(a), abs_bits2(b)), max(abs_bits2(c), abs_bits2(d))));
        }
        for (; p < p1; ++p) mx = max(mx, abs_bits2(z[p * P.ld]));
    } else if (CPLX) {
        for (int64_t p = p0; p < p1; ++p) {
            const double* z = P.X + 2 * (v + p * P.ld);
            mx = max(mx, max(abs_bits(z[0]), abs_bits(z[1])));
        }
    } else if (VEC) {
        // v is even, ld even and the base 16-byte aligned: X + v + p ld is too
        const double* x = P.X + v;
        int64_t p = p0;
        for (; p + 3 < p1; p += 4) {
            const double2 a = load_stream((const double2*)(x + p * P.ld));
            const double2 b = load_stream((const double2*)(x + (p + 1) * P.ld));
            const double2 c = load_stream((const double2*)(x + (p + 2) * P.ld));
            const double2 d = load_stream((const double2*)(x + (p + 3) * P.ld));
            mx = max(mx, max(max(abs_bits(a.x), abs_bits(b.x)), max(abs_bits(c.x), abs_bits(d.x))));
            my = max(my, max(max(abs_bits(a.y), abs_bits(b.y)), max(abs_bits(c.y), abs_bits(d.y))));
        }
        for (; p < p1; ++p) {
            const double2 a = load_stream((const double2*)(x + p * P.ld));
            mx = max(mx, abs_bits(a.x));
            my = max(my, abs_bits(a.y));
        }
    } else {
        const double* x = P.X + v;
        int64_t p = p0;
        for (; p + 3 < p1; p += 4)
            mx = max(mx, max(max(abs_bits(x[p * P.ld]), abs_bits(x[(p + 1) * P.ld])),
                             max(abs_bits(x[(p + 2) * P.ld]), abs_bits(x[(p + 3) * P.ld]))));
        for (; p < p1; ++p) mx = max(mx, abs_bits(x[p * P.ld]));
    }
    if (mx) atomicMax((unsigned long long*)&P.amax[v], (unsigned long long)mx);
    if (VEC && !CPLX && my && v + 1 < P.nvec) atomicMax((unsigned long long*)&P.amax[v + 1], (unsigned long long)my);
}

// ---------------------------------------------------------------- encode
// A block encodes a tile of TV vectors x 64 k-positions.  Every thread owns
// groups of 4 consecutive k-positions of one vector, so that each modulus
// costs one 32-bit store per group; a wavefront writes 4 rows x 64 bytes of
// each plane, 256 contiguous bytes of one k-panel.  Strided operands are transposed through LDS first.
template <bool CONTIG, bool CPLX>
struct EncodeTile {
    // strided tiles are half as tall: their LDS transpose buffer (TV x 65
    // doubles per part) then allows eight wavefronts per SIMD
    static constexpr int TV = CONTIG ? (CPLX ? 32 : 64) : (CPLX ? 16 : 32);  // vectors per tile
    static constexpr int TP = kPanelK;          // k positions per tile: one panel
    static constexpr int GROUPS = TV * TP / 4;  // 4-element groups
    static constexpr int PER_THREAD = GROUPS / 256;
    static_assert(PER_THREAD >= 1 && PER_THREAD * 256 == GROUPS, "tile/thread mismatch");
};

template <bool CONTIG, bool CPLX, bool EXT>
__global__ __launch_bounds__(256) void encode_kernel(EncodeParams P) {
    using T = EncodeTile<CONTIG, CPLX>;
    const int tid = threadIdx.x;
    const int64_t tiles_p = P.kpad / T::TP;
    const int64_t tp = blockIdx.x % tiles_p;
    const int64_t tv = blockIdx.x / tiles_p;
    const int64_t v0 = tv * T::TV, p0 = tp * T::TP;
    constexpr int W = CPLX ? 2 : 1;

    // strided operands: transpose the tile through LDS (re and im planes)
    __shared__ double tile[CONTIG ? 1 : W][CONTIG ? 1 : T::TV][CONTIG ? 1 : T::TP + 1];
    if (!CONTIG) {
        constexpr int ROWS_PER_PASS = 256 / T::TV;
#pragma unroll
        for (int j = 0; j < T::TP / ROWS_PER_PASS; ++j) {
            const int v = tid % T::TV;
            const int p = tid / T::TV + ROWS_PER_PASS * j;
            const int64_t gv = v0 + v, gp = p0 + p;
            double re = 0.0, im = 0.0;
            if (gv < P.nvec && gp < P.k) {
                const double* src = P.X + W * (gv + gp * P.ld);
                re = src[0];
                if (CPLX) im = src[1];
            }
            tile[0][v][p] = re;
            if (CPLX) tile[W - 1][v][p] = im;
        }
        __syncthreads();
    }

    const int64_t plane = P.vpad * P.kpad;
#pragma unroll
    for (int g = 0; g < T::PER_THREAD; ++g) {
        const int grp = tid + 256 * g;
        const int v = grp / (T::TP / 4);
        const int p4 = (grp % (T::TP / 4)) * 4;
        const int64_t gv = v0 + v;
        double xr[4], xi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (CONTIG) {
                const int64_t gp = p0 + p4 + e;
                xr[e] = 0.0;
                xi[e] = 0.0;
                if (gv < P.nvec && gp < P.k) {
                    const double* src = P.X + W * (gv * P.ld + gp);
                    xr[e] = src[0];
                    if (CPLX) xi[e] = src[1];
                }
            } else {
                xr[e] = tile[0][v][p4 + e];
                xi[e] = CPLX ? tile[W - 1][v][p4 + e] : 0.0;
            }
            if (CPLX && P.conj) xi[e] = -xi[e];
        }
        bool bad;
        const int D = scale_of(gv < P.nvec ? P.amax[gv] : 0ull, P.t, bad);
        Limbs<EXT> lr[4], li[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lr[e] = make_limbs<EXT>(xr[e], D, bad);
            if (CPLX) li[e] = make_limbs<EXT>(xi[e], D, bad);
        }
        // k-panel layout: panel p0 / 64, row gv, byte p4
        int8_t* dst = P.planes + (p0 / kPanelK) * P.vpad * kPanelK + gv * kPanelK + p4;
        // the first modulus is 256 (the plan guarantees it): its plane is
        // the low byte of a_hat; then four moduli per trip, whose constants
        // are fetched together
        if (!CPLX) {
            *(uint32_t*)dst = low_byte_word<EXT>(lr);
        } else {
            // re, im, and re + im: the last as a bytewise sum mod 256 (the low
            // seven bits of each byte add without reaching the next byte)
            const uint32_t wr = low_byte_word<EXT>(lr), wi = low_byte_word<EXT>(li);
            *(uint32_t*)dst = wr;
            *(uint32_t*)(dst + P.set_stride) = wi;
            *(uint32_t*)(dst + 2 * P.set_stride) = ((wr & 0x7f7f7f7fu) + (wi & 0x7f7f7f7fu)) ^ ((wr ^ wi) & 0x80808080u);
        }
        for (int t0 = 1; t0 < P.s; t0 += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int t = t0 + u;
            if (t >= P.s) break;
            if (!CPLX) {
                *(uint32_t*)(dst + t * plane) =
                    residue_word<EXT>(lr, P.K[t] + 128u, P.c[t], (float)P.mod[t], P.frcp[t], P.foffb[t]);
            } else {
                uint32_t wr, wi, ws;
                residue_words3<EXT>(lr, li, P.K[t] + 128u, P.c[t], (float)P.mod[t], P.frcp[t], P.foffb[t], wr, wi,
                                    ws);
                *(uint32_t*)(dst + t * plane) = wr;
                *(uint32_t*)(dst + P.set_stride + t * plane) = wi;
                *(uint32_t*)(dst + 2 * P.set_stride + t * plane) = ws;
            }
          }
        }
    }
}

// ------------------------------------------------------------ reconstruct
// bytewise (a + b) mod m of four residues in [0, m)
__device__ __forceinline__ uint32_t add_mod_bytes(uint32_t a, uint32_t b, uint32_t m) {
    uint32_t out = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t x = ((a >> (8 * e)) & 0xffu) + ((b >> (8 * e)) & 0xffu);
        const uint32_t x1 = x - m;
        out |= (x < x1 ? x : x1) << (8 * e);
    }
    return out;
}

typedef double v2d __attribute__((ext_vector_type(2)));

// A wavefront reconstructs 256 consecutive rows of one column (mp is a
// multiple of 256), 4 entries per lane; the column index is wave-uniform.
template <int NL, bool CPLX, bool BETA>
__global__ __launch_bounds__(256) void reconstruct_kernel(ReconParams P) {
    const uint32_t waves_per_col = (uint32_t)(P.mp / 256);
    const uint32_t wid = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t jw = wid / waves_per_col;
    const int64_t j = jw;
    const int64_t i0 = (int64_t)(wid - jw * waves_per_col) * 256 + (threadIdx.x & 63) * 4;
    if (j >= P.n || i0 >= P.m) return;

    Crt<NL> acc[CPLX ? 2 : 1][4];
#pragma unroll
    for (int o = 0; o < (CPLX ? 2 : 1); ++o)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[o][e].init();

    const int64_t plane = P.n * P.mp;
    const uint8_t* src = P.R + j * P.mp + i0;
    // the residue words of 4 entries for every modulus (k runs summed mod m_t,
    // Arc page Sec. 4.3), all loads issued before any arithmetic; s <= 4 NL
    constexpr int SMAX = 4 * NL;
#pragma unroll
    for (int o = 0; o < (CPLX ? 2 : 1); ++o) {
        uint32_t rw[SMAX];
#pragma unroll
        for (int t = 0; t < SMAX; ++t) {
            rw[t] = 0u;
            if (t < P.s) rw[t] = *(const uint32_t*)(src + o * P.r_set_stride + t * plane);
        }
        for (int c = 1; c < P.chunks; ++c) {
#pragma unroll
            for (int t = 0; t < SMAX; ++t)
                if (t < P.s)
                    rw[t] = add_mod_bytes(rw[t], *(const uint32_t*)(src + o * P.r_set_stride + t * plane +
                                                                     c * P.r_chunk_stride),
                                          P.mod[t]);
        }
#pragma unroll
        for (int t = 0; t < SMAX; t += 2) {
            if (t < P.s) {
                const uint32_t Y2 = P.Y2[t >> 1];
                const uint32_t* W2 = P.W2[t >> 1];
                const uint32_t wa = rw[t], wb = rw[t + 1];
                // entry e: byte e of wa in bits 0-7, byte e of wb in bits 16-23
                acc[o][0].add2(__builtin_amdgcn_perm(wb, wa, 0x0c040c00u), Y2, W2);
                acc[o][1].add2(__builtin_amdgcn_perm(wb, wa, 0x0c050c01u), Y2, W2);
                acc[o][2].add2(__builtin_amdgcn_perm(wb, wa, 0x0c060c02u), Y2, W2);
                acc[o][3].add2(__builtin_amdgcn_perm(wb, wa, 0x0c070c03u), Y2, W2);
            }
        }
    }

    bool badB;
    const int E = scale_of(P.amaxB[j], P.t, badB);
    // the four entries' results (rows past m are computed from padding and
    // not stored: amaxA has mp entries)
    double x[4][2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i0 + e;
        bool badA;
        const int D = scale_of(P.amaxA[i], P.t, badA);
#pragma unroll
        for (int o = 0; o < (CPLX ? 2 : 1); ++o) {
            uint32_t w[NL];
            acc[o][e].finish(P.M16, w);
            if (P.chat && i < P.m) {
                uint32_t* dst = P.chat + (((int64_t)o * P.n + j) * P.mp + i) * NL;
#pragma unroll
                for (int q = 0; q < NL; ++q) dst[q] = w[q];
            }
            x[e][o] = words_to_double<NL>(w, D + E);
            if (badA || badB) x[e][o] = __builtin_nan("");
        }
    }
    // alpha / beta epilogue, every operation rounded separately
    double out[4][2];
    double* c0 = P.C + (CPLX ? 2 : 1) * (i0 + j * P.ldc);
    const bool full = i0 + 3 < P.m;
    // the lane's four entries are 32 (complex: 64) contiguous bytes: 16-byte
    // stores when they are 16-byte aligned (wave-uniform: depends on j)
    const bool vec = full && (((uintptr_t)c0 & 15u) == 0);
    // beta != 0: the lane's entries of C, read with the same 16-byte loads
    // when aligned (entry e, part o at cin[e][o])
    double cin[4][2] = {};
    if (BETA) {
        if (vec) {
            const v2d* src = (const v2d*)c0;
#pragma unroll
            for (int q = 0; q < (CPLX ? 4 : 2); ++q) {
                const v2d v = src[q];
                if (CPLX) {
                    cin[q][0] = v.x;
                    cin[q][1] = v.y;
                } else {
                    cin[2 * q][0] = v.x;
                    cin[2 * q + 1][0] = v.y;
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (i0 + e >= P.m) break;
                const double* c = c0 + (CPLX ? 2 : 1) * e;
                cin[e][0] = c[0];
                if (CPLX) cin[e][1] = c[1];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (!vec && i0 + e >= P.m) break;
        if (!CPLX) {
            const double t1 = P.alpha[0] * x[e][0];
            if (BETA) {
                const double t2 = P.beta[0] * cin[e][0];
                out[e][0] = t1 + t2;
            } else {
                out[e][0] = t1;
            }
        } else {
            const double ar = P.alpha[0], ai = P.alpha[1];
            const double t1 = ar * x[e][0], t2 = ai * x[e][1];
            const double ure = t1 - t2;
            const double t3 = ar * x[e][1], t4 = ai * x[e][0];
            const double uim = t3 + t4;
            if (BETA) {
                const double br = P.beta[0], bi = P.beta[1];
                const double cr = cin[e][0], ci = cin[e][1];
                const double t5 = br * cr, t6 = bi * ci;
                const double vre = t5 - t6;
                const double t7 = br * ci, t8 = bi * cr;
                const double vim = t7 + t8;
                out[e][0] = ure + vre;
                out[e][1] = uim + vim;
            } else {
                out[e][0] = ure;
                out[e][1] = uim;
            }
        }
    }
    if (vec) {
        v2d* d = (v2d*)c0;
        if (!CPLX) {
            d[0] = v2d{out[0][0], out[1][0]};
            d[1] = v2d{out[2][0], out[3][0]};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] = v2d{out[e][0], out[e][1]};
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (i0 + e >= P.m) break;
            double* c = c0 + (CPLX ? 2 : 1) * e;
            c[0] = out[e][0];
            if (CPLX) c[1] = out[e][1];
        }
    }
}

template <int NL>
__global__ __launch_bounds__(256) void crt_test_kernel(CrtTestParams P) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= P.count) return;
    Crt<NL> acc;
    acc.init();
    for (int t = 0; t < P.s; t += 2)
        acc.add2(P.R[t * P.count + q], t + 1 < P.s ? P.R[(t + 1) * P.count + q] : 0u, P.Y2[t >> 1],
                 P.W2[t >> 1]);
    uint32_t w[NL];
    acc.finish(P.M16, w);
#pragma unroll
    for (int i = 0; i < NL; ++i) P.words[q * NL + i] = w[i];
}

// C <- beta C (BLAS quick return for alpha = 0 or k = 0); C not read if beta = 0
template <bool CPLX>
__global__ __launch_bounds__(256) void scale_c_kernel(double* C, int64_t m, int64_t n, int64_t ldc,
                                                      double br, double bi) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= m * n) return;
    const int64_t i = gid % m, j = gid / m;
    double* c = C + (CPLX ? 2 : 1) * (i + j * ldc);
    const bool zero = (br == 0.0 && bi == 0.0);
    if (!CPLX) {
        c[0] = zero ? 0.0 : br * c[0];
    } else if (zero) {
        c[0] = 0.0;
        c[1] = 0.0;
    } else {
        const double cr = c[0], ci = c[1];
        const double t3 = br * cr, t4 = bi * ci;
        const double t5 = br * ci, t6 = bi * cr;
        c[0] = t3 - t4;
        c[1] = t5 + t6;
    }
}

int64_t blocks_for(int64_t n, int64_t per) { return (n + per - 1) / per; }

}  // namespace

// ------------------------------------------------------------- launchers
hipError_t launch_fill_u64(uint64_t* p, int64_t n, uint64_t value, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t nb = blocks_for(n, 256);
    if (nb > 4096) nb = 4096;
    hipLaunchKernelGGL(fill_u64_kernel, dim3((unsigned)nb), dim3(256), 0, st, p, n, value);
    return hipGetLastError();
}

hipError_t launch_scan(const ScanParams& P, bool contiguous, bool cplx, hipStream_t st) {
    if (P.nvec <= 0 || P.k <= 0) return hipSuccess;
    const bool aligned = ((uintptr_t)P.X & 15) == 0;
    if (contiguous) {
        // 16-byte pairs when every vector starts 16-byte aligned
        const bool vec = aligned && (cplx || (P.ld & 1) == 0);
        dim3 grid((unsigned)blocks_for(P.nvec, 4));
        if (cplx && vec)
            hipLaunchKernelGGL((scan_contig_kernel<true, true>), grid, dim3(256), 0, st, P);
        else if (cplx)
            hipLaunchKernelGGL((scan_contig_kernel<true, false>), grid, dim3(256), 0, st, P);
        else if (vec)
            hipLaunchKernelGGL((scan_contig_kernel<false, true>), grid, dim3(256), 0, st, P);
        else
            hipLaunchKernelGGL((scan_contig_kernel<false, false>), grid, dim3(256), 0, st, P);
    } else {
        const bool vec = aligned && (cplx || (P.ld & 1) == 0);
        const int64_t per_block = (vec && !cplx) ? 512 : 256;
        dim3 grid((unsigned)blocks_for(P.nvec, per_block), (unsigned)blocks_for(P.k, P.pchunk));
        if (cplx && vec)
            hipLaunchKernelGGL((scan_strided_kernel<true, true>), grid, dim3(256), 0, st, P);
        else if (cplx)
            hipLaunchKernelGGL((scan_strided_kernel<true, false>), grid, dim3(256), 0, st, P);
        else if (vec)
            hipLaunchKernelGGL((scan_strided_kernel<false, true>), grid, dim3(256), 0, st, P);
        else
            hipLaunchKernelGGL((scan_strided_kernel<false, false>), grid, dim3(256), 0, st, P);
    }
    return hipGetLastError();
}

template <bool CONTIG, bool CPLX, bool EXT>
static hipError_t encode_go(const EncodeParams& P, hipStream_t st) {
    using T = EncodeTile<CONTIG, CPLX>;
    const int64_t nb = (P.vpad / T::TV) * (P.kpad / T::TP);
    hipLaunchKernelGGL((encode_kernel<CONTIG, CPLX, EXT>), dim3((unsigned)nb), dim3(256), 0, st, P);
    return hipGetLastError();
}

hipError_t launch_encode(const EncodeParams& P, bool contiguous, bool cplx, bool ext,
                         hipStream_t st) {
    if (P.vpad % 64 || P.kpad % 64) return hipErrorInvalidValue;
    const int idx = (contiguous ? 4 : 0) | (cplx ? 2 : 0) | (ext ? 1 : 0);
    switch (idx) {
        case 0: return encode_go<false, false, false>(P, st);
        case 1: return encode_go<false, false, true>(P, st);
        case 2: return encode_go<false, true, false>(P, st);
        case 3: return encode_go<false, true, true>(P, st);
        case 4: return encode_go<true, false, false>(P, st);
        case 5: return encode_go<true, false, true>(P, st);
        case 6: return encode_go<true, true, false>(P, st);
        default: return encode_go<true, true, true>(P, st);
    }
}

template <int NL>
static hipError_t recon_go(const ReconParams& P, bool cplx, bool beta, hipStream_t st) {
    const int64_t nb = blocks_for((P.mp / 256) * P.n, 4);  // one wavefront per 256 rows of a column
    dim3 g((unsigned)nb), b(256);
    if (cplx) {
        if (beta) hipLaunchKernelGGL((reconstruct_kernel<NL, true, true>), g, b, 0, st, P);
        else hipLaunchKernelGGL((reconstruct_kernel<NL, true, false>), g, b, 0, st, P);
    } else {
        if (beta) hipLaunchKernelGGL((reconstruct_kernel<NL, false, true>), g, b, 0, st, P);
        else hipLaunchKernelGGL((reconstruct_kernel<NL, false, false>), g, b, 0, st, P);
    }
    return hipGetLastError();
}

hipError_t launch_reconstruct(const ReconParams& P, int NL, bool cplx, bool beta_nonzero,
                              hipStream_t st) {
    // wave indices are 32-bit
    if (P.mp % 256 || (P.mp / 256) * P.n > (int64_t)UINT32_MAX - 4) return hipErrorInvalidValue;
    switch (NL) {
        case 2: return recon_go<2>(P, cplx, beta_nonzero, st);
        case 3: return recon_go<3>(P, cplx, beta_nonzero, st);
        case 4: return recon_go<4>(P, cplx, beta_nonzero, st);
        case 5: return recon_go<5>(P, cplx, beta_nonzero, st);
        case 6: return recon_go<6>(P, cplx, beta_nonzero, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_scale_c(double* C, int64_t m, int64_t n, int64_t ldc, const double beta[2],
                          bool cplx, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    dim3 g((unsigned)blocks_for(m * n, 256));
    if (cplx)
        hipLaunchKernelGGL(scale_c_kernel<true>, g, dim3(256), 0, st, C, m, n, ldc, beta[0], beta[1]);
    else
        hipLaunchKernelGGL(scale_c_kernel<false>, g, dim3(256), 0, st, C, m, n, ldc, beta[0], 0.0);
    return hipGetLastError();
}

hipError_t launch_crt_test(const CrtTestParams& P, int NL, hipStream_t st) {
    if (P.count <= 0) return hipSuccess;
    dim3 g((unsigned)blocks_for(P.count, 256));
    switch (NL) {
        case 2: hipLaunchKernelGGL(crt_test_kernel<2>, g, dim3(256), 0, st, P); break;
        case 3: hipLaunchKernelGGL(crt_test_kernel<3>, g, dim3(256), 0, st, P); break;
        case 4: hipLaunchKernelGGL(crt_test_kernel<4>, g, dim3(256), 0, st, P); break;
        case 5: hipLaunchKernelGGL(crt_test_kernel<5>, g, dim3(256), 0, st, P); break;
        case 6: hipLaunchKernelGGL(crt_test_kernel<6>, g, dim3(256), 0, st, P); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace oz2
