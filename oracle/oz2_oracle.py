"""CPU oracle for Ozaki scheme II DGEMM/ZGEMM emulation -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product (``complex_gemm_emulation_amd``)
never imports, links or executes anything under ``oracle/``, and this module
shares no code, tables or constant generators with it.

Source pages (cited by title and section; nothing here is copied from them):

* [P1] "Emulating DGEMM and ZGEMM with INT8 Matrix Engines on Intel Arc GPUs:
  Ozaki Scheme II on the Xe2 Architecture" -- the method's authority
  (Sec. 2.1 notation, Sec. 2.3 the four steps, Sec. 4.1 scaling width and
  Table 2, Sec. 4.4 CRT, Sec. 4.5 Eq. (7), Sec. 5 ZGEMM, Sec. 8.1 tests,
  Sec. 8.3 worst cases, Sec. 9.1 precision policy).
* [P2] "You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode
  Products" -- Sec. 2.2 (Eq. 8-10 CRT form), Sec. 2.3 (Eq. 11-12 centred
  residues), Sec. 4.1 / Fig. 2 (worked example on the basis (7, 5, 3)).

What the oracle computes (its own reading of the pages, step by step):

1. moduli   -- the max-product set of ``s`` pairwise-coprime integers <= 256
               (P1 Sec. 2.3 step 2 and Table 2's log2 M column), found by an
               exhaustive branch-and-bound search below.
2. t        -- the largest t with k * 2**(2t) <= M/4 (real) or 2k * 2**(2t) <= M/4
               (complex), P1 Sec. 4.1 / Sec. 4.4 (|c_hat| <= M/4).
3. scaling  -- D_i = t - e(max_p |a_ip|), e(x) the frexp exponent (P1 Sec. 4.1).
4. a_hat    -- rint(a * 2**D), ties to even (P1 Sec. 2.3 step 1).
5. c_hat    -- the exact integer product of the integerized operands: no
               residues are involved (C part, ``oz2_oracle.c``).
6. output   -- c_hat * 2**(-D_i-E_j) rounded once to double, then alpha/beta.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against printed values of the pages (``tests/golden/``), closed forms, exact
rational arithmetic (``fractions.Fraction``) and brute force; see each test.
The pages give no evaluation order for alpha/beta.  The epilogue is pinned
without one: every output must lie within the rounding bound of separately
rounded products and sums around the exact rational alpha*x + beta*c
(``test_alpha_beta_epilogue_vs_exact_rationals``), which any sign, swap or
conjugation mistake breaks.  Bitwise parity with the product additionally
rests on both sides using the same order.
"""
from __future__ import annotations

import ctypes
import functools
import math
import os
from fractions import Fraction
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboz2_oracle.so")

MAX_MODULUS = 256          # P1 Sec. 2.3 step 2: moduli m_t <= 256
MIN_S, MAX_S = 2, 24       # P1 Sec. 1 contributions / Sec. 9.3: 2 <= s <= 24


# ----------------------------------------------------------------------------
# 1. moduli: max-product set of s pairwise-coprime integers <= 256
# ----------------------------------------------------------------------------
def _primes_upto(n: int) -> list[int]:
    return [p for p in range(2, n + 1) if all(p % q for q in range(2, int(p ** 0.5) + 1))]


@functools.lru_cache(maxsize=None)
def max_product_moduli(s: int) -> tuple[int, ...]:
    """The s pairwise-coprime integers in [2, 256] with the largest product.

    P1 Sec. 2.3 step 2 asks for pairwise coprime moduli <= 256 and Table 2
    prints log2 M per s; the reading adopted is the set of maximal product.
    Ties (equal products) are broken towards the lexicographically largest
    descending sequence, which is what a depth-first search over descending
    candidates that only accepts strictly larger products returns first.
    Returned in descending order (256 first).
    """
    if not (MIN_S <= s <= MAX_S):
        raise ValueError("s must be in [2, 24]")
    primes = _primes_upto(MAX_MODULUS)
    cands = list(range(MAX_MODULUS, 1, -1))
    masks = []
    for c in cands:
        mk = 0
        for bit, p in enumerate(primes):
            if c % p == 0:
                mk |= 1 << bit
        masks.append(mk)
    n = len(cands)
    best = [0, None]
    chosen: list[int] = []

    def dfs(start: int, prod: int, used: int) -> None:
        r = s - len(chosen)
        if r == 0:
            if prod > best[0]:
                best[0], best[1] = prod, tuple(chosen)
            return
        # upper bound: the next r candidates coprime with the chosen ones
        ub, cnt = prod, 0
        for idx in range(start, n):
            if masks[idx] & used == 0:
                ub *= cands[idx]
                cnt += 1
                if cnt == r:
                    break
        if cnt < r or ub <= best[0]:
            return
        for idx in range(start, n):
            c = cands[idx]
            if prod * c ** r <= best[0]:
                break
            if masks[idx] & used == 0:
                chosen.append(c)
                dfs(idx + 1, prod * c, used | masks[idx])
                chosen.pop()

    dfs(0, 1, 0)
    return best[1]


def moduli_product(moduli: Sequence[int]) -> int:
    return math.prod(moduli)


def log2_M(s: int) -> float:
    return math.log2(moduli_product(max_product_moduli(s)))


def n_limbs(s: int) -> int:
    """N_L, the number of 32-bit words holding c_hat in two's complement.

    P1 Sec. 4.4 gives floor(log2 M / 32) + 1; its Table 2 prints 2 for s=4
    (log2 M = 31.9), so the reading is max(2, floor(log2 M / 32) + 1).
    """
    return max(2, int(math.floor(log2_M(s) / 32.0)) + 1)


# ----------------------------------------------------------------------------
# 2. scaling width t(s, k)
# ----------------------------------------------------------------------------
def scaling_width(s: int, k: int, is_complex: bool = False) -> int:
    """Largest integer t with k' * 4**t <= M/4, k' = k (real) or 2k (complex).

    |a_hat|, |b_hat| <= 2**t (P1 Sec. 2.3 step 1) bound |c_hat| by k' * 4**t,
    and the FP32-quotient CRT needs |c_hat| <= M/4 (P1 Sec. 4.4).  Compared
    exactly in integers.  Returns 0 or less when no t >= 1 exists.
    """
    M = moduli_product(max_product_moduli(s))
    kk = max(int(k), 1) * (2 if is_complex else 1)
    t = 0
    while 4 * kk * 4 ** (t + 1) <= M:
        t += 1
    return t


def moduli_for_bits(k: int, bits: int = 53, is_complex: bool = False) -> int:
    """Default-precision policy of P1 Sec. 9.1: the smallest s in [2, 24]
    whose scaling width reaches ``bits``; 24 when none does."""
    for s in range(MIN_S, MAX_S + 1):
        if scaling_width(s, k, is_complex) >= bits:
            return s
    return MAX_S


# ----------------------------------------------------------------------------
# Scalar residue arithmetic (P1 Sec. 2.1 sym_m, Sec. 2.3 step 4;
# P2 Sec. 2.2 Eq. 9 and Sec. 2.3 Eq. 11-12)
# ----------------------------------------------------------------------------
def sym(v: int, m: int) -> int:
    """sym_m(v): representative of v mod m in the window [-h, m-1-h], h = floor((m-1)/2).

    This is the window P1 Sec. 4.2's offset h_m implies.  For odd m it is the
    centred interval of P2 Eq. 11-12; for m = 256 it is [-127, 128].
    """
    h = (m - 1) // 2
    r = v % m
    return r - m if r > m - 1 - h else r


def sym_byte(v: int, m: int) -> int:
    """sym_m(v) as the signed byte that is stored: 128 (only reachable for
    m = 256) is stored as -128, which is congruent mod 256."""
    r = sym(v, m)
    return r - 256 if r >= 128 else r


def crt_weights(moduli: Sequence[int]) -> list[int]:
    """W_t = M_t * (M_t^{-1} mod m_t) with M_t = M / m_t (P2 Eq. 9, P1 Sec. 2.3 step 4)."""
    M = moduli_product(moduli)
    out = []
    for m in moduli:
        Mt = M // m
        out.append(Mt * pow(Mt, -1, m))
    return out


def crt_reconstruct(residues: Sequence[int], moduli: Sequence[int]) -> int:
    """Centred CRT: the unique x in [-(M-1)//2, M//2] ... with x == r_t (mod m_t).

    P2 Eq. 9: sum_t r_t W_t mod M, then the centred representative; the
    result equals the intended integer whenever 2|x| < M.
    """
    M = moduli_product(moduli)
    z = sum(r * w for r, w in zip(residues, crt_weights(moduli))) % M
    return z - M if 2 * z > M else z


# ----------------------------------------------------------------------------
# Exact scalar helpers used by the tests' rational cross-checks
# ----------------------------------------------------------------------------
def frexp_exponent(x: float) -> int:
    """e(x): the e with 2**(e-1) <= |x| < 2**e (math.frexp), for x != 0."""
    return math.frexp(x)[1]


def exact_dot(a: Sequence[float], b: Sequence[float]) -> Fraction:
    """Exact value of sum_p a_p * b_p for finite doubles, as a Fraction.

    Every double is an integer multiple of 2**-1074, so the products are
    integers times 2**-2148 and are summed exactly in Python integers.
    """
    total = 0
    for x, y in zip(a, b):
        if x == 0.0 or y == 0.0:
            continue
        fx, ex = math.frexp(x)
        fy, ey = math.frexp(y)
        ix = int(fx * (1 << 53))
        iy = int(fy * (1 << 53))
        total += (ix * iy) << ((ex - 53) + (ey - 53) + 2300)
    return Fraction(total, 1 << 2300)


def fraction_to_double(q: Fraction) -> float:
    """Correctly rounded double of a rational (CPython's int/int division is
    correctly rounded); +-inf on overflow."""
    try:
        return q.numerator / q.denominator
    except OverflowError:
        return math.inf if q > 0 else -math.inf


# ----------------------------------------------------------------------------
# The C part: exact integer products and correctly rounded output
# ----------------------------------------------------------------------------
class _Lib:
    _lib = None

    @classmethod
    def get(cls):
        if cls._lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"oracle library missing: {LIB_PATH} (run __graft_entry__.build())")
            lib = ctypes.CDLL(LIB_PATH)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            I32 = ctypes.c_int
            C = ctypes.c_char
            lib.orc_gemm_entries.restype = I32
            lib.orc_gemm_entries.argtypes = [
                I32, C, C, I64, I64, I64, P, P, I64, P, I64, P, P, I64, I32,
                I64, P, P, P, P, P, P, P, I32]
            lib.orc_encode_vectors.restype = I32
            lib.orc_encode_vectors.argtypes = [
                I32, C, I32, I64, I64, P, I64, I32, I32, P, P, P, P, P, P]
            lib.orc_residues_i256.restype = None
            lib.orc_residues_i256.argtypes = [I64, P, I32, P, P]
            lib.orc_max_threads.restype = I32
            lib.orc_max_threads.argtypes = []
            cls._lib = lib
        return cls._lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


def _as_f64(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    if np.iscomplexobj(a):
        a = np.ascontiguousarray(a.astype(np.complex128)).view(np.float64)
    return np.ascontiguousarray(a, dtype=np.float64).reshape(-1)


def i256_to_int(words: np.ndarray) -> int:
    """Two's complement 256-bit value from 4 little-endian uint64 words."""
    v = 0
    for w in reversed([int(x) for x in words]):
        v = (v << 64) | w
    return v - (1 << 256) if v >> 255 else v


def max_threads() -> int:
    return int(_Lib.get().orc_max_threads())


def gemm_entries(is_complex: bool, transa: str, transb: str, m: int, n: int, k: int,
                 alpha, A, lda: int, B, ldb: int, beta, C, ldc: int, s: int,
                 rows=None, cols=None, nthreads: int = 0, chat_ints: bool = True) -> dict:
    """Oracle output of C <- alpha op(A) op(B) + beta C at the entries (rows[q], cols[q]).

    Matrices are column-major flat arrays (complex ones as complex128).  With
    rows/cols omitted every entry is computed (column-major order).  Returns
    dict(out=float64 or complex128 array, chat=list of exact integers (or
    (re, im) pairs), D, E, flags) where flags bit0/bit1 mark a non-finite
    row of op(A) / column of op(B) (P1 Sec. 8.1).  chat_ints=False skips the
    list of Python integers (chat is then None; chat_words still holds c_hat
    as 256-bit two's complement words), for calls over millions of entries.
    """
    lib = _Lib.get()
    if rows is None:
        jj, ii = np.meshgrid(np.arange(n), np.arange(m), indexing="ij")
        rows, cols = ii.reshape(-1), jj.reshape(-1)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    ns = rows.size
    ncomp = 2 if is_complex else 1
    t = scaling_width(s, k, is_complex)
    al = np.array([np.real(alpha), np.imag(alpha)] if is_complex else [float(alpha)], dtype=np.float64)
    be = np.array([np.real(beta), np.imag(beta)] if is_complex else [float(beta)], dtype=np.float64)
    Af, Bf = _as_f64(A), _as_f64(B)
    Cf = _as_f64(C) if C is not None else None
    out = np.zeros(ns * ncomp, dtype=np.float64)
    chat = np.zeros(ns * ncomp * 4, dtype=np.uint64)
    D = np.zeros(ns, dtype=np.int32)
    E = np.zeros(ns, dtype=np.int32)
    flags = np.zeros(ns, dtype=np.uint8)
    rc = lib.orc_gemm_entries(int(is_complex), transa.encode(), transb.encode(), m, n, k,
                              _ptr(al), _ptr(Af), lda, _ptr(Bf), ldb, _ptr(be), _ptr(Cf), ldc, t,
                              ns, _ptr(rows), _ptr(cols), _ptr(out), _ptr(chat), _ptr(D), _ptr(E),
                              _ptr(flags), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"orc_gemm_entries failed with {rc}")
    ch = chat.reshape(ns, ncomp, 4)
    outv = out.view(np.complex128) if is_complex else out
    if not chat_ints:
        chat_list = None
    elif is_complex:
        chat_list = [(i256_to_int(ch[q, 0]), i256_to_int(ch[q, 1])) for q in range(ns)]
    else:
        chat_list = [i256_to_int(ch[q, 0]) for q in range(ns)]
    return dict(out=outv, chat=chat_list, chat_words=ch, D=D, E=E, flags=flags, t=t)


def chat_residues(chat_words: np.ndarray, s: int) -> np.ndarray:
    """c_hat mod m_t in [0, m_t) for every modulus of the s-set: array [s, count]."""
    lib = _Lib.get()
    w = np.ascontiguousarray(chat_words, dtype=np.uint64).reshape(-1, 4)
    mods = np.array(max_product_moduli(s), dtype=np.int32)
    out = np.zeros((s, w.shape[0]), dtype=np.uint8)
    lib.orc_residues_i256(w.shape[0], _ptr(w), s, _ptr(mods), _ptr(out))
    return out


def encode_vectors(is_complex: bool, op: str, is_b: bool, k: int, nvec: int, X, ld: int,
                   s: int, t: int) -> dict:
    """Scaling exponents, flags, a_hat and the stored residue bytes of the
    vectors of op(A) (rows, is_b=False) or op(B) (columns, is_b=True).

    Returns dict(D[nvec], flags[nvec], hat_re[nvec,k] (python ints),
    planes[nsets, s, nvec, k] int8) where the sets are (re,) or
    (re, im, re+im) -- the last one is what the 3M product needs (P1 Sec. 5).
    """
    lib = _Lib.get()
    Xf = _as_f64(X)
    mods = np.array(max_product_moduli(s), dtype=np.int32)
    nsets = 3 if is_complex else 1
    D = np.zeros(nvec, dtype=np.int32)
    flags = np.zeros(nvec, dtype=np.uint8)
    hat = np.zeros((2 if is_complex else 1, nvec, k, 2), dtype=np.int64)
    planes = np.zeros((nsets, s, nvec, k), dtype=np.int8)
    rc = lib.orc_encode_vectors(int(is_complex), op.encode(), int(is_b), k, nvec, _ptr(Xf), ld, t, s,
                                _ptr(mods), _ptr(D), _ptr(flags), _ptr(hat), _ptr(planes), None)
    if rc != 0:
        raise RuntimeError(f"orc_encode_vectors failed with {rc}")
    return dict(D=D, flags=flags, hat=hat, planes=planes)


def hat_to_int(pair) -> int:
    lo, hi = int(pair[0]) & ((1 << 64) - 1), int(pair[1])
    return (hi << 64) | lo
