"""GPU parity of oz2_dgemm against the CPU oracle, through the C ABI.

Bar (from the method's statement): residue planes, per-modulus product
residues and the reconstructed integer c_hat are bit-exact; the FP64 output
is within 1 ulp per entry (bit-identical except possibly subnormal results,
which the Arc page allows to be rounded twice, Sec. 4.4).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (check_chat, check_float_parity, check_product_residues,
                            check_residue_planes, from_dev, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    h = oz2.Handle()
    h.set_debug(True)
    yield h
    h.close()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_full(handle, transa, transb, m, n, k, alpha, beta, s, A, lda, B, ldb, C, ldc,
              check_internals=True, label=""):
    import torch
    _say(f"[dgemm] {label} {transa}{transb} m={m} n={n} k={k} s={s}")
    dA, dB = to_dev(A), to_dev(B)
    dC = to_dev(C if C is not None else np.zeros(ldc * n))
    handle.dgemm(transa, transb, m, n, k, alpha, dA, lda, dB, ldb, beta, dC, ldc, s)
    torch.cuda.synchronize()
    got = from_dev(dC).reshape(n, ldc)[:, :m].T
    r = oracle.gemm_entries(False, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta,
                            C, ldc, s)
    want = r["out"].reshape(n, m).T
    nonident = check_float_parity(got, want, label)
    if check_internals and alpha != 0 and k > 0:
        t = oracle.scaling_width(s, k)
        encA = oracle.encode_vectors(False, transa, False, k, m, A, lda, s, t)
        encB = oracle.encode_vectors(False, transb, True, k, n, B, ldb, s, t)
        check_residue_planes(handle.debug_copy(2), encA, m, k, label + " A planes")
        check_residue_planes(handle.debug_copy(3), encB, n, k, label + " B planes")
        check_product_residues(handle.debug_copy(4), r["chat_words"], s, m, n, 0, label)
        words = handle.debug_copy(5)
        rows = [q % m for q in range(m * n)]
        cols = [q // m for q in range(m * n)]
        check_chat(words, r["chat"], rows, cols, 0, label)
    # leading-dimension padding of C untouched
    full = from_dev(dC).reshape(n, ldc)
    if ldc > m and C is not None:
        assert np.array_equal(np.isnan(full[:, m:]), np.isnan(C.reshape(n, ldc)[:, m:]))
    return nonident


def test_config1_full_parity(handle):
    # 256^3, s = 8, N/N, alpha = 1, beta = 0, U(-1,1)
    w = workloads.WORKLOADS[1]
    m, n, k = w["m"], w["n"], w["k"]
    A = workloads.real_matrix(m, k, workloads.seed(1, 0))
    B = workloads.real_matrix(k, n, workloads.seed(1, 1))
    nonident = _run_full(handle, "N", "N", m, n, k, 1.0, 0.0, 8, A, m, B, k, None, m,
                         label="config1")
    assert nonident == 0


CASES = [
    # m, n, k, transa, transb, s, dist
    (300, 77, 130, "N", "N", 8, "uniform"),
    (300, 77, 130, "T", "N", 13, "phi"),
    (77, 300, 130, "N", "T", 16, "phi"),
    (129, 65, 200, "T", "T", 2, "uniform"),
    (257, 513, 65, "C", "N", 24, "phi"),
    (1, 1, 1, "N", "N", 5, "uniform"),
    (5, 3, 700, "T", "N", 19, "phi"),
    (520, 9, 64, "N", "C", 12, "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4]}s{c[5]}" for c in CASES])
def test_ragged_shapes_ops_alpha_beta(handle, case):
    m, n, k, ta, tb, s, dist = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    ra, ca = (m, k) if ta == "N" else (k, m)
    rb, cb = (k, n) if tb == "N" else (n, k)
    lda, ldb, ldc = ra + 3, rb + 1, m + 2
    A = workloads.real_matrix(ra, ca, int(rng.integers(1 << 30)), dist, 2.0, ld=lda)
    B = workloads.real_matrix(rb, cb, int(rng.integers(1 << 30)), dist, 2.0, ld=ldb)
    C = workloads.real_matrix(m, n, int(rng.integers(1 << 30)), "uniform", ld=ldc)
    alpha, beta = float(rng.normal()), float(rng.normal())
    _run_full(handle, ta, tb, m, n, k, alpha, beta, s, A, lda, B, ldb, C, ldc, label=str(case))


def test_nonfinite_rows_and_columns(handle):
    m, n, k = 40, 30, 50
    rng = np.random.default_rng(5)
    A = rng.uniform(-1, 1, m * k)
    B = rng.uniform(-1, 1, k * n)
    A[3 + 7 * m] = np.inf
    A[10 + 2 * m] = -np.inf
    B[5 + 4 * k] = np.nan
    C = rng.uniform(-1, 1, m * n)
    _run_full(handle, "N", "N", m, n, k, 1.0, 0.5, 16, A, m, B, k, C, m, label="nonfinite")


def test_quick_returns(handle):
    import torch
    m, n, k = 20, 10, 30
    rng = np.random.default_rng(6)
    A = rng.uniform(-1, 1, m * k)
    B = rng.uniform(-1, 1, k * n)
    C = rng.uniform(-1, 1, m * n)
    # alpha = 0: C <- beta C, A and B not read (NaN in A does not propagate)
    A2 = A.copy()
    A2[0] = np.nan
    _run_full(handle, "N", "N", m, n, k, 0.0, 0.25, 8, A2, m, B, k, C, m, check_internals=False,
              label="alpha0")
    # beta = 0: C is not read (NaN in C does not propagate)
    Cn = np.full(m * n, np.nan)
    _run_full(handle, "N", "N", m, n, k, 1.0, 0.0, 8, A, m, B, k, Cn, m, label="beta0")
    # k = 0
    dC = to_dev(C)
    handle.dgemm("N", "N", m, n, 0, 1.0, to_dev(A), m, to_dev(B), 1, 2.0, dC, m, 8)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(dC), 2.0 * C)


def test_k_split_runs(handle):
    # k beyond one exact INT32 run (Arc page Sec. 4.3): split runs must give
    # the same c_hat as the oracle's unsplit exact product
    m, n = 9, 7
    for k in (130816, 131071, 131072, 140001):
        A = workloads.real_matrix(m, k, workloads.seed(77, 0) + k, "phi", 1.0)
        B = workloads.real_matrix(k, n, workloads.seed(77, 1) + k, "phi", 1.0)
        _run_full(handle, "N", "N", m, n, k, 1.0, 0.0, 16, A, m, B, k, None, m, label=f"ksplit{k}")
        runs = handle.debug_copy(4).shape[0]
        assert runs == (1 if k <= 130816 else 2)


def test_crt_boundary_one_minus_ulp(handle):
    # Arc page Sec. 8.3: all entries 1 - 2^-53 reach |c_hat| close to M/4; exact for all s
    for s, k in ((8, 64), (16, 4096), (24, 100)):
        m = n = 8
        a = 1.0 - 2.0 ** -53
        A = np.full(m * k, a)
        B = np.full(k * n, a)
        _run_full(handle, "N", "N", m, n, k, 1.0, 0.0, s, A, m, B, k, None, m, label=f"1-u s{s}")


def test_integer_inputs_exact(handle):
    import torch
    rng = np.random.default_rng(8)
    m, n, k = 33, 17, 45
    Ai = rng.integers(-2 ** 12, 2 ** 12, size=(m, k))
    Bi = rng.integers(-2 ** 12, 2 ** 12, size=(k, n))
    A = Ai.astype(np.float64).reshape(-1, order="F")
    B = Bi.astype(np.float64).reshape(-1, order="F")
    dC = to_dev(np.zeros(m * n))
    handle.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.0, dC, m, 10)
    torch.cuda.synchronize()
    got = from_dev(dC).reshape(n, m).T
    assert np.array_equal(got, (Ai @ Bi).astype(np.float64))


@pytest.mark.parametrize("s", range(2, 25))
def test_crt_hook_random_exact_integers(handle, s):
    # the Arc page's CRT unit test (Sec. 8.1): exact integers |c| <= M/4,
    # including +-M/4, reconstructed from residues in [0, m_t)
    import torch
    from tests.gpu_util import words_to_int
    mods = oracle.max_product_moduli(s)
    M = oracle.moduli_product(mods)
    vals = [0, 1, -1, M // 4, -(M // 4), M // 4 - 1, -(M // 4) + 1]
    import random
    rr = random.Random(s)
    vals += [rr.randint(-(M // 4), M // 4) for _ in range(2000)]
    small = min(2 ** 20, M // 4)
    vals += [rr.randint(-small, small) for _ in range(100)]
    count = len(vals)
    res = np.array([[v % mt for v in vals] for mt in mods], dtype=np.uint8)
    nl = oracle.n_limbs(s)
    dres = to_dev(res)
    words = torch.zeros(count * nl, dtype=torch.int32, device="cuda")
    handle.test_crt(dres, s, words)
    torch.cuda.synchronize()
    w = from_dev(words).view(np.uint32).reshape(count, nl)
    for q, v in enumerate(vals):
        assert words_to_int(w[q]) == v, (s, q, v)


@pytest.mark.parametrize("m,n,k,ldc", [(300, 77, 130, 300), (300, 77, 130, 301), (16, 200, 16, 18)],
                         ids=["four-phase-ldc-even", "four-phase-ldc-odd", "fused-k16"])
def test_c_base_only_8_byte_aligned(handle, m, n, k, ldc):
    # C starting one double into its allocation: the 16-byte store path of
    # the reconstruct and fused kernels must fall back to 8-byte stores
    import torch
    rng = np.random.default_rng(m * 7 + ldc)
    A = workloads.real_matrix(m, k, int(rng.integers(1 << 30)), "phi", 1.0)
    B = workloads.real_matrix(k, n, int(rng.integers(1 << 30)), "phi", 1.0)
    C = workloads.real_matrix(ldc, n, int(rng.integers(1 << 30)), "uniform")
    buf = np.concatenate([[7.0], C, [9.0]])
    dbuf = to_dev(buf)
    dC = dbuf[1:1 + ldc * n]
    assert dC.data_ptr() % 16 == 8
    _say(f"[dgemm] C base +8 bytes m={m} n={n} k={k} ldc={ldc}")
    handle.set_debug(False)  # this module runs in debug mode, which bypasses the fused path
    try:
        handle.dgemm("N", "N", m, n, k, -0.5, to_dev(A), m, to_dev(B), k, 1.25, dC, ldc, 12)
        torch.cuda.synchronize()
    finally:
        handle.set_debug(True)
    got = from_dev(dbuf)
    assert got[0] == 7.0 and got[-1] == 9.0
    full = got[1:-1].reshape(n, ldc)
    want = oracle.gemm_entries(False, "N", "N", m, n, k, -0.5, A, m, B, k, 1.25, C, ldc, 12)["out"]
    check_float_parity(full[:, :m].T, want.reshape(n, m).T, f"C+8 {m}x{n}x{k} ldc={ldc}")
    assert np.array_equal(full[:, m:], C.reshape(n, ldc)[:, m:])


@pytest.mark.parametrize("cplx", [False, True])
@pytest.mark.parametrize("ta,tb", [("N", "N"), ("T", "T")])
def test_operands_only_8_byte_aligned(handle, cplx, ta, tb):
    # A and B starting one double into their allocations (and even leading
    # dimensions): the scan's 16-byte-pair paths must not be taken, and the
    # results must match the oracle
    import torch
    m, n, k, s = 300, 260, 200, 16
    ra, ca = workloads.stored_shape(ta, m, k)
    rb, cb = workloads.stored_shape(tb, k, n)
    rng = np.random.default_rng(9 + 2 * int(cplx) + (ta == "T"))
    sd = [int(x) for x in rng.integers(1 << 30, size=4)]
    if cplx:
        A = workloads.complex_matrix(ra, ca, sd[0], sd[1], "phi", 1.0)
        B = workloads.complex_matrix(rb, cb, sd[2], sd[3], "phi", 1.0)
    else:
        A = workloads.real_matrix(ra, ca, sd[0], "phi", 1.0)
        B = workloads.real_matrix(rb, cb, sd[2], "phi", 1.0)
    _say(f"[dgemm] operands +8 bytes cplx={cplx} {ta}{tb}")
    if cplx:
        # complex operands from the raw C ABI with 8-byte-offset pointers
        import ctypes
        import complex_gemm_emulation_amd as oz2
        bufA = to_dev(np.concatenate([[0.0], A.view(np.float64)]))
        bufB = to_dev(np.concatenate([[0.0], B.view(np.float64)]))
        dC = torch.zeros(m * n, dtype=torch.complex128, device="cuda")
        al = (ctypes.c_double * 2)(1.0, 0.0)
        be = (ctypes.c_double * 2)(0.0, 0.0)
        handle._bind_stream()
        st = oz2.lib().oz2_zgemm(handle._h, ta.encode(), tb.encode(), m, n, k, al,
                                 ctypes.c_void_p(bufA.data_ptr() + 8), ra, ctypes.c_void_p(bufB.data_ptr() + 8), rb,
                                 be, ctypes.c_void_p(dC.data_ptr()), m, s)
        assert st == 0
        torch.cuda.synchronize()
        got = from_dev(dC)
    else:
        bufA = to_dev(np.concatenate([[0.0], A]))
        bufB = to_dev(np.concatenate([[0.0], B]))
        dC = to_dev(np.zeros(m * n))
        dA, dB = bufA[1:], bufB[1:]
        assert dA.data_ptr() % 16 == 8 and dB.data_ptr() % 16 == 8
        handle.dgemm(ta, tb, m, n, k, 1.0, dA, ra, dB, rb, 0.0, dC, m, s)
        torch.cuda.synchronize()
        got = from_dev(dC)
    want = oracle.gemm_entries(cplx, ta, tb, m, n, k, 1.0, A, ra, B, rb, 0.0, None, m, s, chat_ints=False)["out"]
    assert check_float_parity(got, want, "operands +8 bytes") == 0
