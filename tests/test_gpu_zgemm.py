"""GPU parity of oz2_zgemm (exact integer 3M form) against the oracle's 4M
exact product, through the C ABI.  Arc page Sec. 5: Re = P0 - P1,
Im = P2 - P0 - P1 in exact integer arithmetic, so the reconstructed Re and Im
c_hat must equal the 4M integers bit for bit."""
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


def _run(handle, ta, tb, m, n, k, alpha, beta, s, A, lda, B, ldb, C, ldc, label):
    import torch
    print(f"[zgemm] {label} {ta}{tb} m={m} n={n} k={k} s={s}", flush=True)
    dC = to_dev(C if C is not None else np.zeros(ldc * n, dtype=np.complex128))
    handle.zgemm(ta, tb, m, n, k, alpha, to_dev(A), lda, to_dev(B), ldb, beta, dC, ldc, s)
    torch.cuda.synchronize()
    got = from_dev(dC).reshape(n, ldc)[:, :m].T
    r = oracle.gemm_entries(True, ta, tb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s)
    want = r["out"].reshape(n, m).T
    check_float_parity(got, want, label)
    if alpha != 0 and k > 0:
        t = oracle.scaling_width(s, k, True)
        encA = oracle.encode_vectors(True, ta, False, k, m, A, lda, s, t)
        encB = oracle.encode_vectors(True, tb, True, k, n, B, ldb, s, t)
        check_residue_planes(handle.debug_copy(2), encA, m, k, label + " A planes")
        check_residue_planes(handle.debug_copy(3), encB, n, k, label + " B planes")
        res = handle.debug_copy(4)
        for o in range(2):
            check_product_residues(res, r["chat_words"], s, m, n, o, f"{label} out{o}")
        words = handle.debug_copy(5)
        rows = [q % m for q in range(m * n)]
        cols = [q // m for q in range(m * n)]
        for o in range(2):
            check_chat(words, r["chat"], rows, cols, o, f"{label} out{o}")


CASES = [
    (64, 48, 96, "N", "N", 16, "uniform"),
    (130, 70, 100, "C", "N", 16, "phi"),
    (70, 130, 100, "N", "C", 8, "phi"),
    (33, 65, 257, "T", "C", 20, "phi"),
    (257, 3, 40, "C", "T", 24, "uniform"),
    (1, 1, 1, "C", "C", 2, "uniform"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4]}s{c[5]}" for c in CASES])
def test_zgemm_ops_alpha_beta(handle, case):
    m, n, k, ta, tb, s, dist = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    ra, ca = (m, k) if ta == "N" else (k, m)
    rb, cb = (k, n) if tb == "N" else (n, k)
    lda, ldb, ldc = ra + 2, rb + 3, m + 1
    sd = [int(x) for x in rng.integers(1 << 30, size=6)]
    A = workloads.complex_matrix(ra, ca, sd[0], sd[1], dist, 1.0, ld=lda)
    B = workloads.complex_matrix(rb, cb, sd[2], sd[3], dist, 1.0, ld=ldb)
    C = workloads.complex_matrix(m, n, sd[4], sd[5], "uniform", ld=ldc)
    alpha = complex(rng.normal(), rng.normal())
    beta = complex(rng.normal(), rng.normal())
    _run(handle, ta, tb, m, n, k, alpha, beta, s, A, lda, B, ldb, C, ldc, str(case))


def test_zgemm_nonfinite_and_beta_zero(handle):
    m, n, k = 20, 12, 30
    rng = np.random.default_rng(44)
    A = rng.uniform(-1, 1, m * k) + 1j * rng.uniform(-1, 1, m * k)
    B = rng.uniform(-1, 1, k * n) + 1j * rng.uniform(-1, 1, k * n)
    A[4 + 3 * m] = complex(1.0, np.inf)
    B[2 + 5 * k] = complex(np.nan, 0.0)
    C = np.full(m * n, complex(np.nan, np.nan))
    _run(handle, "N", "N", m, n, k, complex(1.0, 0.5), 0.0, 16, A, m, B, k, C, m, "nonfinite")


def test_zgemm_3m_matches_4m_on_cancellation(handle):
    # real and imaginary parts of similar size: the integer 3M form loses
    # nothing (EmuGEMM page Sec. IV-B; Arc page Sec. 8.5)
    m, n, k = 48, 40, 64
    rng = np.random.default_rng(45)
    X = rng.uniform(-1, 1, (m, k // 2)) * (1 + 1j)
    Y = rng.uniform(-1, 1, (k // 2, n)) * (1 - 1j)
    Z = rng.uniform(-1, 1, (k // 2, n)) + 1j * rng.uniform(-1, 1, (k // 2, n))
    Am = np.concatenate([X, X], axis=1)
    Bm = np.concatenate([Y, -Y + 2.0 ** -30 * Z], axis=0)
    A = Am.reshape(-1, order="F")
    B = Bm.reshape(-1, order="F")
    _run(handle, "N", "N", m, n, k, 1.0, 0.0, 20, A, m, B, k, None, m, "cancel")
