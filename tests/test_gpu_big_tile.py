"""Bit-exact parity of the 256 x 256 residue GEMM tile, the one the large
products run on, against the CPU oracle through the C ABI.

The library takes the 256 x 256 four-stage tile only when the grid holds at
least 512 such blocks over all moduli and the k-loop of a launch is longer
than 512 positions; every case here is sized to meet both conditions.  Each
case compares what the method fixes exactly: residue planes, per-modulus
product residues (Arc page Sec. 2.3 step 3; EmuGEMM page Sec. IV-A for the
fused mod-m epilogue), the reconstructed integer c_hat (Arc page Sec. 4.4),
and the FP64 output bit for bit.  The k-split case follows Arc page Sec. 4.3
(runs of exact INT32 accumulation summed before the CRT), and the last cases
cover the block order used when the tile count is not a multiple of 8.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (check_chat_words, check_float_parity, check_product_residues,
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


def _pad(x, q=256):
    return (x + q - 1) // q * q


def _selects_big_tile(m, n, k, s, run_k=None):
    """The launch condition of the 256 x 256 tile, from the sizes alone."""
    kk = _pad(k if run_k is None else run_k)
    return (_pad(m) // 256) * (_pad(n) // 256) * s >= 512 and kk > 512


def _real_case(handle, transa, transb, m, n, k, s, ldc, alpha, beta, seed_base, planes=True):
    import torch
    assert _selects_big_tile(m, n, k, s)
    ra, ca = workloads.stored_shape(transa, m, k)
    rb, cb = workloads.stored_shape(transb, k, n)
    A = workloads.real_matrix(ra, ca, seed_base, "phi", 1.0)
    B = workloads.real_matrix(rb, cb, seed_base + 1, "phi", 1.0)
    C = workloads.real_matrix(m, n, seed_base + 2, "uniform", ld=ldc)
    _say(f"[big-tile] dgemm {transa}{transb} m={m} n={n} k={k} s={s} ldc={ldc}")
    dC = to_dev(C)
    handle.dgemm(transa, transb, m, n, k, alpha, to_dev(A), ra, to_dev(B), rb, beta, dC, ldc, s)
    torch.cuda.synchronize()
    full = from_dev(dC).reshape(n, ldc)
    got = full[:, :m].T
    _say("[big-tile]   oracle over every entry")
    r = oracle.gemm_entries(False, transa, transb, m, n, k, alpha, A, ra, B, rb, beta, C, ldc, s,
                            chat_ints=False)
    want = r["out"].reshape(n, m).T
    assert check_float_parity(got, want, "output") == 0
    assert np.array_equal(np.isnan(full[:, m:]), np.isnan(C.reshape(n, ldc)[:, m:]))
    check_product_residues(handle.debug_copy(4), r["chat_words"], s, m, n, 0, "residues")
    check_chat_words(handle.debug_copy(5), r["chat_words"], m, 0, label="c_hat")
    if planes:
        t = oracle.scaling_width(s, k)
        check_residue_planes(handle.debug_copy(2), oracle.encode_vectors(False, transa, False, k, m, A, ra, s, t),
                             m, k, "A planes")
        check_residue_planes(handle.debug_copy(3), oracle.encode_vectors(False, transb, True, k, n, B, rb, s, t),
                             n, k, "B planes")


def test_big_tile_dgemm_ragged_ldc_beta(handle):
    # 8 x 9 tiles x 8 moduli = 576 blocks, k = 1280: op(B) transposed, ldc ragged, beta != 0
    _real_case(handle, "N", "T", 2048, 2304, 1280, 8, 2048 + 5, -0.75, 1.25, workloads.seed(20, 0))


@pytest.mark.parametrize("s", [24, 23])
def test_big_tile_block_order_fallback(handle, s):
    # 5 x 5 = 25 tiles per modulus, not a multiple of 8: the block order falls
    # back to the per-XCD contiguous ranges (600 blocks, a multiple of 8) or
    # to the plain order (575 blocks); extended-width residues at these s
    _real_case(handle, "T", "N", 1280, 1280, 1024, s, 1280, 1.5, -0.5, workloads.seed(21, s), planes=False)


def test_big_tile_zgemm_3m_conj(handle):
    # ZGEMM C/N, 8 x 4 tiles x 16 moduli = 512 blocks, k = 640 (768 padded):
    # Re and Im residues of the fused 3M kernel and both c_hat words
    import torch
    m, n, k, s = 2048, 1024, 640, 16
    assert _selects_big_tile(m, n, k, s)
    sd = workloads.seed(22, 0)
    A = workloads.complex_matrix(k, m, sd, sd + 3, "phi", 0.5)
    B = workloads.complex_matrix(k, n, sd + 1, sd + 4, "phi", 0.5)
    C = workloads.complex_matrix(m, n, sd + 2, sd + 5)
    al, be = complex(0.7, -0.3), complex(0.2, 0.1)
    _say(f"[big-tile] zgemm CN m={m} n={n} k={k} s={s}")
    dC = to_dev(C.copy())
    handle.zgemm("C", "N", m, n, k, al, to_dev(A), k, to_dev(B), k, be, dC, m, s)
    torch.cuda.synchronize()
    got = from_dev(dC).reshape(n, m).T
    r = oracle.gemm_entries(True, "C", "N", m, n, k, al, A, k, B, k, be, C, m, s, chat_ints=False)
    want = r["out"].reshape(n, m).T
    assert check_float_parity(got, want, "zgemm output") == 0
    res = handle.debug_copy(4)
    words = handle.debug_copy(5)
    for out, name in ((0, "Re"), (1, "Im")):
        check_product_residues(res, r["chat_words"], s, m, n, out, f"{name} residues")
        check_chat_words(words, r["chat_words"], m, out, label=f"{name} c_hat")


def test_big_tile_k_split(handle):
    # k = 131330: a run of 130816 positions and one of 514 (768 padded), both
    # on the 256 x 256 tile; residues, c_hat and outputs at sampled entries
    import torch
    m = n = 2048
    k, s = 131330, 8
    assert _selects_big_tile(m, n, k, s, run_k=130816) and _selects_big_tile(m, n, k, s, run_k=k - 130816)
    A = workloads.real_matrix(m, k, workloads.seed(23, 0), "uniform")
    B = workloads.real_matrix(k, n, workloads.seed(23, 1), "uniform")
    _say(f"[big-tile] dgemm k-split m={m} n={n} k={k} s={s}")
    dC = to_dev(np.zeros(m * n))
    handle.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.0, dC, m, s)
    torch.cuda.synchronize()
    got = from_dev(dC).reshape(n, m).T
    res = handle.debug_copy(4)
    assert res.shape[0] == 2, "two exact runs expected"
    words = handle.debug_copy(5)
    rng = np.random.default_rng(23)
    rows = np.concatenate([[0, m - 1, 0, m - 1, 255, 256], rng.integers(0, m, 58)])
    cols = np.concatenate([[0, 0, n - 1, n - 1, 256, 255], rng.integers(0, n, 58)])
    r = oracle.gemm_entries(False, "N", "N", m, n, k, 1.0, A, m, B, k, 0.0, None, m, s,
                            rows=rows, cols=cols, chat_ints=False)
    assert check_float_parity(got[rows, cols], r["out"], "sampled outputs") == 0
    check_product_residues(res, r["chat_words"], s, m, n, 0, "sampled residues", rows=rows, cols=cols)
    check_chat_words(words, r["chat_words"], m, 0, rows=rows, cols=cols, label="sampled c_hat")
