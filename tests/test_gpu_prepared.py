"""GPU parity of prepared operands (oz2_operand_create / _update /
oz2_gemm_prepared) through the C ABI.

A prepared operand holds exactly what the scan and encode phases of one
oz2_dgemm / oz2_zgemm call compute for that operand, so a product from
prepared operands must be bitwise the product of the plain call on the same
data (the Arc page's reuse of A's residues across calls, Sec. 10; the chain
page's cached operator residues, Algorithm 6).  The plain call is itself
checked against the oracle elsewhere; here one case per kind is also checked
against the oracle directly.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_float_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oz2mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    return oz2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


REAL_CASES = [
    # m, n, k, transa, transb, s, beta
    (300, 200, 700, "N", "N", 8, 0.0),
    (257, 129, 1000, "T", "N", 16, -0.5),
    (64, 300, 40, "N", "T", 12, 0.0),
    (48, 33, 17, "T", "T", 6, 1.0),      # k <= 32, m <= 64: dgemm takes the fused path
    (513, 511, 2049, "T", "T", 20, 0.25),  # extended-width residues
    (70, 90, 140001, "N", "N", 8, 0.0),  # two k runs
]


@pytest.mark.parametrize("m,n,k,ta,tb,s,beta", REAL_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4]}s{c[5]}" for c in REAL_CASES])
def test_prepared_dgemm_bitwise(oz2mod, m, n, k, ta, tb, s, beta):
    import torch
    _say(f"[prepared dgemm] {m}x{n}x{k} {ta}{tb} s={s}")
    ra, ca = workloads.stored_shape(ta, m, k)
    rb, cb = workloads.stored_shape(tb, k, n)
    A = workloads.real_matrix(ra, ca, 7100 + m, "phi", 1.0)
    B = workloads.real_matrix(rb, cb, 7200 + n, "phi", 1.0)
    C = workloads.real_matrix(m, n, 7300 + k % 1000, "uniform")
    dA, dB = to_dev(A), to_dev(B)
    with oz2mod.Handle() as h:
        ref = to_dev(C)
        h.dgemm(ta, tb, m, n, k, 1.25, dA, ra, dB, rb, beta, ref, m, s)
        pa = h.prepare("A", ta, m, k, dA, ra, s)
        pb = h.prepare("B", tb, n, k, dB, rb, s)
        got = to_dev(C)
        h.gemm_prepared(pa, pb, 1.25, beta, got, m)
        torch.cuda.synchronize()
        g, r = from_dev(got), from_dev(ref)
        assert np.array_equal(g.view(np.int64), r.view(np.int64)), f"{int(np.sum(g != r))} entries differ"
        if k <= 2049:
            want = oracle.gemm_entries(False, ta, tb, m, n, k, 1.25, A, ra, B, rb, beta, C, m, s)["out"]
            check_float_parity(g, want, "prepared vs oracle")
        pa.close()
        pb.close()


def test_prepared_zgemm_bitwise(oz2mod):
    import torch
    m, n, k, s = 130, 70, 300, 16
    _say(f"[prepared zgemm] {m}x{n}x{k} C/N s={s}")
    A = workloads.complex_matrix(k, m, 7401, 7402, "phi", 0.5)  # stored k x m, op C
    B = workloads.complex_matrix(k, n, 7403, 7404, "phi", 0.5)
    C = workloads.complex_matrix(m, n, 7405, 7406, "uniform")
    alpha, beta = complex(0.7, -0.3), complex(0.2, 0.1)
    dA, dB = to_dev(A), to_dev(B)
    with oz2mod.Handle() as h:
        ref = to_dev(C)
        h.zgemm("C", "N", m, n, k, alpha, dA, k, dB, k, beta, ref, m, s)
        with h.prepare("A", "C", m, k, dA, k, s, cplx=True) as pa, \
                h.prepare("B", "N", n, k, dB, k, s, cplx=True) as pb:
            got = to_dev(C)
            h.gemm_prepared(pa, pb, alpha, beta, got, m)
            torch.cuda.synchronize()
        g, r = from_dev(got), from_dev(ref)
        assert np.array_equal(g.view(np.int64), r.view(np.int64))
        want = oracle.gemm_entries(True, "C", "N", m, n, k, alpha, A, k, B, k, beta, C, m, s)["out"]
        check_float_parity(g, want, "prepared zgemm vs oracle")


def test_prepared_a_reused_across_calls(oz2mod):
    """One op(A) prepared once; three different B re-encoded into one
    prepared op(B) in turn: each product equals the plain call."""
    import torch
    m, n, k, s = 384, 256, 1536, 12
    _say(f"[prepared reuse] {m}x{n}x{k} s={s}")
    A = workloads.real_matrix(m, k, 7501, "phi", 0.5)
    dA = to_dev(A)
    with oz2mod.Handle() as h:
        pa = h.prepare("A", "N", m, k, dA, m, s)
        pb = None
        for q in range(3):
            B = workloads.real_matrix(n, k, 7510 + q, "phi", 2.0)  # stored n x k, op T
            dB = to_dev(B)
            if pb is None:
                pb = h.prepare("B", "T", n, k, dB, n, s)
            else:
                h.update(pb, dB, n)
            got = torch.zeros(m * n, dtype=torch.float64, device="cuda")
            ref = torch.zeros_like(got)
            h.gemm_prepared(pa, pb, 1.0, 0.0, got, m)
            h.dgemm("N", "T", m, n, k, 1.0, dA, m, dB, n, 0.0, ref, m, s)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int64), ref.view(torch.int64)), q
        pa.close()
        pb.close()


def test_prepared_argument_errors(oz2mod):
    import ctypes
    import torch
    lib = oz2mod.lib()
    A = to_dev(workloads.real_matrix(64, 64, 7601))
    with oz2mod.Handle() as h:
        pa = h.prepare("A", "N", 64, 64, A, 64, 8)
        pb8 = h.prepare("B", "N", 64, 64, A, 64, 8)
        pb12 = h.prepare("B", "N", 64, 64, A, 64, 12)
        pbk = h.prepare("B", "N", 64, 32, A, 64, 8)
        C = torch.zeros(64 * 64, dtype=torch.float64, device="cuda")
        al = (ctypes.c_double * 2)(1.0, 0.0)
        cp = ctypes.c_void_p(C.data_ptr())
        assert lib.oz2_gemm_prepared(h._h, pb8._p, pb8._p, al, al, cp, 64) == -2   # pa is a B side
        assert lib.oz2_gemm_prepared(h._h, pa._p, pa._p, al, al, cp, 64) == -3    # pb is an A side
        assert lib.oz2_gemm_prepared(h._h, pa._p, pb12._p, al, al, cp, 64) == -3  # s differs
        assert lib.oz2_gemm_prepared(h._h, pa._p, pbk._p, al, al, cp, 64) == -3   # k differs
        assert lib.oz2_gemm_prepared(h._h, pa._p, pb8._p, al, al, cp, 63) == -7   # ldc < m
        assert lib.oz2_gemm_prepared(h._h, pa._p, pb8._p, al, al, cp, 64) == 0
        out = ctypes.c_void_p()
        xp = ctypes.c_void_p(A.data_ptr())
        assert lib.oz2_operand_create(h._h, b"X", 0, b"N", 64, 64, xp, 64, 8, ctypes.byref(out)) == -2
        assert lib.oz2_operand_create(h._h, b"A", 0, b"Q", 64, 64, xp, 64, 8, ctypes.byref(out)) == -4
        assert lib.oz2_operand_create(h._h, b"A", 0, b"N", 64, 64, xp, 63, 8, ctypes.byref(out)) == -8
        assert lib.oz2_operand_create(h._h, b"A", 0, b"N", 64, 64, xp, 64, 25, ctypes.byref(out)) == -9
        assert not out.value
        assert lib.oz2_operand_update(h._h, pa._p, xp, 63) == -4
        torch.cuda.synchronize()
        for op in (pa, pb8, pb12, pbk):
            op.close()
