"""GPU parity of the fused short-k path (k <= 32 with one output dimension
<= 64, single products and strided batches) against the CPU oracle, through
the C ABI.  The same bar as the four-phase path: FP64 output within 1 ulp of
the oracle per entry (bit-identical away from subnormal results), and
bit-identical to the four-phase path on the same inputs.  The tensor-chain
cases follow the workload of "You Only Convert Twice: Ozaki Scheme II for
Chained Tensor Mode Products" (Sec. 2.1 Eq. (5), Sec. 5.1 OzII-Composed):
each mode is one emulated product whose row and column exponents are the
per-fiber and per-operator-row scales."""
import zlib

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_float_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    h = oz2.Handle()
    yield h
    h.close()


def _oracle_batched(ta, tb, m, n, k, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, batch, s):
    outs = []
    for b in range(batch):
        Cb = None if C is None else C[b * sC:]
        r = oracle.gemm_entries(False, ta, tb, m, n, k, alpha, A[b * sA:], lda, B[b * sB:], ldb,
                                beta, Cb, ldc, s)
        outs.append(r["out"].reshape(n, m))
    return outs


BATCH_CASES = [
    # m, n, k, ta, tb, s, batch, shareA, shareB, dist
    (16, 16, 16, "N", "T", 16, 7, False, True, "uniform"),
    (16, 16, 16, "N", "N", 8, 5, True, False, "phi"),
    (13, 9, 5, "T", "N", 12, 6, False, False, "phi"),
    (40, 3, 32, "N", "T", 20, 4, False, True, "phi"),
    (3, 70, 31, "T", "T", 24, 3, True, False, "phi"),
    (64, 64, 1, "N", "N", 2, 3, False, False, "uniform"),
    (17, 33, 17, "T", "N", 17, 5, False, False, "phi"),
    (256, 16, 16, "N", "T", 16, 3, False, True, "uniform"),
]


@pytest.mark.parametrize("case", BATCH_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4]}s{c[5]}b{c[6]}" for c in BATCH_CASES])
def test_strided_batched_fused(handle, case):
    import torch
    m, n, k, ta, tb, s, batch, shA, shB, dist = case
    print(f"[small batched] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    ra, ca = (m, k) if ta == "N" else (k, m)
    rb, cb = (k, n) if tb == "N" else (n, k)
    lda, ldb, ldc = ra + 1, rb + 2, m + 3
    sA = 0 if shA else lda * ca + 5
    sB = 0 if shB else ldb * cb + 3
    sC = ldc * n + 7
    A = workloads.real_matrix(lda, (sA if sA else lda * ca) * max(batch, 1) // lda + 1,
                              int(rng.integers(1 << 30)), dist, 2.0)
    B = workloads.real_matrix(ldb, (sB if sB else ldb * cb) * max(batch, 1) // ldb + 1,
                              int(rng.integers(1 << 30)), dist, 2.0)
    C = workloads.real_matrix(sC, batch, int(rng.integers(1 << 30)), "uniform")
    alpha, beta = float(rng.normal()), float(rng.normal())
    dC = to_dev(C)
    handle.dgemm_strided_batched(ta, tb, m, n, k, alpha, to_dev(A), lda, sA, to_dev(B), ldb, sB,
                                 beta, dC, ldc, sC, batch, s)
    torch.cuda.synchronize()
    got = from_dev(dC)
    want = _oracle_batched(ta, tb, m, n, k, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC,
                           batch, s)
    for b in range(batch):
        gb = got[b * sC: b * sC + ldc * n].reshape(n, ldc)[:, :m]
        check_float_parity(gb, want[b], f"{case} batch {b}")
        # padding rows of C untouched
        assert np.array_equal(got[b * sC: b * sC + ldc * n].reshape(n, ldc)[:, m:],
                              C[b * sC: b * sC + ldc * n].reshape(n, ldc)[:, m:])


SINGLE_CASES = [
    # m, n, k, ta, tb, s, beta
    (16, 3000, 16, "N", "N", 16, 0.0),
    (5000, 7, 9, "T", "N", 10, 0.5),
    (64, 1000, 32, "N", "T", 24, -1.0),
    (200, 64, 2, "T", "T", 5, 0.0),
]


@pytest.mark.parametrize("case", SINGLE_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}{c[4]}s{c[5]}" for c in SINGLE_CASES])
def test_dgemm_fused_matches_oracle_and_four_phase(handle, case):
    import torch
    m, n, k, ta, tb, s, beta = case
    print(f"[small single] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    ra, ca = (m, k) if ta == "N" else (k, m)
    rb, cb = (k, n) if tb == "N" else (n, k)
    A = workloads.real_matrix(ra, ca, int(rng.integers(1 << 30)), "phi", 1.5)
    B = workloads.real_matrix(rb, cb, int(rng.integers(1 << 30)), "phi", 1.5)
    C = workloads.real_matrix(m, n, int(rng.integers(1 << 30)), "uniform")
    dA, dB = to_dev(A), to_dev(B)
    outs = []
    for debug in (False, True):  # debug mode forces the four-phase path
        handle.set_debug(debug)
        dC = to_dev(C)
        handle.dgemm(ta, tb, m, n, k, 0.75, dA, ra, dB, rb, beta, dC, m, s)
        torch.cuda.synchronize()
        outs.append(from_dev(dC))
    handle.set_debug(False)
    assert np.array_equal(outs[0].view(np.uint64), outs[1].view(np.uint64)), "fused != four-phase"
    want = oracle.gemm_entries(False, ta, tb, m, n, k, 0.75, A, ra, B, rb, beta, C, m, s)["out"]
    check_float_parity(outs[0], want, str(case))


def test_fused_nonfinite_rows_columns(handle):
    import torch
    m, n, k = 20, 40, 12
    rng = np.random.default_rng(9)
    A = rng.uniform(-1, 1, m * k)
    B = rng.uniform(-1, 1, k * n)
    A[7 + 3 * m] = np.nan
    B[2 + 33 * k] = -np.inf
    C = rng.uniform(-1, 1, m * n)
    dC = to_dev(C)
    handle.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.25, dC, m, 16)
    torch.cuda.synchronize()
    got = from_dev(dC)
    want = oracle.gemm_entries(False, "N", "N", m, n, k, 1.0, A, m, B, k, 0.25, C, m, 16)["out"]
    check_float_parity(got, want, "fused nonfinite")
    g = got.reshape(n, m)
    assert np.isnan(g[:, 7]).all() and np.isnan(g[33, :]).all()


def _oracle_chain(Xb, Aop, Bop, Cop, n, s):
    """The three modes of one tensor with the oracle (same mode decomposition)."""
    n2 = n * n
    z1 = oracle.gemm_entries(False, "N", "N", n, n2, n, 1.0, Aop, n, Xb, n, 0.0, None, n, s)["out"]
    z2 = np.zeros(n * n2)
    for kk in range(n):
        sl = z1[kk * n2:(kk + 1) * n2]
        z2[kk * n2:(kk + 1) * n2] = oracle.gemm_entries(False, "N", "T", n, n, n, 1.0, sl, n, Bop, n,
                                                        0.0, None, n, s)["out"]
    return oracle.gemm_entries(False, "N", "T", n2, n, n, 1.0, z2, n2, Cop, n, 0.0, None, n2, s)["out"]


def _chain_inputs(n, batch):
    X = workloads.tensor_batch(n, batch, workloads.seed(5, 0))
    Aop = workloads.real_matrix(n, n, workloads.seed(5, 1))
    Bop = workloads.real_matrix(n, n, workloads.seed(5, 2))
    Cop = workloads.real_matrix(n, n, workloads.seed(5, 3))
    return X, Aop, Bop, Cop


def test_tensor_chain_small_batch_full_parity(handle):
    import torch
    n, batch, s = 16, 6, 16
    X, Aop, Bop, Cop = _chain_inputs(n, batch)
    Y = handle.tensor_mode_chain(to_dev(X), to_dev(Aop), to_dev(Bop), to_dev(Cop), n, batch, s)
    torch.cuda.synchronize()
    got = from_dev(Y)
    n3 = n ** 3
    for b in range(batch):
        want = _oracle_chain(X[b * n3:(b + 1) * n3], Aop, Bop, Cop, n, s)
        check_float_parity(got[b * n3:(b + 1) * n3], want, f"chain tensor {b}")


def test_tensor_chain_full_size_sampled(handle):
    # 32768 tensors of 16^3 (the benchmark's chain), tensors sampled across
    # the batch including the first and last, each checked against the oracle
    import torch
    w = workloads.WORKLOADS[5]
    n, batch, s = w["n"], w["batch"], w["s"][0]
    print(f"[chain full] n={n} batch={batch} s={s}", flush=True)
    X, Aop, Bop, Cop = _chain_inputs(n, batch)
    Y = handle.tensor_mode_chain(to_dev(X), to_dev(Aop), to_dev(Bop), to_dev(Cop), n, batch, s)
    torch.cuda.synchronize()
    got = from_dev(Y)
    n3 = n ** 3
    rng = np.random.default_rng(55)
    for b in sorted({0, batch - 1, *rng.choice(batch, 6, replace=False).tolist()}):
        want = _oracle_chain(X[b * n3:(b + 1) * n3], Aop, Bop, Cop, n, s)
        check_float_parity(got[b * n3:(b + 1) * n3], want, f"chain tensor {b}")


def test_fused_pairs_and_lone_last_tile_at_scale(handle):
    # k = 16 takes tiles in pairs.  16387 tiles make runs of 4 tiles per
    # wavefront, and the last run holds 3: two full pairs elsewhere, one pair
    # and one lone tile at the end.  Every output is compared with the oracle.
    import torch
    m, k, n, s = 16, 16, 16 * 16387, 16
    rng = np.random.default_rng(16387)
    A = workloads.real_matrix(m, k, int(rng.integers(1 << 30)), "phi", 1.0)
    B = workloads.real_matrix(k, n, int(rng.integers(1 << 30)), "phi", 1.0)
    print(f"[small pairs at scale] m={m} n={n} k={k} s={s}", flush=True)
    dC = torch.zeros(m * n, dtype=torch.float64, device="cuda")
    handle.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.0, dC, m, s)
    torch.cuda.synchronize()
    got = from_dev(dC)
    want = oracle.gemm_entries(False, "N", "N", m, n, k, 1.0, A, m, B, k, 0.0, None, m, s)["out"]
    check_float_parity(got, want, "pairs at scale")
