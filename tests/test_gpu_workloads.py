"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration bench.py times, on seeded samples of output entries that the
oracle computes one by one (first and last rows/columns included), plus the
accuracy level against the exact product."""
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


def _sample(m, n, side, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, side, replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, side, replace=False)]))
    ii, jj = np.meshgrid(rows, cols, indexing="ij")
    return ii.reshape(-1), jj.reshape(-1)


def _normwise(got, rows, cols, Am, Bm, count):
    """||e||_F / ||C||_F on the first `count` sampled entries against the exact product."""
    num = den = 0.0
    for q in range(count):
        i, j = rows[q], cols[q]
        ex = oracle.fraction_to_double(oracle.exact_dot(Am[i, :], Bm[:, j]))
        num += (got[q] - ex) ** 2
        den += ex ** 2
    return (num / den) ** 0.5


@pytest.mark.parametrize("s", [8, 12, 16])
def test_dgemm_8192_sampled(handle, s):
    import torch
    w = workloads.WORKLOADS[2]
    m, n, k = w["m"], w["n"], w["k"]
    print(f"[workload 8192] s={s}", flush=True)
    A = workloads.real_matrix(m, k, workloads.seed(2, 0), "phi", 0.5)
    B = workloads.real_matrix(k, n, workloads.seed(2, 1), "phi", 0.5)
    dC = torch.zeros(m * n, dtype=torch.float64, device="cuda")
    handle.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.0, dC, m, s)
    torch.cuda.synchronize()
    rows, cols = _sample(m, n, 24, 100 + s)
    got = from_dev(dC)[rows + cols * m]
    r = oracle.gemm_entries(False, "N", "N", m, n, k, 1.0, A, m, B, k, 0.0, None, m, s,
                            rows=rows, cols=cols)
    check_float_parity(got, r["out"], f"8192 s={s}")
    if s == 16:
        Am, Bm = A.reshape(k, m).T, B.reshape(n, k).T
        err = _normwise(got, rows, cols, Am, Bm, 40)
        assert err <= 1e-15, err


@pytest.mark.parametrize("s", [20, 24])
def test_dgemm_4096_wide_exponent_TN_sampled(handle, s):
    import torch
    w = workloads.WORKLOADS[3]
    m, n, k = w["m"], w["n"], w["k"]
    print(f"[workload 4096 wide] s={s}", flush=True)
    A = workloads.real_matrix(k, m, workloads.seed(3, 0), "phi", 4.0)   # stored k x m, op T
    B = workloads.real_matrix(k, n, workloads.seed(3, 1), "phi", 4.0)
    C = workloads.real_matrix(m, n, workloads.seed(3, 2), "uniform")
    dC = to_dev(C)
    handle.dgemm("T", "N", m, n, k, 1.5, to_dev(A), k, to_dev(B), k, -0.5, dC, m, s)
    torch.cuda.synchronize()
    rows, cols = _sample(m, n, 24, 200 + s)
    got = from_dev(dC)[rows + cols * m]
    r = oracle.gemm_entries(False, "T", "N", m, n, k, 1.5, A, k, B, k, -0.5, C, m, s,
                            rows=rows, cols=cols)
    check_float_parity(got, r["out"], f"4096 TN s={s}")


def test_zgemm_4096_conj_sampled(handle):
    import torch
    w = workloads.WORKLOADS[4]
    m, n, k = w["m"], w["n"], w["k"]
    print("[workload zgemm 4096]", flush=True)
    A = workloads.complex_matrix(k, m, workloads.seed(4, 0), workloads.seed(4, 3), "phi", 0.5)
    B = workloads.complex_matrix(k, n, workloads.seed(4, 1), workloads.seed(4, 4), "phi", 0.5)
    C = workloads.complex_matrix(m, n, workloads.seed(4, 2), workloads.seed(4, 5), "uniform")
    al, be = w["alpha"], w["beta"]
    dC = to_dev(C)
    handle.zgemm("C", "N", m, n, k, al, to_dev(A), k, to_dev(B), k, be, dC, m, 16)
    torch.cuda.synchronize()
    rows, cols = _sample(m, n, 16, 400)
    got = from_dev(dC)[rows + cols * m]
    r = oracle.gemm_entries(True, "C", "N", m, n, k, al, A, k, B, k, be, C, m, 16,
                            rows=rows, cols=cols)
    check_float_parity(got, r["out"], "zgemm 4096")
