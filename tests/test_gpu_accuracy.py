"""The accuracy facts the Arc page states for its worst cases and its
well-scaled data (Sec. 8.2, Sec. 8.3, Tables 6 and 8), checked on this GPU
against the exact products of 256 sampled entries of 512 x 512 x 4096
products (the statistics of bench.py's accuracy workload):

* U(-1, 1) data is correctly rounded at s = 16 (max 0.5 ulp);
* a spike 2^40 times larger than the rest of its row: DGEMM-level accuracy
  at s = 20 and correct rounding at s = 24;
* cancellation A = [X X], B = [Y; -Y + 2^-30 Z]: a normwise error near the
  unit roundoff at s = 20 and correct rounding at s = 24;
* every entry 1 - 2^-53 (|c_hat| = M/4 at the CRT range's boundary): exact,
  i.e. correctly rounded, at every s.

The pages' seeds are unknown, so these are checks in distribution."""
import sys

import numpy as np
import pytest

import bench
import workloads

pytestmark = pytest.mark.gpu

M = N = 512
K = 4096


@pytest.fixture(scope="module")
def run():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    h = oz2.Handle()
    rng = np.random.default_rng(778)
    ri = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 16, replace=False)]))[:16]
    cj = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 16, replace=False)]))[:16]
    rows, cols = (x.reshape(-1) for x in np.meshgrid(ri, cj, indexing="ij"))

    def go(data, s):
        print(f"[accuracy] {data} s={s}", flush=True)
        sys.stdout.flush()
        A, B = bench.accuracy_operands(data, M, N, K, workloads.seed(9, 10 * bench.ACCURACY_DATA.index(data)))
        dC = torch.zeros(M * N, dtype=torch.float64, device="cuda")
        h.dgemm("N", "N", M, N, K, 1.0, torch.from_numpy(A).cuda(), M, torch.from_numpy(B).cuda(), K, 0.0, dC, M, s)
        torch.cuda.synchronize()
        got = dC.cpu().numpy()[rows + cols * M]
        return bench.entry_accuracy(got, A.reshape(K, M).T, B.reshape(N, K), rows, cols)

    yield go
    h.close()


def test_uniform_correctly_rounded_at_16(run):
    st = run("uniform", 16)
    assert st["cr_pct"] == 100.0 and st["max_ulp"] <= 0.5, st


def test_spike(run):
    st20 = run("spike", 20)
    assert st20["normwise"] < 1e-15 and st20["componentwise"] < 1e-15, st20
    st24 = run("spike", 24)
    assert st24["cr_pct"] == 100.0 and st24["max_ulp"] <= 0.5, st24


def test_cancellation(run):
    st20 = run("cancel", 20)
    assert st20["normwise"] < 1e-14, st20
    st24 = run("cancel", 24)
    assert st24["cr_pct"] == 100.0 and st24["max_ulp"] <= 0.5, st24


@pytest.mark.parametrize("s", [16, 20, 24])
def test_crt_range_boundary_exact(run, s):
    st = run("one_minus_ulp", s)
    assert st["cr_pct"] == 100.0 and st["max_ulp"] <= 0.5, st
