"""GPU parity on the non-square shapes of the Arc page's Table 10 (Sec. 7.1),
at full size, in the launch configuration bench.py times, on seeded samples
of output entries that the oracle computes one by one (first and last rows
and columns included).  4000 x 8000 x 4000 is ragged in every dimension
(not a multiple of the 256-row tiles or of the 64-position k panels)."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_float_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu

W = workloads.NONSQUARE
SHAPES = [tuple(x) for x in W["shapes"]]

# (shape index, s): every shape but the two 4 GiB-operand ones
# (8192 x 65536 x 8192 runs the same code path as 8192 x 32768 x 8192)
CASES = [(0, 8), (0, 16), (1, 16), (2, 8), (4, 16), (5, 8), (6, 16), (6, 8), (7, 16)]


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
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, min(side, m), replace=False)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(side, n), replace=False)]))
    ii, jj = np.meshgrid(rows, cols, indexing="ij")
    return ii.reshape(-1), jj.reshape(-1)


@pytest.mark.parametrize("q,s", CASES, ids=[f"{'x'.join(map(str, SHAPES[q]))}s{s}" for q, s in CASES])
def test_nonsquare_sampled(handle, q, s):
    import torch
    m, k, n = SHAPES[q]
    print(f"[nonsquare] {m}x{k}x{n} s={s}", flush=True)
    A = workloads.real_matrix(m, k, workloads.nonsquare_seed(q, 0), W["dist"])
    B = workloads.real_matrix(k, n, workloads.nonsquare_seed(q, 1), W["dist"])
    dC = torch.zeros(m * n, dtype=torch.float64, device="cuda")
    handle.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.0, dC, m, s)
    torch.cuda.synchronize()
    side = 24 if k <= 8192 else 12
    rows, cols = _sample(m, n, side, 600 + 10 * q + s)
    got = from_dev(dC)[rows + cols * m]
    r = oracle.gemm_entries(False, "N", "N", m, n, k, 1.0, A, m, B, k, 0.0, None, m, s,
                            rows=rows, cols=cols, nthreads=oracle.max_threads())
    check_float_parity(got, r["out"], f"{m}x{k}x{n} s={s}")
