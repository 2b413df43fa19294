"""oz2_dgemm_noalloc against oz2_dgemm, through the C ABI: the same product
with the library's fixed device scratch as workspace must give bitwise the
same output, on calls in a row of decreasing size, on a product that has to
run in blocks to fit the scratch, and on the fused short-k path; a product
too large for the scratch is refused before anything is enqueued."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_float_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def handles():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    ref, na = oz2.Handle(), oz2.Handle()
    yield ref, na
    ref.close()
    na.close()


def _pair(handles, ta, tb, m, n, k, s, alpha, beta, ldc, seed):
    import torch
    ref, na = handles
    ra, ca = workloads.stored_shape(ta, m, k)
    rb, cb = workloads.stored_shape(tb, k, n)
    A = workloads.real_matrix(ra, ca, seed, "phi", 1.0)
    B = workloads.real_matrix(rb, cb, seed + 1, "phi", 1.0)
    C = workloads.real_matrix(m, n, seed + 2, "uniform", ld=ldc)
    dA, dB = to_dev(A), to_dev(B)
    dC1, dC2 = to_dev(C), to_dev(C)
    _say(f"[noalloc] {ta}{tb} m={m} n={n} k={k} s={s} ldc={ldc}")
    ref.dgemm(ta, tb, m, n, k, alpha, dA, ra, dB, rb, beta, dC1, ldc, s)
    na.dgemm_noalloc(ta, tb, m, n, k, alpha, dA, ra, dB, rb, beta, dC2, ldc, s)
    torch.cuda.synchronize()
    g1, g2 = from_dev(dC1), from_dev(dC2)
    assert np.array_equal(g1.view(np.uint64), g2.view(np.uint64)), \
        f"{np.count_nonzero(g1.view(np.uint64) != g2.view(np.uint64))} entries differ"
    assert na.workspace_size() == 0, "the no-alloc handle grew a workspace of its own"
    return A, B, C, g2


def test_noalloc_matches_dgemm_on_calls_in_a_row(handles):
    # a product that fits the scratch whole, then a smaller one
    _pair(handles, "N", "N", 1024, 1024, 1024, 16, 1.0, 0.0, 1024, workloads.seed(40, 0))
    A, B, C, got = _pair(handles, "T", "N", 300, 200, 500, 8, -0.75, 1.25, 303, workloads.seed(40, 10))
    want = oracle.gemm_entries(False, "T", "N", 300, 200, 500, -0.75, A, 500, B, 500, 1.25, C, 303, 8,
                               chat_ints=False)["out"]
    full = got.reshape(200, 303)
    assert check_float_parity(full[:, :300].T, want.reshape(200, 300).T, "noalloc vs oracle") == 0
    assert np.array_equal(np.isnan(full[:, 300:]), np.isnan(C.reshape(200, 303)[:, 300:]))


def test_noalloc_blocks_to_fit_the_scratch(handles):
    # the whole workspace (about 420 MB) exceeds the 128 MiB scratch: blocks of C
    _pair(handles, "N", "T", 3000, 2600, 3000, 16, 1.5, -0.5, 3001, workloads.seed(41, 0))


def test_noalloc_fused_short_k(handles):
    _pair(handles, "N", "N", 16, 5000, 16, 16, 1.0, 0.0, 16, workloads.seed(42, 0))


def test_noalloc_refuses_too_large(handles):
    import torch
    import complex_gemm_emulation_amd as oz2
    _, na = handles
    m = n = 256
    k = 20000  # one 256 x 256 block with all of k needs about 165 MB at s = 16
    dA = torch.zeros(m * k, dtype=torch.float64, device="cuda")
    dB = torch.zeros(k * n, dtype=torch.float64, device="cuda")
    dC = torch.full((m * n,), 3.0, dtype=torch.float64, device="cuda")
    with pytest.raises(oz2.Oz2Error) as ei:
        na.dgemm_noalloc("N", "N", m, n, k, 1.0, dA, m, dB, k, 0.0, dC, m, 16)
    assert ei.value.status == 7
    torch.cuda.synchronize()
    assert bool(torch.all(dC == 3.0))
