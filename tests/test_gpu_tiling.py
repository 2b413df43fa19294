"""Memory-aware tiling (Arc page Sec. 6; its tests require tiled = untiled
bitwise, Sec. 8.1): under a workspace cap the product is computed in blocks
of C, each with all of k, and must equal the untiled result bit for bit and
the oracle to the usual bar."""
import zlib

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import check_float_parity, from_dev, to_dev

pytestmark = pytest.mark.gpu

MiB = 1 << 20


def _handle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    return oz2


CASES = [
    # cplx, m, n, k, ta, tb, s, limit
    (False, 700, 600, 300, "T", "N", 16, 6 * MiB),
    (False, 300, 1100, 70, "N", "T", 8, 2 * MiB),
    (True, 300, 520, 200, "C", "N", 12, 8 * MiB),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{'z' if c[0] else 'd'}{c[1]}x{c[2]}x{c[3]}{c[4]}{c[5]}s{c[6]}" for c in CASES])
def test_tiled_equals_untiled_and_oracle(case):
    import torch
    oz2 = _handle()
    cplx, m, n, k, ta, tb, s, limit = case
    print(f"[tiling] {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    ra, ca = workloads.stored_shape(ta, m, k)
    rb, cb = workloads.stored_shape(tb, k, n)
    sd = [int(x) for x in rng.integers(1 << 30, size=6)]
    if cplx:
        A = workloads.complex_matrix(ra, ca, sd[0], sd[1], "phi", 1.0)
        B = workloads.complex_matrix(rb, cb, sd[2], sd[3], "phi", 1.0)
        C = workloads.complex_matrix(m, n, sd[4], sd[5], "uniform")
        al, be = complex(0.5, 0.25), complex(-0.75, 0.5)
    else:
        A = workloads.real_matrix(ra, ca, sd[0], "phi", 1.0)
        B = workloads.real_matrix(rb, cb, sd[2], "phi", 1.0)
        C = workloads.real_matrix(m, n, sd[4], "uniform")
        al, be = 1.25, -0.5
    dA, dB = to_dev(A), to_dev(B)
    outs = []
    for lim in (0, limit):
        with oz2.Handle() as h:
            h.set_memory_limit(lim)
            dC = to_dev(C)
            fn = h.zgemm if cplx else h.dgemm
            fn(ta, tb, m, n, k, al, dA, ra, dB, rb, be, dC, m, s)
            torch.cuda.synchronize()
            outs.append(from_dev(dC))
            if lim:
                assert 0 < h.workspace_size() <= lim
    assert np.array_equal(outs[0].view(np.uint64), outs[1].view(np.uint64)), "tiled != untiled"
    want = oracle.gemm_entries(cplx, ta, tb, m, n, k, al, A, ra, B, rb, be, C, m, s)["out"]
    check_float_parity(outs[1], want, f"tiled {case}")


def test_limit_below_one_block_is_reported():
    oz2 = _handle()
    m = n = 512
    k = 512
    A = workloads.real_matrix(m, k, 1)
    B = workloads.real_matrix(k, n, 2)
    with oz2.Handle() as h:
        h.set_memory_limit(1 * MiB)
        with pytest.raises(oz2.Oz2Error) as ei:
            h.dgemm("N", "N", m, n, k, 1.0, to_dev(A), m, to_dev(B), k, 0.0, to_dev(np.zeros(m * n)), m, 16)
        assert ei.value.status == 4  # OZ2_STATUS_WORKSPACE_LIMIT
