"""Memory-aware tiling (Arc page Sec. 6; its tests require tiled = untiled
bitwise, Sec. 8.1): under a workspace cap the product is computed in blocks
of C, each with all of k, and must equal the untiled result bit for bit and
the oracle to the usual bar.  The blocking comes from the library's cost
model (block sides a power-of-two multiple of 256 or the whole dimension,
Table 16's 2^j tiles; the operand whose encoded block is kept chosen too);
the cases below are sized so that it picks non-square blocks and either
operand, and the expected blocking is the model's."""
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
    # cplx, m, n, k, ta, tb, s, limit, expected blocking (mb, nb, held)
    (False, 700, 600, 300, "T", "N", 16, 6 * MiB, (256, 256, "A")),
    (False, 300, 1100, 70, "N", "T", 8, 2 * MiB, (256, 256, "A")),
    (True, 300, 520, 200, "C", "N", 12, 8 * MiB, (256, 256, "A")),
    # tall: two block rows over all columns, op(B) encoded once and kept
    (False, 2000, 300, 600, "N", "N", 8, 12 * MiB, (1024, 300, "B")),
    # wide: four block columns over all rows, op(A) kept
    (False, 300, 2000, 600, "T", "T", 8, 12 * MiB, (300, 512, "A")),
    # both split, non-square blocks
    (False, 1500, 1500, 300, "N", "T", 16, 10 * MiB, (256, 512, "B")),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{'z' if c[0] else 'd'}{c[1]}x{c[2]}x{c[3]}{c[4]}{c[5]}s{c[6]}" for c in CASES])
def test_tiled_equals_untiled_and_oracle(case):
    import torch
    oz2 = _handle()
    cplx, m, n, k, ta, tb, s, limit, plan = case
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
                tp = h.tile_plan()
                assert (tp["mb"], tp["nb"], tp["held"]) == plan, tp
            else:
                assert h.tile_plan() == dict(mb=m, nb=n, held="untiled")
    assert np.array_equal(outs[0].view(np.uint64), outs[1].view(np.uint64)), "tiled != untiled"
    want = oracle.gemm_entries(cplx, ta, tb, m, n, k, al, A, ra, B, rb, be, C, m, s)["out"]
    assert check_float_parity(outs[1], want, f"tiled {case}") == 0


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


PREPARED = [
    # cplx, m, n, k, s, limit, expected blocks (mb, nb)
    (False, 1500, 1300, 400, 16, 12 * MiB, (1500, 512)),
    (True, 700, 900, 300, 12, 10 * MiB, (700, 512)),
]


@pytest.mark.parametrize("case", PREPARED, ids=[f"{'z' if c[0] else 'd'}{c[1]}x{c[2]}x{c[3]}s{c[4]}" for c in PREPARED])
def test_prepared_product_tiles_bitwise(case):
    # the prepared product holds only residues in its workspace; under a cap it
    # runs in blocks that read their rows and columns of the prepared planes in
    # place, bitwise equal to the untiled prepared product and the plain call
    import torch
    oz2 = _handle()
    cplx, m, n, k, s, limit, blocks = case
    print(f"[tiling] prepared {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    sd = [int(x) for x in rng.integers(1 << 30, size=6)]
    if cplx:
        A = workloads.complex_matrix(m, k, sd[0], sd[1], "phi", 1.0)
        B = workloads.complex_matrix(k, n, sd[2], sd[3], "phi", 1.0)
        C = workloads.complex_matrix(m, n, sd[4], sd[5], "uniform")
        al, be = complex(0.5, 0.25), complex(-0.75, 0.5)
    else:
        A = workloads.real_matrix(m, k, sd[0], "phi", 1.0)
        B = workloads.real_matrix(k, n, sd[2], "phi", 1.0)
        C = workloads.real_matrix(m, n, sd[4], "uniform")
        al, be = 1.25, -0.5
    dA, dB = to_dev(A), to_dev(B)
    outs = []
    with oz2.Handle() as h:
        pa = h.prepare("A", "N", m, k, dA, m, s, cplx)
        pb = h.prepare("B", "N", n, k, dB, k, s, cplx)
        for lim in (0, limit):
            h.set_memory_limit(lim)
            dC = to_dev(C)
            h.gemm_prepared(pa, pb, al, be, dC, m)
            torch.cuda.synchronize()
            outs.append(from_dev(dC))
            tp = h.tile_plan()
            if lim:
                assert (tp["mb"], tp["nb"], tp["held"]) == (*blocks, "prepared"), tp
            else:
                assert tp["held"] == "untiled"
        pa.close()
        pb.close()
        h.set_memory_limit(0)
        dC = to_dev(C)
        (h.zgemm if cplx else h.dgemm)("N", "N", m, n, k, al, dA, m, dB, k, be, dC, m, s)
        torch.cuda.synchronize()
        outs.append(from_dev(dC))
    for q in (1, 2):
        assert np.array_equal(outs[0].view(np.uint64), outs[q].view(np.uint64)), f"output {q} differs"
    want = oracle.gemm_entries(cplx, "N", "N", m, n, k, al, A, m, B, k, be, C, m, s)["out"]
    assert check_float_parity(outs[1], want, f"tiled prepared {case}") == 0
