"""CPU tests of bench.py's own measurement arithmetic: the exact dot products
behind the reported normwise errors, the algorithmic byte and operation
counts behind the roofline fields, the traffic records' source keys, the
RescaleBE operation count, and the single-GPU contract."""
import json
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _vectors(rng, k, spread):
    a = (rng.random(k) - 0.5) * np.exp2(rng.integers(-spread, spread, k))
    b = (rng.random(k) - 0.5) * np.exp2(rng.integers(-spread, spread, k))
    return a, b


@pytest.mark.parametrize("seed,spread", [(1, 4), (2, 60), (3, 300)])
def test_exact_dot_is_the_rational_sum_rounded_once(seed, spread):
    rng = np.random.default_rng(seed)
    for k in (1, 7, 64, 500):
        a, b = _vectors(rng, k, spread)
        exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b))
        assert bench.exact_dot_fraction(a, b) == exact
        # float(Fraction) rounds correctly to nearest, ties to even
        assert bench.exact_dot(a, b) == float(exact)


def test_exact_dot_under_total_cancellation():
    # x + y - x: the naive float sum loses y entirely
    a = np.array([1e300 / 2 ** 900, 3.0, -1e300 / 2 ** 900])
    b = np.array([2.0 ** 900, 1e-300, 2.0 ** 900])
    exact = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b))
    assert bench.exact_dot(a, b) == float(exact) == 3e-300


def test_normwise_error_definition():
    ref = np.array([3.0, -4.0])
    got = np.array([3.0, -4.0 + 5e-16])
    assert bench.normwise_error(got, ref) == pytest.approx(5e-16 / 5.0, rel=1e-12)
    assert bench.normwise_error(ref, ref) == 0.0


@pytest.mark.parametrize("s,ops,encode_gb,gemm_gb,recon_gb", [
    # 8192^3, beta = 0: INT8 ops, encode bytes, GEMM minimum bytes and
    # reconstruct bytes per call, as tabulated for the headline workload
    (8, 8.80e12, 2.15, 1.61, 1.07),
    (12, 1.32e13, 2.68, 2.42, 1.34),
    (16, 1.76e13, 3.22, 3.22, 1.61),
])
def test_algorithmic_counts_of_the_headline_workload(s, ops, encode_gb, gemm_gb, recon_gb):
    w = bench.algorithmic(8192, 8192, 8192, s)
    assert w["int8_ops"] == 2 * 8192 ** 3 * s
    assert w["int8_ops"] == pytest.approx(ops, rel=5e-3)
    assert w["scan_bytes"] == 8 * 2 * 8192 ** 2
    assert w["encode_bytes"] / 1e9 == pytest.approx(encode_gb, abs=6e-3)
    assert w["gemm_bytes"] / 1e9 == pytest.approx(gemm_gb, abs=6e-3)
    assert w["recon_bytes"] / 1e9 == pytest.approx(recon_gb, abs=6e-3)


def test_algorithmic_counts_complex_and_beta():
    m = n = k = 4096
    s = 16
    w = bench.algorithmic(m, n, k, s, cplx=True, beta_nonzero=True)
    assert w["int8_ops"] == 2 * m * n * k * s * 3            # three products per modulus (3M)
    assert w["encode_bytes"] == (16 + 3 * s) * (m * k + k * n)
    assert w["gemm_bytes"] == 3 * s * (m * k + k * n) + 2 * s * m * n
    assert w["recon_bytes"] == (2 * s + 16) * m * n + 16 * m * n


def test_rescale_be_operation_count_at_the_workload():
    # s = 16, drops g = 7 after the first two products of a depth-3 chain
    assert bench.rbe_valu_ops_per_entry(16, [7, 7, 0]) == 2144
    # one rescaling product: 16 reductions (3 each), drops over 15 .. 9
    # remaining moduli (84 steps of 5), 36 digit steps of 5 among the 9 kept,
    # 7 extensions of 9 products and a reduction
    assert bench.rbe_product_ops_per_entry(16, 7) == 48 + 420 + 180 + 84
    # the chain is two such products, the last product's 16 reductions and
    # the reconstruction (120 digit steps, 15 fp64 Horner FMAs, one scaling)
    assert bench.rbe_valu_ops_per_entry(16, [7, 7, 0]) == 2 * 732 + 48 + 600 + 30 + 2


def test_traffic_records_are_keyed_on_workload_and_sources(tmp_path):
    rec_path = os.path.join(ROOT, "profiles", "small_gemm_traffic.json")
    with open(rec_path) as f:
        rec = json.load(f)
    # a record is only used for its own workload
    assert bench.measured_traffic("dgemm8192", rec_path) is None
    # and only while its sources hash as recorded
    stale = dict(rec, source_sha256_16="0" * 16)
    p = tmp_path / "stale.json"
    p.write_text(json.dumps(stale))
    assert bench.measured_traffic(rec["bench_workload"], str(p)) is None
    fresh = tmp_path / "fresh.json"
    fresh.write_text(json.dumps(rec))
    got = bench.measured_traffic(rec["bench_workload"], str(fresh))
    assert got is None or got == rec["bytes_per_launch"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_entry_accuracy_statistics():
    # correctly rounded entries give 100% and at most half an ulp; an entry
    # moved by one ulp counts as not correctly rounded with an error near 1 ulp
    rng = np.random.default_rng(71)
    k, m, n = 40, 3, 4
    Am = rng.uniform(-1, 1, (m, k))
    Bm = rng.uniform(-1, 1, (n, k))
    rows = np.array([0, 1, 2, 0])
    cols = np.array([0, 1, 2, 3])
    exact = [bench.exact_dot_fraction(Am[i], Bm[j]) for i, j in zip(rows, cols)]
    good = np.array([float(x) for x in exact])
    st = bench.entry_accuracy(good, Am, Bm, rows, cols)
    assert st["cr_pct"] == 100.0 and st["max_ulp"] <= 0.5
    assert st["normwise"] < 2.0 ** -52
    bad = good.copy()
    bad[2] = np.nextafter(bad[2], np.inf)
    st2 = bench.entry_accuracy(bad, Am, Bm, rows, cols)
    assert st2["cr_pct"] == 75.0 and 0.5 < st2["max_ulp"] <= 1.5
    aabb = float(np.abs(Am[2]) @ np.abs(Bm[2]))
    assert st2["componentwise"] == pytest.approx(float(abs(Fraction(bad[2]) - exact[2])) / aabb)


def test_accuracy_operands_shapes_and_structure():
    m, n, k = 8, 6, 10
    for data in bench.ACCURACY_DATA:
        A, B = bench.accuracy_operands(data, m, n, k, 123)
        assert A.size == m * k and B.size == k * n, data
    A, _ = bench.accuracy_operands("spike", m, n, k, 5)
    Am = A.reshape(k, m).T
    for i in range(m):  # one element per row of A is 2^40 times the scale of the others
        big = np.abs(Am[i]) > 2.0 ** 20
        assert big.sum() == 1
    A, B = bench.accuracy_operands("cancel", m, n, k, 6)
    Am, Bm = A.reshape(k, m).T, B.reshape(n, k).T
    assert np.array_equal(Am[:, : k // 2], Am[:, k // 2:])
    C = Am @ Bm
    assert np.max(np.abs(C)) < 2.0 ** -25 * np.max(np.abs(Am) @ np.abs(Bm))


def test_gemm_block_terms_follow_the_tile_choice():
    # 256 x 256 tile when >= 512 such blocks over all moduli and k > 512;
    # 8192^3 at s = 16: 32 x 32 x 16 blocks = 64 waves of 256 CUs, 128 steps
    assert bench.gemm_block_terms(8192, 8192, 8192, 16) == [64, 64 * 128, 0, 0]
    # short k takes the 128 x 128 tile, four blocks per CU
    assert bench.gemm_block_terms(8192, 8192, 256, 8) == [0, 0, 32, 32 * 4]
    # few blocks: 1024^2 at s = 8 is 128 blocks of 256 x 256
    assert bench.gemm_block_terms(1024, 1024, 1024, 8)[:2] == [0, 0]
    # k beyond one exact run: two launches
    t = bench.gemm_block_terms(2048, 2048, 131330, 8)
    assert t[0] == 2 * 2 and t[1] == 2 * (2044 + 12)
    # the complex 3M kernel runs three k-loops per block
    assert bench.gemm_block_terms(4096, 4096, 4096, 16, cplx=True)[1] == 16 * 64 * 3
