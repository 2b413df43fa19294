"""GPU parity of the persistent tensor-mode chain (oz2_chain_plan_create /
oz2_chain_rescale_be, OzII-RescaleBE of "You Only Convert Twice: Ozaki
Scheme II for Chained Tensor Mode Products", Algorithm 7, chains of depth
1 to 8) against the CPU oracle (oracle/rescale_be.py), through the C ABI,
on the kernel that keeps each tensor's residues in LDS (oz2_chain.hip; the
handle asks for it, since n <= 8 would otherwise run on the HBM kernels of
tests/test_gpu_chain_hbm.py).

Bar: the plan (b, g) equals the oracle planner's, and every output entry is
bit-identical to the oracle's: every step is exact integer arithmetic except
the FP64 Horner evaluation and the final scaling, which both sides perform in
the same order with the same roundings.  The parity cases run the base
extension in both forms (the CRT one where the plan allows it, and the
mixed-radix one of the page's Algorithm 4).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import from_dev, to_dev

pytestmark = pytest.mark.gpu
rb = oracle.rescale_be


@pytest.fixture(scope="module")
def handle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    h = oz2.Handle()
    h.set_chain_kernel("lds")   # n <= 8 would otherwise run on the HBM kernels
    yield h
    h.close()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ops(n, seed, dist="uniform", phi=0.5, d=3):
    return [workloads.real_matrix(n, n, seed + q, dist, phi) for q in range(d)]


def _check_bitwise(got, want, label):
    g = np.ascontiguousarray(got).view(np.int64)
    w = np.ascontiguousarray(want).view(np.int64)
    nan = np.isnan(got) & np.isnan(want)
    bad = np.nonzero((g != w) & ~nan)[0]
    assert bad.size == 0, (f"{label}: {bad.size} entries differ, first {bad[:4]}: "
                           f"got {got[bad[:4]]} want {want[bad[:4]]}")


def _run_forms(handle, cp, X, n, batch):
    """the chain with the base extension in the CRT form (where the plan
    allows it) and in the mixed-radix form after every product"""
    import torch
    out = []
    for crt in (True, False):
        handle.set_chain_crt(crt)
        try:
            dY = torch.full((n ** 3 * batch,), 7.0, dtype=torch.float64, device="cuda")
            handle.chain_rescale_be(cp, to_dev(X), dY, batch)
            torch.cuda.synchronize()
        finally:
            handle.set_chain_crt(True)
        out.append(("crt" if crt else "mixed radix", from_dev(dY)))
    return out


CASES = [
    # n, s, batch, tensor distribution
    (16, 16, 3, "uniform"),
    (16, 12, 2, "phi"),
    (8, 16, 4, "uniform"),
    (5, 10, 3, "uniform"),   # ragged: padded to 16 inside the kernel
    (12, 8, 2, "phi"),
    (1, 6, 5, "uniform"),
]


@pytest.mark.parametrize("n,s,batch,dist", CASES, ids=[f"n{c[0]}s{c[1]}b{c[2]}{c[3]}" for c in CASES])
def test_chain_matches_oracle_bitwise(handle, n, s, batch, dist):
    import torch
    _say(f"[chain] n={n} s={s} batch={batch} {dist}")
    ops = _ops(n, 8000 + 10 * n + s)
    if dist == "uniform":
        X = workloads.tensor_batch(n, batch, 8100 + n + s)
    else:
        X = workloads.real_matrix(n ** 3, batch, 8200 + n + s, "phi", 2.0)
    want, plan = rb.rescale_be_chain(X, ops, n, s, batch)
    assert plan is not None
    with handle.chain_plan(ops, n, s) as cp:
        assert (cp.depth, cp.b, list(cp.g)) == (3, plan["b"], plan["g"]), (cp.b, cp.g, plan["b"], plan["g"])
        for form, got in _run_forms(handle, cp, X, n, batch):
            _check_bitwise(got, want, f"n={n} s={s} {form}")


def test_chain_edge_tensors(handle):
    """zero tensor, a non-finite entry, a subnormal-scale tensor, a huge-range
    tensor and an ordinary one in one batch"""
    import torch
    n, s = 16, 16
    ops = _ops(n, 8300, "phi", 1.0)
    n3 = n ** 3
    X = workloads.tensor_batch(n, 5, 8301)
    X[:n3] = 0.0
    X[n3 + 77] = np.nan
    X[2 * n3:3 * n3] *= 2.0 ** -1060          # subnormal entries
    X[3 * n3:4 * n3] = workloads.real_matrix(n3, 1, 8302, "phi", 6.0)
    want, plan = rb.rescale_be_chain(X, ops, n, s, 5)
    with handle.chain_plan(ops, n, s) as cp:
        dY = torch.empty(n3 * 5, dtype=torch.float64, device="cuda")
        handle.chain_rescale_be(cp, to_dev(X), dY, 5)
        torch.cuda.synchronize()
    got = from_dev(dY)
    assert np.all(got[:n3] == 0.0)
    assert np.all(np.isnan(got[n3:2 * n3]))
    _check_bitwise(got, want, "edge tensors")


def test_chain_full_workload_sampled(handle):
    """The 32768-tensor batch of 16^3 tensors at s = 16 in the launch bench.py
    times; the first, last and six seeded tensors against the oracle."""
    import torch
    w = workloads.WORKLOADS[5]
    n, batch, s = w["n"], w["batch"], w["s"][0]
    n3 = n ** 3
    X = workloads.tensor_batch(n, batch, workloads.seed(5, 0))
    ops = [workloads.real_matrix(n, n, workloads.seed(5, q)) for q in (1, 2, 3)]
    plan = rb.prepare_chain(ops, n, s)
    with handle.chain_plan(ops, n, s) as cp:
        dY = torch.empty(n3 * batch, dtype=torch.float64, device="cuda")
        handle.chain_rescale_be(cp, to_dev(X), dY, batch)
        torch.cuda.synchronize()
    rng = np.random.default_rng(8400)
    picks = sorted({0, batch - 1, *rng.choice(batch, 6, replace=False).tolist()})
    Y = from_dev(dY)
    for t in picks:
        _say(f"[chain full] tensor {t}")
        want = rb.chain_tensor(X[t * n3:(t + 1) * n3], plan)
        _check_bitwise(Y[t * n3:(t + 1) * n3], want, f"tensor {t}")


DEPTH_CASES = [
    # n, s, depth, batch
    (16, 16, 1, 2),
    (16, 16, 2, 2),
    (16, 16, 4, 2),   # every g = 7: the compile-time instance
    (16, 14, 5, 2),
    (8, 16, 8, 3),    # the page's deepest chain; the last drop count differs
    (5, 12, 6, 2),
    (16, 16, 7, 1),
]


@pytest.mark.parametrize("n,s,d,batch", DEPTH_CASES, ids=[f"n{c[0]}s{c[1]}d{c[2]}" for c in DEPTH_CASES])
def test_chain_depth_matches_oracle_bitwise(handle, n, s, d, batch):
    """Longer chains revisit the directions (operator i along direction
    i mod 3), with the pending row scales folded into the next operator on a
    direction; every layout rotation d mod 3 is covered."""
    import torch
    _say(f"[chain depth] n={n} s={s} d={d} batch={batch}")
    ops = _ops(n, 8500 + 10 * n + d, d=d)
    X = workloads.tensor_batch(n, batch, 8600 + n + d)
    want, plan = rb.rescale_be_chain(X, ops, n, s, batch)
    assert plan is not None
    with handle.chain_plan(ops, n, s) as cp:
        assert (cp.depth, cp.b, list(cp.g)) == (d, plan["b"], plan["g"]), (cp.b, cp.g, plan["b"], plan["g"])
        for form, got in _run_forms(handle, cp, X, n, batch):
            _check_bitwise(got, want, f"n={n} s={s} d={d} {form}")


MODE_CASES = [
    # n, s, modes (1-based), batch
    (16, 16, [2, 3, 1], 2),        # first product along direction 2: byte-wise encode stores
    (16, 16, [1, 1, 2], 2),        # one direction twice in a row (store kind 2)
    (16, 16, [1, 3, 2], 2),        # the fibre direction next (store kind 1)
    (8, 16, [3, 3, 3, 1, 2], 2),
    (12, 14, [2, 1, 2, 3, 3, 1], 1),
    (5, 12, [3, 1, 1, 2], 2),      # drop counts 5, 6, 6: the guarded instance
    (16, 12, [3, 2, 1], 2),        # depth 3 in another order: the run-time instance
]


@pytest.mark.parametrize("n,s,modes,batch", MODE_CASES, ids=["m" + "".join(map(str, c[2])) + f"n{c[0]}" for c in MODE_CASES])
def test_chain_mode_sequences_match_oracle_bitwise(handle, n, s, modes, batch):
    """Algorithm 7 with any sequence of modes: every residue layout kind and
    first direction, through the run-time instance of the kernel"""
    import torch
    d = len(modes)
    _say(f"[chain modes] n={n} s={s} modes={modes} batch={batch}")
    ops = _ops(n, 8700 + 10 * n + d, d=d)
    X = workloads.tensor_batch(n, batch, 8800 + n + d)
    want, plan = rb.rescale_be_chain(X, ops, n, s, batch, [m - 1 for m in modes])
    assert plan is not None
    with handle.chain_plan(ops, n, s, modes) as cp:
        assert (cp.depth, cp.b, list(cp.g)) == (d, plan["b"], plan["g"]), (cp.b, cp.g, plan["b"], plan["g"])
        for form, got in _run_forms(handle, cp, X, n, batch):
            _check_bitwise(got, want, f"modes={modes} {form}")


def test_chain_argument_errors(handle):
    import ctypes
    import complex_gemm_emulation_amd as oz2
    lib = oz2.lib()
    A = np.eye(4)
    p = A.ctypes.data_as(ctypes.c_void_p)
    three = (ctypes.c_void_p * 3)(p, p, p)
    out = ctypes.c_void_p()
    assert lib.oz2_chain_plan_create(handle._h, 0, 3, three, None, 8, ctypes.byref(out)) == -2
    assert lib.oz2_chain_plan_create(handle._h, 257, 3, three, None, 8, ctypes.byref(out)) == -2
    assert lib.oz2_chain_plan_create(handle._h, 4, 0, three, None, 8, ctypes.byref(out)) == -3
    assert lib.oz2_chain_plan_create(handle._h, 4, 9, three, None, 8, ctypes.byref(out)) == -3
    assert lib.oz2_chain_plan_create(handle._h, 4, 3, None, None, 8, ctypes.byref(out)) == -4
    holey = (ctypes.c_void_p * 3)(p, None, p)
    assert lib.oz2_chain_plan_create(handle._h, 4, 3, holey, None, 8, ctypes.byref(out)) == -4
    badm = (ctypes.c_int * 3)(1, 4, 2)
    assert lib.oz2_chain_plan_create(handle._h, 4, 3, three, badm, 8, ctypes.byref(out)) == -5
    assert lib.oz2_chain_plan_create(handle._h, 4, 3, three, None, 17, ctypes.byref(out)) == -6
    assert lib.oz2_chain_plan_create(handle._h, 4, 3, three, None, 8, None) == -7
    bad = np.eye(4)
    bad[1, 2] = np.inf
    badp = (ctypes.c_void_p * 3)(p, bad.ctypes.data_as(ctypes.c_void_p), p)
    assert lib.oz2_chain_plan_create(handle._h, 4, 3, badp, None, 8, ctypes.byref(out)) == -4
    assert not out.value
    with handle.chain_plan([A, A, A], 4, 8) as cp:
        assert lib.oz2_chain_rescale_be(handle._h, cp._p, None, None, 0) == 0   # empty batch
        assert lib.oz2_chain_rescale_be(handle._h, cp._p, None, None, 1) == -3
        assert lib.oz2_chain_rescale_be(handle._h, cp._p, None, None, -1) == -5
