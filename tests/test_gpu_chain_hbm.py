"""GPU parity of the persistent tensor-mode chain on HBM-resident residues
(OzII-RescaleBE of "You Only Convert Twice: Ozaki Scheme II for Chained
Tensor Mode Products", Algorithm 7; the kernels of oz2_chain_hbm.hip, which
run every chain with n <= 8 or n > 16 and, on request, the others) against
the CPU oracle (oracle/rescale_be.py), through the C ABI.

Bar: the plan (b, g) equals the oracle planner's, and every output entry is
bit-identical to the oracle's (every step is exact integer arithmetic except
the FP64 Horner evaluation and the final scaling, which both sides do in the
same order with the same roundings), with the base extension in the CRT form
(where the plan allows it) and in the mixed-radix form.  For n <= 16 the HBM
kernels must also equal the LDS kernel bit for bit.  The sides cover padding (n not a multiple
of 8, operator rows beyond a multiple of 16), the drop counts of the
compile-time instances and the run-time one, every residue layout kind,
small s (2: a rescaling product with no drop; 4), the sub-batches under a
memory limit, and the edge tensors.  Larger sides
(100, 128, 136, 200, 256: the staged form of the product kernels) are
checked against stored oracle samples in test_chain_hbm_golden_samples.
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import from_dev, to_dev

pytestmark = pytest.mark.gpu
rb = oracle.rescale_be
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def handle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import complex_gemm_emulation_amd as oz2
    h = oz2.Handle()
    yield h
    h.close()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ops(n, seed, d=3, dist="uniform", phi=0.5):
    return [workloads.real_matrix(n, n, seed + q, dist, phi) for q in range(d)]


def _check_bitwise(got, want, label):
    g = np.ascontiguousarray(got).view(np.int64)
    w = np.ascontiguousarray(want).view(np.int64)
    nan = np.isnan(got) & np.isnan(want)
    bad = np.nonzero((g != w) & ~nan)[0]
    assert bad.size == 0, (f"{label}: {bad.size} entries differ, first {bad[:4]}: "
                           f"got {got[bad[:4]]} want {want[bad[:4]]}")


def _run(handle, ops, n, s, X, batch, modes=None, kernel="auto", crt=True):
    import torch
    handle.set_chain_kernel(kernel)
    handle.set_chain_crt(crt)
    try:
        with handle.chain_plan(ops, n, s, modes) as cp:
            dY = torch.full((n ** 3 * batch,), 7.0, dtype=torch.float64, device="cuda")
            handle.chain_rescale_be(cp, to_dev(X), dY, batch)
            torch.cuda.synchronize()
            info = (cp.depth, cp.b, list(cp.g))
    finally:
        handle.set_chain_kernel("auto")
        handle.set_chain_crt(True)
    return from_dev(dY), info


CASES = [
    # n, s, modes (1-based, None: in turn), batch
    (24, 16, None, 5),             # np = 24, the last operator-row tile half used; g = 7, 7
    (32, 16, None, 4),
    (20, 12, None, 4),             # np = 24: padded positions; g = 6, 6
    (17, 8, None, 3),              # np = 24: the most padding; run-time drop counts
    (64, 15, None, 2),             # the chain page's s; two k chunks of the MFMA
    (40, 16, [1, 2, 3, 1, 2], 2),  # depth 5
    (24, 16, [3, 1, 2], 3),        # first product along direction 3: strided encode
    (24, 12, [2, 2, 1, 3], 2),     # one direction twice (store kind 2), then kind 1
    (36, 10, [1, 3], 3),           # depth 2, store kind 1, np = 40
    (48, 16, [2], 2),              # depth 1: encode, then the last product
    (72, 16, None, 1),             # three k chunks, five operator-row tiles
    (20, 12, [1, 2, 3, 1, 2, 3, 1, 2], 2),  # depth 8: seven rescaling products, buffers in turn
    (100, 10, [3, 2, 1], 1),       # staged form (2 chunk pairs, ragged), stores np apart
    (24, 2, None, 2),              # g = 0, 1, 0: a rescaling product with no drop; 14 slots of modulus 1
    (24, 4, None, 2),              # g = 1, 2; the reconstruction's first digit block holds only slots of modulus 1
]


@pytest.mark.parametrize("n,s,modes,batch", CASES,
                         ids=[f"n{c[0]}s{c[1]}" + ("" if c[2] is None else "m" + "".join(map(str, c[2])))
                              for c in CASES])
def test_chain_hbm_matches_oracle_bitwise(handle, n, s, modes, batch):
    d = 3 if modes is None else len(modes)
    _say(f"[chain hbm] n={n} s={s} modes={modes} batch={batch}")
    ops = _ops(n, 9000 + 10 * n + s, d)
    X = workloads.tensor_batch(n, batch, 9100 + n + s)
    want, plan = rb.rescale_be_chain(X, ops, n, s, batch, None if modes is None else [m - 1 for m in modes])
    assert plan is not None
    # the CRT base extension where the plan's bound allows it, and the
    # mixed-radix one after every product
    for crt in (True, False):
        got, info = _run(handle, ops, n, s, X, batch, modes, crt=crt)
        assert info == (d, plan["b"], plan["g"]), (info, plan["b"], plan["g"])
        _check_bitwise(got, want, f"n={n} s={s} modes={modes} crt={crt}")


SMALL_CASES = [
    # n <= 16 on the HBM kernels: n, s, modes, batch
    (16, 16, None, 6),
    (12, 16, [2, 3, 1], 4),   # np = 16
    (5, 6, None, 7),          # np = 8
    (1, 8, [3, 3], 9),
]


@pytest.mark.parametrize("n,s,modes,batch", SMALL_CASES, ids=[f"n{c[0]}s{c[1]}" for c in SMALL_CASES])
def test_chain_hbm_equals_lds_kernel(handle, n, s, modes, batch):
    d = 3 if modes is None else len(modes)
    _say(f"[chain hbm vs lds] n={n} s={s} modes={modes} batch={batch}")
    ops = _ops(n, 9200 + 10 * n + s, d)
    X = workloads.tensor_batch(n, batch, 9300 + n + s)
    want, plan = rb.rescale_be_chain(X, ops, n, s, batch, None if modes is None else [m - 1 for m in modes])
    hbm, _ = _run(handle, ops, n, s, X, batch, modes, "hbm")
    lds, _ = _run(handle, ops, n, s, X, batch, modes, "lds")
    _check_bitwise(hbm, lds, f"hbm vs lds n={n}")
    _check_bitwise(hbm, want, f"hbm vs oracle n={n}")


def test_chain_hbm_edge_tensors(handle):
    """zero tensor, a non-finite entry, a subnormal-scale tensor, a
    huge-range tensor and an ordinary one in one batch"""
    n, s, batch = 24, 16, 5
    ops = _ops(n, 9400, 3, "phi", 1.0)
    n3 = n ** 3
    X = workloads.tensor_batch(n, batch, 9401)
    X[:n3] = 0.0
    X[n3 + 1234] = np.inf
    X[2 * n3:3 * n3] *= 2.0 ** -1060
    X[3 * n3:4 * n3] = workloads.real_matrix(n3, 1, 9402, "phi", 6.0)
    want, _ = rb.rescale_be_chain(X, ops, n, s, batch)
    got, _ = _run(handle, ops, n, s, X, batch)
    assert np.all(got[:n3] == 0.0)
    assert np.all(np.isnan(got[n3:2 * n3]))
    _check_bitwise(got, want, "edge tensors")


def test_chain_hbm_sub_batches_under_memory_limit(handle):
    """a fresh handle limited to two tensors' planes: the batch runs in equal
    sub-batches within the limit, with results bitwise those of one pass, and
    a limit below one tensor is refused"""
    import torch
    import complex_gemm_emulation_amd as oz2
    n, s, batch = 32, 16, 7
    ops = _ops(n, 9500)
    X = workloads.tensor_batch(n, batch, 9501)
    whole, _ = _run(handle, ops, n, s, X, batch)
    per_tensor = 2 * s * n ** 3 + 8
    limit = 2 * per_tensor + 1024
    with oz2.Handle() as h2:
        h2.set_memory_limit(limit)
        parts, _ = _run(h2, ops, n, s, X, batch)
        assert 0 < h2.workspace_size() <= limit, h2.workspace_size()
    with oz2.Handle() as h3:
        h3.set_memory_limit(per_tensor // 2)
        with h3.chain_plan(ops, n, s) as cp:
            dY = torch.empty(n ** 3 * batch, dtype=torch.float64, device="cuda")
            with pytest.raises(oz2.Oz2Error):
                h3.chain_rescale_be(cp, to_dev(X), dY, batch)
    _check_bitwise(parts, whole, "sub-batches")
    want, _ = rb.rescale_be_chain(X[:2 * n ** 3], ops, n, s, 2)
    _check_bitwise(whole[:2 * n ** 3], want, "first two tensors")


def test_chain_hbm_lds_kernel_refuses_large_n(handle):
    import complex_gemm_emulation_amd as oz2
    n = 20
    ops = _ops(n, 9600)
    handle.set_chain_kernel("lds")
    try:
        import torch
        with handle.chain_plan(ops, n, 8) as cp:
            dY = torch.empty(n ** 3, dtype=torch.float64, device="cuda")
            with pytest.raises(oz2.Oz2Error):
                handle.chain_rescale_be(cp, to_dev(workloads.tensor_batch(n, 1, 9601)), dY, 1)
    finally:
        handle.set_chain_kernel("auto")


def test_chain_kernel_choice():
    """the automatic choice: the HBM kernels (which take the handle's
    workspace for the residue planes) for n <= 8 and n > 16, the LDS kernel
    (no workspace) for 8 < n <= 16"""
    import torch
    import complex_gemm_emulation_amd as oz2
    for n, lds in ((8, False), (9, True), (16, True), (17, False)):
        ops = _ops(n, 9650 + n)
        X = workloads.tensor_batch(n, 2, 9660 + n)
        with oz2.Handle() as h, h.chain_plan(ops, n, 12) as cp:
            dY = torch.empty(2 * n ** 3, dtype=torch.float64, device="cuda")
            h.chain_rescale_be(cp, to_dev(X), dY, 2)
            torch.cuda.synchronize()
            assert (h.workspace_size() == 0) == lds, (n, h.workspace_size())


def _golden_cases():
    path = os.path.join(GOLDEN, "chain_hbm_samples.json")
    with open(path) as f:
        return json.load(f)["cases"]


def _golden_id(c):
    return f"n{c['n']}" + ("" if c.get("modes") is None else "m" + "".join(map(str, c["modes"])))


GOLDEN_CASES = _golden_cases()


@pytest.mark.parametrize("case", range(len(GOLDEN_CASES)), ids=[_golden_id(c) for c in GOLDEN_CASES])
def test_chain_hbm_golden_samples(handle, case):
    """the staged product kernels with 2, 3 and 4 pairs of k chunks (n = 100,
    128, 136, 200, 256; 8 wavefronts per block at 256), in turn and in other
    mode orders (store kinds 1 and 2), with both forms of the base extension:
    seeded entries of each tensor against values the oracle computed once
    (tests/golden/make_chain_hbm_samples.py)"""
    c = GOLDEN_CASES[case]
    n, s, batch, modes = c["n"], c["s"], c["batch"], c.get("modes")
    d = 3 if modes is None else len(modes)
    _say(f"[chain hbm golden] n={n} s={s} batch={batch} modes={modes}")
    ops = _ops(n, c["ops_seed"], d)
    X = workloads.tensor_batch(n, batch, c["x_seed"])
    idx = np.array(c["index"], dtype=np.int64)
    want = np.array([float.fromhex(v) for v in c["value"]])
    for crt in (True, False):
        got, info = _run(handle, ops, n, s, X, batch, modes, crt=crt)
        assert info == (d, c["b"], c["g"]), info
        _check_bitwise(got[idx], want, f"golden n={n} modes={modes} crt={crt}")
