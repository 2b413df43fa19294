"""Pins of the OzII-RescaleBE oracle (oracle/rescale_be.py) to what the chain
page ("You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode
Products") and plain integer arithmetic fix -- never to the oracle itself:

* the worked example of Sec. 4.1 / Figure 2 (tests/golden/);
* Eq. (11)-(12) against a brute-force search for the centred representative;
* rescaling on residues (Eq. 15) against big-integer division (Eq. 14);
* mixed-radix digits and base extension (Eq. 24-26) against the integer
  itself, and the exact coverage of the centred interval the page claims
  for the even-modulus-first order;
* the drop planner (Algorithm 2) on a schedule derived by hand;
* the whole chain (Algorithm 7): residues at every stage equal the residues
  of the same chain run in exact big-integer arithmetic, and the FP64 result
  is within the page's reported error range of the exact rational result.
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

rb = oracle.rescale_be
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chain_fig2_rescale_base_extension.json")


def test_fig2_rescale_and_base_extension():
    g = json.load(open(GOLDEN))
    basis = g["basis"]
    R = {p: np.array([r]) for p, r in zip(basis, g["doubled"]["residues"])}
    # the doubled residues are those of 24 (Eq. 11)
    assert [rb.centered(g["doubled"]["value"], p) for p in basis] == g["doubled"]["residues"]
    R2, L = rb.rns_drop(R, basis, g["drop"]["modulus"])
    assert L == g["drop"]["reduced_basis"]
    assert [int(R2[p][0]) for p in L] == g["drop"]["residues"]
    digits = rb.mrc_digits(R2, g["mixed_radix"]["order"])
    assert [int(d[0]) for d in digits] == g["mixed_radix"]["digits"]
    W = rb.mixed_radix_weights(g["mixed_radix"]["order"])
    assert sum(int(d[0]) * w for d, w in zip(digits, W)) == g["mixed_radix"]["value"]
    R3 = rb.base_extend(R2, L, [g["base_extension"]["target"]])
    assert int(R3[g["base_extension"]["target"]][0]) == g["base_extension"]["residue"]
    assert [int(R3[p][0]) for p in basis] == g["base_extension"]["residues"]
    # reconstruction on the full basis, even-first order not needed for odd moduli
    v = rb.reconstruct_fp64(R3, basis, 1.0)
    assert float(v[0]) == g["reconstruct"]["value"]
    assert g["drop"]["alpha"] * float(v[0]) == g["reconstruct"]["scaled"]
    rc = g["rounding_case"]
    R = {p: np.array([rb.centered(rc["doubled"], p)]) for p in basis}
    assert rb.centered(rc["doubled"], 3) == rc["centred_residue_mod_3"]
    R2, L = rb.rns_drop(R, basis, 3)
    q = rb.reconstruct_fp64(R2, L, 1.0)
    assert float(q[0]) == rc["quotient"] and 3 * float(q[0]) == rc["scaled"]


def test_centered_residue_eq11_12():
    # Sec. 2.3 text: the nonnegative remainder 5 modulo 7 becomes -2
    assert rb.centered(5, 7) == -2
    for p in (2, 3, 4, 7, 197, 255, 256):
        for v in range(-3 * p, 3 * p):
            # brute force: the unique representative in [-floor(p/2), ceil(p/2) - 1]
            want = [r for r in range(-(p // 2), (p + 1) // 2) if (v - r) % p == 0]
            assert len(want) == 1
            assert rb.centered(v, p) == want[0]
        v = np.arange(-3 * p, 3 * p)
        assert np.array_equal(rb.centered_array(v, p), [rb.centered(int(x), p) for x in v])


def _random_ints(seed, bound, count):
    """`count` seeded integers in [-bound, bound], spread over all magnitudes"""
    r = random.Random(seed)
    out = []
    for _ in range(count):
        bits = r.randrange(1, bound.bit_length() + 1)
        v = r.randrange(0, min(bound, (1 << bits) - 1) + 1)
        out.append(-v if r.random() < 0.5 else v)
    return out


@pytest.mark.parametrize("s", [8, 16, 24])
def test_rns_drop_is_rounded_division(s):
    basis = list(oracle.max_product_moduli(s))
    P = oracle.moduli_product(basis)
    vals = [v for v in _random_ints(s, P // 2 - 1, 300) if 2 * abs(v) < P]
    vals += [0, 1, -1, P // 2 - 1, -(P // 2) + 1]
    L = list(basis)
    R = {p: np.array([rb.centered(v, p) for v in vals], dtype=np.int64) for p in basis}
    cur = list(vals)
    for _ in range(min(4, s - 1)):
        q = min(L)
        R, L = rb.rns_drop(R, L, q)
        nxt = []
        for v in cur:
            vq = (v - rb.centered(v, q)) // q          # Eq. (14), exact division
            assert (v - rb.centered(v, q)) % q == 0
            assert abs(Fraction(vq) - Fraction(v, q)) <= Fraction(1, 2)
            nxt.append(vq)
        cur = nxt
        for p in L:
            assert [int(x) for x in R[p]] == [rb.centered(v, p) for v in cur], (q, p)


@pytest.mark.parametrize("s,targets", [(16, 7), (12, 5), (24, 9)])
def test_base_extension_recovers_direct_residues(s, targets):
    basis = list(oracle.max_product_moduli(s))
    reduced = basis[:len(basis) - targets]          # the smallest moduli removed
    D = basis[len(basis) - targets:]
    Pr = oracle.moduli_product(reduced)
    vals = [v for v in _random_ints(100 + s, Pr // 2 - 1, 200) if 2 * abs(v) < Pr]
    vals += [0, -1, (Pr - 1) // 2, -((Pr - 1) // 2)]
    R = {p: np.array([rb.centered(v, p) for v in vals], dtype=np.int64) for p in reduced}
    digits = rb.mrc_digits(R, reduced)
    W = rb.mixed_radix_weights(reduced)
    for x, v in enumerate(vals):
        # Eq. (25): the digits are centred and their weighted sum is v itself
        assert sum(int(d[x]) * w for d, w in zip(digits, W)) == v
        for d, q in zip(digits, reduced):
            assert -(q // 2) <= int(d[x]) <= (q + 1) // 2 - 1
    ext = rb.base_extend(R, reduced, D)
    for p in D:
        assert [int(x) for x in ext[p]] == [rb.centered(v, p) for v in vals]


def test_mixed_radix_covers_the_centred_interval_with_even_modulus_first():
    # Sec. 4.4: with the even modulus first the digit sums cover exactly
    # [-floor(P/2), ceil(P/2) - 1]; check every integer of small bases
    for order in ([8, 5, 3], [4, 7, 5], [2, 3], [6, 7, 5, 11]):
        P = math.prod(order)
        vs = np.arange(-(P // 2), (P + 1) // 2, dtype=np.int64)
        R = {p: rb.centered_array(vs, p) for p in order}
        digits = rb.mrc_digits(R, order)
        W = rb.mixed_radix_weights(order)
        back = sum(d * w for d, w in zip(digits, W))
        assert np.array_equal(back, vs), order


def test_horner_is_exact_below_2_53_and_close_above():
    basis = list(oracle.max_product_moduli(16))
    P = oracle.moduli_product(basis)
    rng = np.random.default_rng(7)
    small = [int(x) for x in rng.integers(-(1 << 53), 1 << 53, 200)] + [0, 1, -1, (1 << 53) - 1]
    big = [v for v in _random_ints(8, P // 2 - 1, 200) if 2 * abs(v) < P and abs(v) >= 1 << 53]
    for vals, exact in ((small, True), (big, False)):
        R = {p: np.array([rb.centered(v, p) for v in vals], dtype=np.int64) for p in basis}
        V = rb.reconstruct_fp64(R, basis, 1.0)
        for x, v in enumerate(vals):
            if exact:
                assert V[x] == float(v)
            else:
                # 15 roundings of at most half an ulp each, relative to |v|
                assert abs(Fraction(V[x]) - v) <= abs(v) * Fraction(16, 1 << 53)


def test_greedy_rescale_hand_example():
    # Sec. 4.3 around Eq. (23), basis (7, 5, 3), b = 2: after a product bounded
    # by 12, floor(12/3) = 4 >= 2^2 drops 3 and leaves 4 + 1 = 5 with
    # 2 * 5 < 35; floor(5/5) = 1 < 4 stops.
    assert rb.greedy_rescale(12, 2, [7, 5, 3]) == (1, 5, [5, 7])
    # a bound too small for any drop leaves everything
    assert rb.greedy_rescale(11, 2, [7, 5, 3]) == (0, 11, [3, 5, 7])
    # floor(200/3) + 1 = 67 but 2 * 67 >= 35: the quotient is not recoverable
    assert rb.greedy_rescale(200, 2, [7, 5, 3]) is None
    # b = 1, bound 40: 3 leaves (13 + 1 = 14, 2 * 14 < 35), then 5
    # (2 + 1 = 3, 2 * 3 < 7); one modulus always remains
    assert rb.greedy_rescale(40, 1, [7, 5, 3]) == (2, 3, [7])


def test_drop_plan_hand_example():
    # basis (7, 5, 3), P = 105, b = 2, rho = (3, 3), restoration on:
    #   B = 4; i = 1: B = 12, 2B = 24 < 105; floor(12/3) = 4 >= 2^2 -> drop 3:
    #   B' = 4 + 1 = 5, 2 B' = 10 < 105/3 = 35, L = (7, 5), B = 5, g1 = 1;
    #   floor(5/5) = 1 < 4 -> stop; restore L = (7, 5, 3).
    #   i = 2 (last): B = 15, 2B = 30 < 105; g2 = 0.
    assert rb.drop_plan(2, [3, 3], [7, 5, 3], 1) == [1, 0]
    # without restoration the second product sees P_L = 35: 2 * 15 = 30 < 35 still fits
    assert rb.drop_plan(2, [3, 3], [7, 5, 3], 0) == [1, 0]
    # rho = (3, 4): 2 * 5 * 4 = 40 >= 35 fails only without restoration
    assert rb.drop_plan(2, [3, 4], [7, 5, 3], 1) == [1, 0]
    assert rb.drop_plan(2, [3, 4], [7, 5, 3], 0) is None
    # a first product that overflows the range fails at once
    assert rb.drop_plan(2, [20, 1], [7, 5, 3], 1) is None


def _exact_integer_chain(plan, Xbar):
    """The chain of Algorithm 7 in big-integer arithmetic: products with the
    integer operators, drops as exact rounded divisions (Eq. 14)."""
    stages = []
    v = np.array(Xbar, dtype=object)
    for i in range(len(plan["g"])):
        v = rb.mode_product(v, np.array(plan["Abar"][i], dtype=object), plan["modes"][i])
        stages.append(("product", v))
        if plan["g"][i] > 0:
            for q in plan["drops"][i]:
                v = np.vectorize(lambda x, q=q: (x - rb.centered(int(x), q)) // q, otypes=[object])(v)
            stages.append(("extended", v))
    return stages


@pytest.mark.parametrize("n,s,d", [(4, 16, 3), (8, 16, 3), (8, 12, 3), (4, 16, 1), (4, 16, 2), (8, 16, 5),
                                   (4, 12, 8)])
def test_residue_chain_equals_integer_chain(n, s, d):
    X = workloads.tensor_batch(n, 1, 900 + n + s)
    ops = [workloads.real_matrix(n, n, 910 + q) for q in range(d)]
    plan = rb.prepare_chain(ops, n, s)
    keep = {}
    rb.chain_tensor(X, plan, keep)
    ints = _exact_integer_chain(plan, keep["encoded"][0])
    assert [k for k, _ in ints] == [k for k, _, _ in keep["stages"]]
    P = oracle.moduli_product(plan["basis"])
    for (kind, v), (_, i, R) in zip(ints, keep["stages"]):
        assert max(abs(int(x)) for x in v.reshape(-1)) * 2 < P   # Eq. (19) on the full basis
        for p in plan["basis"]:
            want = np.vectorize(lambda x: rb.centered(int(x), p))(v)
            assert np.array_equal(R[p], want), (kind, i, p)


def _exact_chain(X, ops, n, modes=None):
    """the chain in rational arithmetic; operator i along direction modes[i]
    (i mod 3 by default)"""
    T = np.vectorize(Fraction)(rb.tensor_from_flat(X, n))
    for i, a in enumerate(ops):
        M = np.vectorize(Fraction)(rb.matrix_from_flat(a, n))
        m = i % 3 if modes is None else modes[i]
        T = np.moveaxis(np.tensordot(M, T, axes=([1], [m])), 0, m)
    return np.vectorize(float)(rb.tensor_to_flat(T))


@pytest.mark.parametrize("n,d", [(4, 3), (8, 3), (16, 3), (8, 1), (8, 2), (8, 5), (8, 7), (8, 8), (4, 8)])
def test_chain_accuracy_against_exact(n, d):
    # the abstract reports normwise errors from 2.5e-16 to 2.6e-15 for depths
    # 3 .. 7 and from 7e-14 to 6e-13 at depth 8 (n = 8, 15 moduli of another
    # library's table); the basis here is larger (16 max-product moduli), so
    # those upper ends bound the errors
    X = workloads.tensor_batch(n, 1, 700 + n)
    ops = [workloads.real_matrix(n, n, 710 + q) for q in range(d)]
    Y, plan = rb.rescale_be_chain(X, ops, n, 16, 1)
    assert plan["b"] == 53 and plan["g"][-1] == 0 and len(plan["g"]) == d
    ex = _exact_chain(X, ops, n)
    err = np.linalg.norm(Y - ex) / np.linalg.norm(ex)
    assert err < (6e-13 if d == 8 else 2.6e-15), err


def test_pending_row_scales_fold_into_the_next_operator_on_a_direction():
    # Sec. 5.2: a depth-4 chain applies its fourth operator along direction 1
    # again; the row scales of the first operator are folded into its columns
    # before encoding.  Hand example, n = 2, b = 3:
    #   A1 = [[1, 0], [0, 4]]: row maxima 1, 4 -> E = 1, 3 -> f1 = (2, 0),
    #   A1bar = [[4, 0], [0, 4]];
    #   A4 = [[1, 1], [1, 1]] -> A4 diag(2^-2, 2^0) = [[1/4, 1], [1/4, 1]]:
    #   row maxima 1 -> f4 = (2, 2), A4bar = [[1, 4], [1, 4]];
    #   pending on direction 1 afterwards: f4; on 2 and 3: the identities' f = (2, 2).
    A1 = np.array([[1.0, 0.0], [0.0, 4.0]])
    eye = np.eye(2)
    A4 = np.ones((2, 2))
    Abar, f, pending = rb.effective_operators([A1, eye, eye, A4], 3)
    assert Abar[0].tolist() == [[4, 0], [0, 4]] and f[0].tolist() == [2, 0]
    assert Abar[3].tolist() == [[1, 4], [1, 4]] and f[3].tolist() == [2, 2]
    assert [p.tolist() for p in pending] == [[2, 2], [2, 2], [2, 2]]
    # depth 3: nothing is pending when an operator is encoded
    Abar3, f3, _ = rb.effective_operators([A4, A1, eye], 3)
    assert Abar3[0].tolist() == [[4, 4], [4, 4]] and Abar3[1].tolist() == [[4, 0], [0, 4]]


def test_zero_and_nonfinite_tensors():
    n = 4
    ops = [workloads.real_matrix(n, n, 720 + q) for q in range(3)]
    X = np.zeros(2 * n ** 3)
    X[n ** 3 + 5] = np.inf
    Y, plan = rb.rescale_be_chain(X, ops, n, 16, 2)
    assert np.all(Y[:n ** 3] == 0.0)
    assert np.all(np.isnan(Y[n ** 3:]))


@pytest.mark.parametrize("modes", [[1, 0, 2], [0, 0, 1], [2, 2, 2, 0], [1, 2, 1, 0, 0]])
def test_any_mode_sequence(modes):
    """Algorithm 7 takes any sequence of modes: the residue chain equals the
    big-integer chain and the result is as accurate as the cyclic one"""
    n, s = 8, 16
    d = len(modes)
    X = workloads.tensor_batch(n, 1, 950 + d)
    ops = [workloads.real_matrix(n, n, 960 + q) for q in range(d)]
    plan = rb.prepare_chain(ops, n, s, modes)
    keep = {}
    Y = rb.chain_tensor(X, plan, keep)
    ints = _exact_integer_chain(plan, keep["encoded"][0])
    for (kind, v), (_, i, R) in zip(ints, keep["stages"]):
        for p in plan["basis"]:
            want = np.vectorize(lambda x: rb.centered(int(x), p))(v)
            assert np.array_equal(R[p], want), (kind, i, p)
    ex = _exact_chain(X, ops, n, modes)
    err = np.linalg.norm(Y - ex) / np.linalg.norm(ex)
    assert err < 2.6e-15, err
