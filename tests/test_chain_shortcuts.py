"""The three shortcuts the chain kernels take, pinned on the CPU against the
oracle's own steps of "You Only Convert Twice: Ozaki Scheme II for Chained
Tensor Mode Products" (oracle/rescale_be.py), in exact integers:

- the g drops at once: g successive RnsDrops (Algorithm 1, Eq. 15) by the
  smallest moduli take v to v_g = (v - D) / Q, with Q the product of the
  dropped moduli and D the part of v that its mixed-radix digits over them
  represent; so each kept residue is [r_p Q^-1 - sum_j d_j prod_{l<j} q_l
  Q^-1]_p, from the digits over the dropped moduli alone;
- the final digits in blocks: the mixed-radix digits over all moduli
  (Algorithm 4's MrcDigits, Eq. 24) are those over the first block followed
  by those of (v - A) / M1 over the rest, block by block, whose residues
  come from one such sum each;
- the base extension by the CRT: the residues of v on the dropped moduli
  from those on the kept ones (product M) as [sum_i xi_i [M/m_i]_p -
  alpha [M]_p]_p, xi_i = [r_i (M/m_i)^-1]_{m_i}, alpha the rounding of
  sum_i xi_i / m_i, equal Algorithm 4's BaseExtend for |v| <= (1/2 - 2^-13) M;
  alpha is rounded here as the kernels round it (an FP32 fused multiply-add
  chain, then floor(S + 1/2) in FP32), at both ends of that range.

The kernels compute these sums in FP32 from tables the library builds on the
host (checked against the same definitions by tests/sanitize); here the
identities themselves are checked, with the oracle's rns_drop and
mrc_digits as the reference, on random integers of every size the moduli
allow, for every s and drop count.  The bounds the kernels rely on are
checked too: every sum stays below 2^19 in magnitude."""
import numpy as np
import pytest

import oracle

rb = oracle.rescale_be


def _rand_ints(P, count, seed):
    """count random integers in the centred range of P (Python ints)."""
    rng = np.random.default_rng(seed)
    lim = P // 2 - 1
    out = []
    for _ in range(count):
        words = [int(w) for w in rng.integers(0, 2 ** 32, size=(P.bit_length() + 31) // 32 + 1)]
        v = sum(w << (32 * i) for i, w in enumerate(words)) % (2 * lim + 1)
        out.append(v - lim)
    return out


def _residues(vals, basis):
    return {p: np.array([rb.centered(v, p) for v in vals], dtype=np.int64) for p in basis}


@pytest.mark.parametrize("s", [4, 8, 12, 15, 16])
def test_drops_at_once_equal_repeated_rns_drop(s):
    basis = list(rb.max_product_moduli(s))            # descending: 256 first
    vals = _rand_ints(rb.moduli_product(basis), 64, 7000 + s)
    R = _residues(vals, basis)
    for g in range(1, s):
        dropped = sorted(basis)[:g]                   # smallest first: q_0, q_1, ..
        kept = [p for p in basis if p not in dropped]
        # the oracle: g successive drops
        Rs, L = dict(R), list(basis)
        for q in dropped:
            Rs, L = rb.rns_drop(Rs, L, q)
        # at once: the digits over the dropped moduli, then one sum per kept modulus
        digits = rb.mrc_digits(R, dropped)
        Q = rb.moduli_product(dropped)
        for p in kept:
            qinv = pow(Q % p, -1, p)
            acc = R[p] * rb.centered(qinv, p)
            for j, d in enumerate(digits):
                Wj = rb.moduli_product(dropped[:j])
                acc = acc - d * rb.centered(Wj * qinv % p, p)
            assert np.all(np.abs(acc) < 2 ** 19), (s, g, p)
            assert np.array_equal(rb.centered_array(acc, p), Rs[p]), (s, g, p)


@pytest.mark.parametrize("s", [4, 8, 12, 15, 16])
@pytest.mark.parametrize("split", [4, 8])
def test_digits_in_blocks_equal_one_elimination(s, split):
    """the digits block by block: each block's by elimination among its
    moduli, then the later moduli's residues of (v - A) / M_b by one sum each"""
    basis = list(rb.max_product_moduli(s))
    if split >= s:
        pytest.skip("one block")
    vals = _rand_ints(rb.moduli_product(basis), 64, 7100 + s + split)
    R = _residues(vals, basis)
    want = rb.mrc_digits(R, basis)
    got, rest, Rb = [], list(basis), dict(R)
    while rest:
        block, rest = rest[:split], rest[split:]
        d = rb.mrc_digits(Rb, block)
        got += d
        Mb = rb.moduli_product(block)
        nxt = {}
        for p in rest:
            qinv = pow(Mb % p, -1, p)
            acc = Rb[p] * rb.centered(qinv, p)
            for i, di in enumerate(d):
                acc = acc - di * rb.centered(rb.moduli_product(block[:i]) * qinv % p, p)
            assert np.all(np.abs(acc) < 2 ** 19), (s, split, p)
            nxt[p] = rb.centered_array(acc, p)
        Rb = nxt
    for i, (a, b) in enumerate(zip(got, want)):
        assert np.array_equal(a, b), (s, split, i)
    # and the digits rebuild the integers (Eq. 24)
    W = rb.mixed_radix_weights(basis)
    for k, v in enumerate(vals[:8]):
        assert sum(int(d[k]) * w for d, w in zip(got, W)) == v


def _fma32(a, b, c):
    """fl32(a b + c) for float32 a, b, c, with one rounding: the product of two
    24-bit significands and the sum below are exact in float64 at these
    magnitudes (at most 40 significant bits)"""
    return np.float32(np.float64(a) * np.float64(b) + np.float64(c))


@pytest.mark.parametrize("s", [4, 8, 12, 15, 16])
def test_crt_base_extension_equals_mixed_radix(s):
    basis = list(rb.max_product_moduli(s))            # descending: the kernels' slot order
    for g in range(1, s):
        dropped = sorted(basis)[:g]
        kept = [p for p in basis if p not in dropped]
        M = rb.moduli_product(kept)
        lim = M // 2 - (M + 8191) // 8192              # (1/2 - 2^-13) M, rounded down
        vals = [lim, -lim] + [v % (2 * lim + 1) - lim for v in _rand_ints(M, 48, 7200 + 16 * s + g)]
        R = _residues(vals, kept)
        want = rb.base_extend(R, kept, dropped)
        xi = {p: rb.centered_array(R[p] * rb.centered(pow(M // p % p, -1, p), p), p) for p in kept}
        S = np.zeros(len(vals), dtype=np.float32)
        for p in kept:
            S = np.array([_fma32(np.float32(x), np.float32(1.0) / np.float32(p), v) for x, v in zip(xi[p], S)],
                         dtype=np.float32)
        alpha = np.floor(S + np.float32(0.5)).astype(np.int64)
        exact = [(sum(int(xi[p][k]) * (M // p) for p in kept) - v) // M for k, v in enumerate(vals)]
        assert alpha.tolist() == exact, (s, g)
        for q in dropped:
            acc = -alpha * rb.centered(M % q, q)
            for p in kept:
                acc = acc + xi[p] * rb.centered(M // p % q, q)
            assert np.all(np.abs(acc) < 2 ** 18), (s, g, q)
            assert np.array_equal(rb.centered_array(acc, q), want[q]), (s, g, q)
