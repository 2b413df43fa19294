"""CPU oracle for OzII-RescaleBE (persistent Ozaki scheme II tensor mode-product
chains) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product never imports, links or
executes anything under ``oracle/``, and this module shares no code, tables or
constant generators with it.

Source page (cited by title and section; nothing here is copied from it):
"You Only Convert Twice: Ozaki Scheme II for Chained Tensor Mode Products"

* Sec. 2.3, Eq. (11)-(12): centred residues [v]_p.
* Sec. 2.3.1, Eq. (14)-(15), and Algorithm 1 (RnsDrop): rescaling by a
  modulus q on the residues, v' = (v - [v]_q) / q, scale alpha' = alpha q.
* Sec. 2.3.2, Eq. (16)-(17), Sec. 4.4, Eq. (24)-(26), and Algorithm 4
  (MrcDigits, BaseExtend): centred mixed-radix digits by successive modular
  elimination, weights omega_{i,p} = [prod_{j<i} q_j]_p.
* Sec. 4.3, Eq. (21)-(23), and Algorithms 2-3 (DropPlan, Planner): operator
  row-sum bounds rho_i, the greedy drop schedule, the search for b.
* Sec. 5.1, Eq. (27), and Algorithm 5 (Encode, ToRns, ReconstructFP64).
* Sec. 5.2, Eq. (28), and Algorithm 7 (OzII-RescaleBE): encode the tensor
  once with one exponent, a residue product per modulus and mode, g_i drops
  and one base extension after each non-final mode, one reconstruction with
  the scale alpha * Gamma.

Readings where the page leaves a step open:

1. Working basis: the page takes the first s entries of an external library's
   modulus table, of which it prints only the first three (256, 255, 253).
   Here the basis is the max-product set of s pairwise-coprime moduli <= 256
   that the DGEMM emulation uses (``oracle.max_product_moduli``), in
   descending order, so 256 -- the only even modulus -- comes first, as
   Algorithm 4 and ReconstructFP64 require.
2. fl64(q_j V + d_j) in ReconstructFP64 is one rounding of the exact value
   (a fused multiply-add), as fl64(expression) denotes.
3. The scalar scale alpha is a double: alpha <- fl64(alpha q) at each drop,
   in drop order.  Gamma (Eq. 28) is a power of two per entry, so
   sigma = alpha Gamma is exact and the result is fl64(sigma V).
4. One exponent per tensor of a batch (the encoding group of the persistent
   method is "the complete tensor").
5. A chain of depth d applies d operators, by default the i-th along
   direction ((i - 1) mod 3) + 1: depth 3 is the three-direction pass of the
   page's Eq. (1), longer chains revisit the directions in turn (Sec. 6);
   Algorithm 7 also takes any sequence of modes, and so does this oracle.
   A row scale still pending on a direction is folded into the columns of
   the next operator on it before that operator is encoded (Sec. 5.2).
6. Non-finite input entries are outside the algorithm ("assume finite
   operands"); a tensor with any non-finite entry maps to an all-NaN output.

Tensors are flat column-major arrays X[i + n j + n^2 k]; operators are flat
column-major n x n arrays A[i + n j] = A_ij.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from .oz2_oracle import max_product_moduli, moduli_product

MAX_BITS = 53  # Algorithm 3 starts the search at the FP64 significand


# ----------------------------------------------------------------------------
# Residues (Sec. 2.3, Eq. 11-12)
# ----------------------------------------------------------------------------
def centered(v: int, p: int) -> int:
    """[v]_p: the remainder r = v - p floor(v/p), moved to r - p when r >= ceil(p/2)."""
    r = v % p
    return r if r < (p + 1) // 2 else r - p


def centered_array(v: np.ndarray, p: int) -> np.ndarray:
    """Eq. (11) entrywise on an int64 array (|v| < 2^62)."""
    r = np.mod(v, p)
    return np.where(r < (p + 1) // 2, r, r - p)


def to_rns(vbar: np.ndarray, basis: Sequence[int]) -> dict:
    """ToRns (Algorithm 5): one centred residue plane per modulus."""
    return {p: centered_array(vbar, p) for p in basis}


# ----------------------------------------------------------------------------
# Rescaling (Sec. 2.3.1, Eq. 14-15, Algorithm 1)
# ----------------------------------------------------------------------------
def rns_drop(R: dict, L: Sequence[int], q: int):
    """RnsDrop: residues of v' = (v - [v]_q)/q on L without q, by Eq. (15)
    [v']_p = [([v]_p - r_q)(q^{-1} mod p)]_p.  Returns (R', L')."""
    S = R[q]
    out = {}
    for p in L:
        if p == q:
            continue
        out[p] = centered_array((R[p] - S) * pow(q, -1, p), p)
    return out, [p for p in L if p != q]


# ----------------------------------------------------------------------------
# Base extension (Sec. 2.3.2, Sec. 4.4 Eq. 24-26, Algorithm 4)
# ----------------------------------------------------------------------------
def mrc_digits(R: dict, order: Sequence[int]) -> list:
    """MrcDigits: d_i = U_i, then U_j <- [(U_j - d_i)(q_i^{-1} mod q_j)]_{q_j}
    for the later moduli j, in the given order (even modulus first)."""
    U = {p: np.array(R[p], dtype=np.int64, copy=True) for p in order}
    digits = []
    for i, qi in enumerate(order):
        di = U[qi]
        digits.append(di)
        for qj in order[i + 1:]:
            U[qj] = centered_array((U[qj] - di) * pow(qi, -1, qj), qj)
    return digits


def mixed_radix_weights(order: Sequence[int]) -> list:
    """W_i = prod_{j<i} q_j (Eq. 24), as exact integers."""
    W, w = [], 1
    for q in order:
        W.append(w)
        w *= q
    return W


def base_extend(R: dict, order: Sequence[int], targets: Sequence[int]) -> dict:
    """BaseExtend: the residues of the same integer on the target moduli,
    t <- [t + d_i omega_{i,p}]_p with omega_{i,p} = [W_i]_p (Eq. 26); the
    digits are computed once and shared by every target."""
    digits = mrc_digits(R, order)
    W = mixed_radix_weights(order)
    out = dict(R)
    for p in targets:
        t = np.zeros_like(digits[0])
        for di, Wi in zip(digits, W):
            t = centered_array(t + di * centered(Wi, p), p)
        out[p] = t
    return out


# ----------------------------------------------------------------------------
# Encoding and reconstruction (Sec. 5.1 Eq. 27, Algorithm 5)
# ----------------------------------------------------------------------------
def encode_group(values: np.ndarray, b: int):
    """Encode for one group: E with 2^(E-1) <= max|G| < 2^E, e = b - E,
    Gbar = round(2^e G) with ties to even.  An all-zero group gives (0, 0)."""
    v = np.asarray(values, dtype=np.float64)
    mx = float(np.max(np.abs(v))) if v.size else 0.0
    if mx == 0.0:
        return np.zeros(v.shape, dtype=np.int64), 0
    E = math.frexp(mx)[1]
    e = b - E
    return np.rint(np.ldexp(v, e)).astype(np.int64), e


def encode_rows(M: np.ndarray, b: int):
    """Encode with every row of M as one group (operator rows, Eq. 27):
    returns (Mbar, f) with f the row exponents."""
    rows = [encode_group(M[a, :], b) for a in range(M.shape[0])]
    return np.stack([r[0] for r in rows]), np.array([r[1] for r in rows], dtype=np.int64)


def horner_fp64(digits: Sequence[np.ndarray], order: Sequence[int]) -> np.ndarray:
    """V = fl64(d_m); V <- fl64(q_j V + d_j) for j = m-1 .. 1, each step one
    rounding of the exact value (reading 2)."""
    m = len(order)
    flat = [np.asarray(d).reshape(-1) for d in digits]
    out = np.empty(flat[0].size)
    for x in range(flat[0].size):
        V = float(int(flat[m - 1][x]))
        for j in range(m - 2, -1, -1):
            V = float(order[j] * int(V) + int(flat[j][x]))
        out[x] = V
    return out.reshape(np.asarray(digits[0]).shape)


def reconstruct_fp64(R: dict, order: Sequence[int], sigma) -> np.ndarray:
    """ReconstructFP64: centred MRC digits on the ordered basis, FP64 Horner,
    then fl64(sigma * V) entrywise."""
    V = horner_fp64(mrc_digits(R, order), order)
    return np.asarray(sigma, dtype=np.float64) * V


# ----------------------------------------------------------------------------
# Planning (Sec. 4.3 Eq. 21-23, Algorithms 2-3)
# ----------------------------------------------------------------------------
def row_sum_bound(Mbar: np.ndarray) -> int:
    """rho = max_j sum_k |Mbar_jk| (Eq. 21), exact."""
    return max(sum(abs(int(x)) for x in row) for row in Mbar)


def greedy_rescale(B: int, b: int, available: Sequence[int]):
    """The rescaling after a non-final product (Sec. 4.3, around Eq. 23).

    A product leaves entries bounded by B.  Moduli are removed smallest
    first for as long as the quotient bound floor(B/q) still has b bits
    and more than one modulus would remain.  Removing q leaves the bound
    floor(B/q) + 1 (the extra unit covers the rounding of the division) on
    the basis without q, where it must stay recoverable: 2 B' < P_L / q.
    Returns (number removed, the bound left, the moduli left), or None when
    a removal would break that range condition."""
    left = sorted(available)
    P_left = moduli_product(left)
    removed = 0
    while len(left) > 1:
        q = left[0]
        if B // q < (1 << b):
            break
        B, P_left = B // q + 1, P_left // q
        if not 2 * B < P_left:
            return None
        left = left[1:]
        removed += 1
    return removed, B, left


def drop_plan(b: int, rhos: Sequence[int], basis: Sequence[int], tau: int = 1):
    """Drop counts (g_1 .. g_d) of a chain whose products have the operator
    row-sum bounds rhos (Sec. 4.3, Eq. 21-23; the schedule the page calls
    DropPlan), or None.

    The bound starts at 2^b (every encoded entry) and follows the chain:
    each product multiplies it by its rho (Eq. 22) and must keep it
    recoverable on the moduli then available, 2 B < P_L; each non-final
    product is followed by greedy_rescale.  With restoration (tau = 1, the
    proposed method) base extension brings back the whole basis before the
    next product; without it (tau = 0) the next product sees only the
    moduli left.  The last product is decoded directly (g_d = 0)."""
    B = 1 << b
    available = list(basis)
    g = []
    for i, rho in enumerate(rhos):
        B *= rho
        if not 2 * B < moduli_product(available):
            return None
        if i == len(rhos) - 1:
            g.append(0)
            break
        step = greedy_rescale(B, b, available)
        if step is None:
            return None
        removed, B, left = step
        g.append(removed)
        available = list(basis) if tau == 1 else left
    return g


def chain_mode(i: int) -> int:
    """Direction (0-based) of the i-th mode product: the chain visits the
    three directions in turn, 1, 2, 3, 1, 2, ... (Sec. 6: a pass over all
    three directions has depth 3, longer chains revisit them)."""
    return i % 3


def default_modes(d: int) -> list:
    """The directions in turn: 0, 1, 2, 0, 1, ..."""
    return [chain_mode(i) for i in range(d)]


def effective_operators(ops: Sequence[np.ndarray], b: int, modes: Sequence[int] | None = None):
    """The integer operators the chain actually applies (Sec. 5.2, the
    paragraph after Eq. 28): a pending row scale 2^-f on a direction is
    folded into the columns of the next operator on that direction before it
    is encoded, and that operator's row exponents replace it.  Returns
    (Abar list, f list, the exponents left pending on each direction); the
    scales are powers of two, so the folding is exact.  modes[i] is the
    direction (0-based) operator i contracts, the directions in turn if None."""
    n = ops[0].shape[0]
    modes = default_modes(len(ops)) if modes is None else list(modes)
    pending = [np.zeros(n, dtype=np.int64) for _ in range(3)]
    Abar, f = [], []
    for i, M in enumerate(ops):
        m = modes[i]
        Meff = np.ldexp(np.asarray(M, dtype=np.float64), -pending[m][None, :])
        Ai, fi = encode_rows(Meff, b)
        Abar.append(Ai)
        f.append(fi)
        pending[m] = fi
    return Abar, f, pending


def planner(ops: Sequence[np.ndarray], basis: Sequence[int], modes: Sequence[int] | None = None):
    """The significand bits b and drop counts of a chain (Sec. 4.3; the page's
    Planner): the largest b <= 53 whose schedule with restoration passes,
    the row-sum bounds rho_i(b) taken from the effective operators encoded
    at that b (encoding changes with b).  Returns (b, g) or None when no
    b >= 1 passes."""
    def schedule(b):
        return drop_plan(b, [row_sum_bound(A) for A in effective_operators(ops, b, modes)[0]], basis, 1)
    return next(((b, g) for b in range(MAX_BITS, 0, -1) for g in [schedule(b)] if g is not None), None)


# ----------------------------------------------------------------------------
# The chain (Sec. 5.2, Eq. 28, Algorithm 7)
# ----------------------------------------------------------------------------
def tensor_from_flat(x: np.ndarray, n: int) -> np.ndarray:
    """T[i, j, k] = x[i + n j + n^2 k]"""
    return np.asarray(x).reshape(n, n, n).transpose(2, 1, 0)


def tensor_to_flat(T: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(T.transpose(2, 1, 0)).reshape(-1)


def matrix_from_flat(a: np.ndarray, n: int) -> np.ndarray:
    """M[i, j] = a[i + n j]"""
    return np.asarray(a, dtype=np.float64).reshape(n, n).T


def mode_product(T: np.ndarray, M: np.ndarray, mode: int) -> np.ndarray:
    """T x_{mode+1} M: the operator's second index contracts the mode."""
    if mode == 0:
        return np.einsum("ak,kjl->ajl", M, T)
    if mode == 1:
        return np.einsum("ak,ikl->ial", M, T)
    return np.einsum("ak,ijk->ija", M, T)


def residue_mode_product(R: np.ndarray, Ares: np.ndarray, mode: int) -> np.ndarray:
    """One residue product of Algorithm 7 (one modulus, one mode) before its
    reduction, exactly.  Every entry is a sum of n products of centred
    residues of moduli <= 256 (each |r| <= 128), so every partial sum is an
    integer below n 2^14 < 2^53 and float64 arithmetic forms it without
    rounding, in any order: the contraction is a BLAS product on the
    residues as doubles."""
    n = Ares.shape[0]
    if n * 128 * 128 >= 2 ** 53:
        raise ValueError("residue product not exact in float64")
    T, M = np.asarray(R, dtype=np.float64), np.asarray(Ares, dtype=np.float64)
    if mode == 0:
        out = np.tensordot(M, T, axes=([1], [0]))                  # (a, j, l)
    elif mode == 1:
        out = np.moveaxis(np.tensordot(M, T, axes=([1], [1])), 0, 1)  # (i, a, l)
    else:
        out = np.tensordot(T, M, axes=([2], [1]))                  # (i, j, a)
    return out.astype(np.int64)


def prepare_chain(ops_flat: Sequence[np.ndarray], n: int, s: int, modes: Sequence[int] | None = None):
    """Plan and prepare the operators of a chain of depth d = len(ops_flat)
    (Algorithm 7, the steps before the tensor is encoded): returns a dict
    with basis, b, g, the effective integer operators and their row
    exponents, the exponents left pending on each direction, the operator
    residues per modulus, and the dropped moduli per mode.  modes[i]: the direction (0-based) of operator i, the
    directions in turn if None (Algorithm 7 takes any sequence)."""
    basis = list(max_product_moduli(s))           # descending: 256 first
    ops = [matrix_from_flat(a, n) for a in ops_flat]
    modes = default_modes(len(ops)) if modes is None else [int(m) for m in modes]
    if len(modes) != len(ops) or any(m not in (0, 1, 2) for m in modes):
        raise ValueError("one direction in {0, 1, 2} per operator")
    plan = planner(ops, basis, modes)
    if plan is None:
        return None
    b, g = plan
    Abar, f, pending = effective_operators(ops, b, modes)
    drops = []
    for gi in g:
        L = list(basis)
        dq = []
        for _ in range(gi):
            q = min(L)
            dq.append(q)
            L.remove(q)
        drops.append(dq)
    return dict(basis=basis, b=b, g=g, modes=modes, Abar=Abar, f=f, F=pending,
                Ares=[{p: centered_array(A, p) for p in basis} for A in Abar], drops=drops, n=n, s=s)


def chain_tensor(x_flat: np.ndarray, plan: dict, keep: dict | None = None) -> np.ndarray:
    """Algorithm 7 for one tensor; returns the flat column-major result.
    `keep`, if given, receives the residues after every stage (for tests)."""
    n, basis, b = plan["n"], plan["basis"], plan["b"]
    x = np.asarray(x_flat, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return np.full(n ** 3, np.nan)
    T = tensor_from_flat(x, n)
    Xbar, e = encode_group(T, b)
    alpha = math.ldexp(1.0, -e)
    R = to_rns(Xbar, basis)
    if keep is not None:
        keep["encoded"] = (Xbar, e)
        keep["stages"] = []
    for i in range(len(plan["g"])):
        R = {p: centered_array(residue_mode_product(R[p], plan["Ares"][i][p], plan["modes"][i]), p) for p in basis}
        if keep is not None:
            keep["stages"].append(("product", i, dict(R)))
        if plan["g"][i] > 0:
            L = list(basis)
            for q in plan["drops"][i]:
                R, L = rns_drop(R, L, q)
                alpha = alpha * q
            R = base_extend(R, L, [p for p in basis if p not in L])
            if keep is not None:
                keep["stages"].append(("extended", i, dict(R)))
    F1, F2, F3 = plan["F"]   # Gamma (Eq. 28) from the scales left on each direction
    gamma_exp = -(F1[:, None, None] + F2[None, :, None] + F3[None, None, :])
    sigma = np.ldexp(alpha, gamma_exp)
    if keep is not None:
        keep["alpha"] = alpha
    return tensor_to_flat(reconstruct_fp64(R, basis, sigma))


def rescale_be_chain(X: np.ndarray, ops_flat: Sequence[np.ndarray], n: int, s: int, batch: int,
                     modes: Sequence[int] | None = None):
    """Y = X x_{m1} A1 x_{m2} A2 ... (one operator per mode product, the
    directions in turn unless `modes` gives them) for `batch` tensors by
    OzII-RescaleBE; returns (Y flat, plan) or (None, None) when the planner
    finds no b."""
    plan = prepare_chain(ops_flat, n, s, modes)
    if plan is None:
        return None, None
    n3 = n ** 3
    Y = np.empty(n3 * batch)
    for t in range(batch):
        Y[t * n3:(t + 1) * n3] = chain_tensor(X[t * n3:(t + 1) * n3], plan)
    return Y, plan
