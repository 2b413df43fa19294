"""Seeded synthetic inputs for the Ozaki scheme II DGEMM/ZGEMM emulation.

This module holds only random-number generation and array shaping -- none of
the method's arithmetic -- so that the tests, ``bench.py`` and the oracle can
share inputs without sharing any code of the method.

Distributions, as the pages describe their workloads:

* ``uniform``: U(-1, 1) ("Emulating DGEMM and ZGEMM with INT8 Matrix Engines on
  Intel Arc GPUs", Sec. 7 test matrices; "You Only Convert Twice", Sec. 6.2.1
  Uniform dataset).
* ``phi``: (U(0,1) - 1/2) * exp(phi * N(0,1)) (same Sec. 7; the EmuGEMM page
  generates its inputs the same way).
* ``sincos``, ``spike`` and ``cancel``: Sec. 7 and Sec. 8.3 of the Arc page.

No page gives seeds or literal matrices.  Seeds here follow one fixed rule:
seed = 20260000 + 100 * workload + operand, with operand 0 for A, 1 for B,
2 for C, and 3, 4 and 5 for the imaginary parts of A, B and C.

All matrices are returned as flat column-major float64 (or complex128)
numpy arrays with the leading dimension equal to the row count, unless
``ld`` says otherwise.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20260000

# the workloads named by the headline benchmark and its companion cases
WORKLOADS = {
    1: dict(name="dgemm_256_s8", kind="real", m=256, n=256, k=256, s=(8,), transa="N",
            transb="N", alpha=1.0, beta=0.0, dist="uniform"),
    2: dict(name="dgemm_8192_s8_12_16", kind="real", m=8192, n=8192, k=8192, s=(8, 12, 16),
            transa="N", transb="N", alpha=1.0, beta=0.0, dist="phi", phi=0.5),
    3: dict(name="dgemm_4096_wide_s20_24", kind="real", m=4096, n=4096, k=4096, s=(20, 24),
            transa="T", transb="N", alpha=1.5, beta=-0.5, dist="phi", phi=4.0),
    4: dict(name="zgemm_4096_3m_s16", kind="complex", m=4096, n=4096, k=4096, s=(16,),
            transa="C", transb="N", alpha=complex(0.7, -0.3), beta=complex(0.2, 0.1),
            dist="phi", phi=0.5),
    5: dict(name="tensor_chain_n16_b32768_s16", kind="chain", n=16, batch=32768, s=(16,),
            dist="uniform"),
}

# Non-square shapes (m, k, n) at s = 8 and 16, N/N, U(-1, 1) inputs: the
# shape list of the Arc page's Table 10 (Sec. 7.1).  The emulation's run time
# does not depend on the values, so the cheapest distribution to draw is used.
NONSQUARE = dict(id=6, s=(8, 16), dist="uniform",
                 shapes=((8192, 256, 8192), (8192, 1024, 8192), (8192, 32768, 8192),
                         (8192, 65536, 8192), (65536, 4096, 1024), (1024, 4096, 65536),
                         (4000, 8000, 4000), (16384, 2048, 16384)))


def nonsquare_seed(shape_index: int, operand: int) -> int:
    """seed of operand (0 = A, 1 = B) of the shape_index-th non-square shape"""
    return seed(NONSQUARE["id"], 10 * int(shape_index) + int(operand))


def seed(workload: int, operand: int) -> int:
    return SEED_BASE + 100 * int(workload) + int(operand)


def _draw(rng: np.random.Generator, size: int, dist: str, phi: float) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size)
    if dist == "phi":
        u = rng.random(size)
        g = rng.standard_normal(size)
        return (u - 0.5) * np.exp(phi * g)
    raise ValueError(dist)


def real_matrix(rows: int, cols: int, seed_value: int, dist: str = "uniform", phi: float = 0.5,
                ld: int | None = None) -> np.ndarray:
    """rows x cols column-major float64 with leading dimension ld (>= rows);
    padding entries beyond the rows are filled with NaN so that a kernel
    that reads them by mistake shows up in the results."""
    ld = rows if ld is None else ld
    rng = np.random.default_rng(seed_value)
    vals = _draw(rng, rows * cols, dist, phi).reshape(cols, rows)
    if ld == rows:
        return np.ascontiguousarray(vals.reshape(-1))
    out = np.full((cols, ld), np.nan)
    out[:, :rows] = vals
    return out.reshape(-1)


def complex_matrix(rows: int, cols: int, seed_re: int, seed_im: int, dist: str = "uniform",
                   phi: float = 0.5, ld: int | None = None) -> np.ndarray:
    re = real_matrix(rows, cols, seed_re, dist, phi, ld)
    im = real_matrix(rows, cols, seed_im, dist, phi, ld)
    return re + 1j * im


def stored_shape(op: str, rows: int, cols: int) -> tuple[int, int]:
    """(stored rows, stored cols) of a matrix whose op() is rows x cols."""
    return (rows, cols) if op.upper() == "N" else (cols, rows)


def sincos_matrix(rows: int, cols: int, seed_value: int) -> np.ndarray:
    """sin/cos test matrices with random phases (a smooth, structured input)."""
    rng = np.random.default_rng(seed_value)
    i = np.arange(rows)[None, :]
    j = np.arange(cols)[:, None]
    ph = rng.uniform(0, 2 * np.pi, size=2)
    return np.ascontiguousarray((np.sin(0.37 * i + ph[0]) * np.cos(0.11 * j * (i + 1) + ph[1])).reshape(-1))


def spike_matrix(rows: int, cols: int, seed_value: int, factor_log2: int = 40) -> np.ndarray:
    """U(-1,1) with one entry per row 2**factor_log2 times larger (Arc page Sec. 8.3)."""
    rng = np.random.default_rng(seed_value)
    a = rng.uniform(-1.0, 1.0, size=(cols, rows))
    where = rng.integers(0, cols, size=rows)
    a[where, np.arange(rows)] *= 2.0 ** factor_log2
    return np.ascontiguousarray(a.reshape(-1))


def cancel_pair(m: int, n: int, k: int, seed_value: int) -> tuple[np.ndarray, np.ndarray]:
    """A = [X X] (m x k) and B = [Y; -Y + 2^-30 Z] (k x n), X, Y, Z from
    U(-1, 1), k even: C = X (2^-30 Z) is about 2^-30 |A||B| (Arc page
    Sec. 8.3, cancellation).  Column-major flat arrays."""
    rng = np.random.default_rng(seed_value)
    h = k // 2
    X = rng.uniform(-1.0, 1.0, (m, h))
    Y = rng.uniform(-1.0, 1.0, (h, n))
    Z = rng.uniform(-1.0, 1.0, (h, n))
    A = np.concatenate([X, X], axis=1)
    B = np.concatenate([Y, -Y + 2.0 ** -30 * Z], axis=0)
    return A.reshape(-1, order="F"), B.reshape(-1, order="F")


def tensor_batch(n: int, batch: int, seed_value: int) -> np.ndarray:
    """batch independent n x n x n tensors, column-major X[i + n j + n^2 k + n^3 b]."""
    rng = np.random.default_rng(seed_value)
    return rng.uniform(-1.0, 1.0, size=n * n * n * batch)
