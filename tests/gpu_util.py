"""Helpers shared by the GPU parity tests: device copies, ulp distances and
the checks of the product's intermediate buffers against the oracle."""
import numpy as np

import oracle


def ordered(x: np.ndarray) -> np.ndarray:
    i = np.ascontiguousarray(x, dtype=np.float64).view(np.int64)
    return np.where(i < 0, np.int64(-(2 ** 63)) - i, i)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in units in the last place (0 for two NaNs; huge for NaN vs number)."""
    a = np.ascontiguousarray(a, dtype=np.float64).reshape(-1)
    b = np.ascontiguousarray(b, dtype=np.float64).reshape(-1)
    d = np.abs(ordered(a).astype(object) - ordered(b).astype(object)).astype(np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    d[both_nan] = 0
    d[np.isnan(a) ^ np.isnan(b)] = np.inf
    return d


def to_dev(x: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to("cuda")


def from_dev(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def words_to_int(words) -> int:
    v = 0
    for w in reversed([int(x) for x in words]):
        v = (v << 32) | w
    nbits = 32 * len(words)
    return v - (1 << nbits) if v >> (nbits - 1) else v


def check_float_parity(got: np.ndarray, want: np.ndarray, label: str, max_ulp: int = 1) -> int:
    """<= max_ulp per entry (NaN where the oracle has NaN); returns the count
    of entries that are not bit-identical."""
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    if np.iscomplexobj(want):
        got = got.view(np.float64)
        want = want.view(np.float64)
    d = ulp_diff(got, want)
    bad = np.nonzero(d > max_ulp)[0]
    assert bad.size == 0, (f"{label}: {bad.size} entries beyond {max_ulp} ulp, first at "
                           f"{bad[:5]}: got {got.reshape(-1)[bad[:5]]} want {want.reshape(-1)[bad[:5]]}")
    return int(np.count_nonzero(d))


def check_chat(words: np.ndarray, want_chat: list, rows, cols, out: int = 0, label: str = ""):
    """words: [outs][n][mp][NL]; want_chat: exact ints (or (re, im) pairs)."""
    for q, (i, j) in enumerate(zip(rows, cols)):
        w = want_chat[q][out] if isinstance(want_chat[q], tuple) else want_chat[q]
        got = words_to_int(words[out, j, i])
        assert got == w, f"{label} c_hat mismatch at ({i},{j}): {got} vs {w}"


def check_residue_planes(planes: np.ndarray, enc: dict, nvec: int, k: int, label: str):
    """planes: product's [sets][s][vpad][kpad]; enc: oracle.encode_vectors."""
    want = enc["planes"]  # [sets][s][nvec][k]
    sets, s = want.shape[0], want.shape[1]
    got = planes[:sets, :s, :nvec, :k]
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{label}: {len(mism)} residue bytes differ, first {mism[:3].tolist()}"
    # padding must be zero (it enters the exact products)
    assert not planes[:sets, :s, nvec:, :].any(), f"{label}: nonzero row padding"
    assert not planes[:sets, :s, :, k:].any(), f"{label}: nonzero k padding"


def check_product_residues(res: np.ndarray, chat_words: np.ndarray, s: int, m: int, n: int,
                           out: int, label: str):
    """res: product's [runs][outs][s][n][mp]; chat_words: oracle's [count][ncomp][4]
    (column-major entry order over m x n)."""
    mods = oracle.max_product_moduli(s)
    total = res[0, out].astype(np.int64)
    for c in range(1, res.shape[0]):
        total = total + res[c, out]
    want = oracle.chat_residues(chat_words[:, out, :], s).reshape(s, n, m)
    for t, mt in enumerate(mods):
        got = total[t, :, :m] % mt
        mism = np.argwhere(got != want[t])
        assert mism.size == 0, f"{label}: modulus {mt}: {len(mism)} residues differ, first {mism[:3].tolist()}"
