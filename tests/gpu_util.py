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
    """Bit-identical wherever the oracle's result is normal, infinite or NaN
    (NaN where the oracle has NaN); within max_ulp where it is subnormal or
    zero, since a subnormal result may be rounded twice (Arc page Sec. 4.4,
    Sec. 9.3).  Returns the count of entries that are not bit-identical."""
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    if np.iscomplexobj(want):
        got = got.view(np.float64)
        want = want.view(np.float64)
    d = ulp_diff(got, want)
    w = want.reshape(-1)
    tiny = np.abs(np.nan_to_num(w, nan=1.0)) < 2.0 ** -1022
    bad = np.nonzero(((d > 0) & ~tiny) | (d > max_ulp))[0]
    assert bad.size == 0, (f"{label}: {bad.size} entries not bit-identical (or beyond {max_ulp} ulp "
                           f"where subnormal), first at {bad[:5]}: got {got.reshape(-1)[bad[:5]]} "
                           f"want {want.reshape(-1)[bad[:5]]}")
    return int(np.count_nonzero(d))


def check_chat(words: np.ndarray, want_chat: list, rows, cols, out: int = 0, label: str = ""):
    """words: [outs][n][mp][NL]; want_chat: exact ints (or (re, im) pairs)."""
    for q, (i, j) in enumerate(zip(rows, cols)):
        w = want_chat[q][out] if isinstance(want_chat[q], tuple) else want_chat[q]
        got = words_to_int(words[out, j, i])
        assert got == w, f"{label} c_hat mismatch at ({i},{j}): {got} vs {w}"


def check_chat_words(words: np.ndarray, chat_words: np.ndarray, m: int, out: int = 0,
                     rows=None, cols=None, label: str = ""):
    """Vectorised c_hat check.  words: the product's [outs][n][mp][N_L] uint32
    (two's complement mod 2^(32 N_L)); chat_words: the oracle's [count][ncomp][4]
    uint64 (two's complement 256-bit) over column-major entries, or over the
    sampled (rows, cols) when given.  The low 32 N_L bits must agree and the
    oracle's higher bits must be the sign extension (|c_hat| < 2^(32 N_L - 1))."""
    nl = words.shape[-1]
    ow = np.ascontiguousarray(chat_words[:, out, :]).view(np.uint32).reshape(-1, 8)
    if rows is None:
        got = words[out][:, :m, :].reshape(-1, nl)
    else:
        got = words[out][np.asarray(cols), np.asarray(rows), :]
    assert got.shape[0] == ow.shape[0], (got.shape, ow.shape)
    low = ow[:, :nl]
    mism = np.nonzero(np.any(got != low, axis=1))[0]
    assert mism.size == 0, f"{label} c_hat words differ at {mism.size} entries, first {mism[:5].tolist()}"
    sign = (low[:, nl - 1] >> 31).astype(np.uint32)
    ext = np.where(sign[:, None] == 1, np.uint32(0xFFFFFFFF), np.uint32(0))
    assert np.all(ow[:, nl:] == ext), f"{label}: oracle c_hat exceeds {32 * nl} bits"


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
                           out: int, label: str, rows=None, cols=None):
    """res: product's [runs][outs][s][n][mp]; chat_words: oracle's [count][ncomp][4]
    (column-major entry order over m x n, or over the sampled (rows, cols))."""
    mods = oracle.max_product_moduli(s)
    total = res[0, out].astype(np.int64)
    for c in range(1, res.shape[0]):
        total = total + res[c, out]
    if rows is None:
        want = oracle.chat_residues(chat_words[:, out, :], s).reshape(s, n, m)
    else:
        want = oracle.chat_residues(chat_words[:, out, :], s)
        total = total[:, np.asarray(cols), np.asarray(rows)]
    for t, mt in enumerate(mods):
        got = (total[t, :, :m] if rows is None else total[t]) % mt
        mism = np.argwhere(got != want[t])
        assert mism.size == 0, f"{label}: modulus {mt}: {len(mism)} residues differ, first {mism[:3].tolist()}"
