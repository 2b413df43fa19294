"""oz2 -- Ozaki scheme II DGEMM/ZGEMM emulation on AMD Instinct MI355X (gfx950).

Thin Python binding of the C ABI in ``include/oz2.h``: argument marshalling
and host-side extent checks only.  Every step of the computation runs in the
HIP kernels of ``liboz2.so``; torch is used for device memory and streams.
If the library is missing, every entry point raises -- there is no fallback.

Matrices follow BLAS conventions: column-major, op in {'N', 'T', 'C'},
leading dimensions.  A torch tensor passed as a matrix is used through its
data pointer as flat column-major storage, so a row-major torch tensor of
shape (cols, ld) is a column-major (ld x cols) matrix.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["Handle", "Operand", "ChainPlan", "Oz2Error", "lib", "plan_info", "moduli_for_bits",
           "EXPORTED_SYMBOLS", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboz2.so")

# every function declared in include/oz2.h
EXPORTED_SYMBOLS = (
    "oz2_create", "oz2_destroy", "oz2_set_stream", "oz2_set_memory_limit",
    "oz2_get_workspace_size", "oz2_set_timing", "oz2_get_phase_times", "oz2_moduli_for_bits",
    "oz2_plan_info", "oz2_dgemm", "oz2_zgemm", "oz2_dgemm_strided_batched", "oz2_status_string",
    "oz2_set_debug", "oz2_debug_copy", "oz2_test_crt", "oz2_operand_create",
    "oz2_operand_update", "oz2_operand_destroy", "oz2_gemm_prepared", "oz2_chain_plan_create",
    "oz2_chain_plan_info", "oz2_chain_rescale_be", "oz2_chain_plan_destroy", "oz2_dgemm_noalloc",
    "oz2_get_tile_plan", "oz2_set_chain_kernel", "oz2_set_chain_crt",
)

_lib = None


class Oz2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        text = _raw().oz2_status_string(status).decode() if _lib is not None else str(status)
        if status < 0:
            text = f"argument {-status} is invalid"
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def _raw():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, C, D, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_char,
                               ctypes.c_double, ctypes.c_size_t)
        sig = {
            "oz2_create": [P],
            "oz2_destroy": [P],
            "oz2_set_stream": [P, P],
            "oz2_set_memory_limit": [P, SZ],
            "oz2_get_workspace_size": [P, P],
            "oz2_set_timing": [P, I],
            "oz2_get_phase_times": [P, P],
            "oz2_moduli_for_bits": [I64, I, I],
            "oz2_plan_info": [I, I64, I, P, P, P, P],
            "oz2_dgemm": [P, C, C, I64, I64, I64, D, P, I64, P, I64, D, P, I64, I],
            "oz2_dgemm_noalloc": [P, C, C, I64, I64, I64, D, P, I64, P, I64, D, P, I64, I],
            "oz2_get_tile_plan": [P, P, P, P],
            "oz2_set_chain_kernel": [P, I],
            "oz2_set_chain_crt": [P, I],
            "oz2_zgemm": [P, C, C, I64, I64, I64, P, P, I64, P, I64, P, P, I64, I],
            "oz2_dgemm_strided_batched": [P, C, C, I64, I64, I64, D, P, I64, I64, P, I64, I64, D,
                                          P, I64, I64, I64, I],
            "oz2_set_debug": [P, I],
            "oz2_debug_copy": [P, I, P, SZ, P, P],
            "oz2_test_crt": [P, I64, I, P, P],
            "oz2_operand_create": [P, C, I, C, I64, I64, P, I64, I, P],
            "oz2_operand_update": [P, P, P, I64],
            "oz2_operand_destroy": [P],
            "oz2_gemm_prepared": [P, P, P, P, P, P, I64],
            "oz2_chain_plan_create": [P, I64, I, P, P, I, P],
            "oz2_chain_plan_info": [P, P, P, P],
            "oz2_chain_rescale_be": [P, P, P, P, I64],
            "oz2_chain_plan_destroy": [P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I
        L.oz2_status_string.argtypes = [I]
        L.oz2_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    return _raw()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Oz2Error(fn, status)


def plan_info(s: int, k: int, is_complex: bool = False) -> dict:
    mods = (ctypes.c_int32 * 24)()
    t, nl, l2 = ctypes.c_int(), ctypes.c_int(), ctypes.c_double()
    _check("oz2_plan_info", _raw().oz2_plan_info(s, k, int(is_complex), mods, ctypes.byref(t),
                                                  ctypes.byref(nl), ctypes.byref(l2)))
    return dict(moduli=tuple(mods[:s]), t=t.value, NL=nl.value, log2M=l2.value)


def moduli_for_bits(k: int, bits: int = 53, is_complex: bool = False) -> int:
    return int(_raw().oz2_moduli_for_bits(k, bits, int(is_complex)))


def _extent(rows: int, cols: int, ld: int) -> int:
    return 0 if rows == 0 or cols == 0 else (cols - 1) * ld + rows


def _dev_ptr(x, dtype_name: str, need: int, what: str):
    """Device pointer of a CUDA torch tensor holding at least `need` elements."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    want = {"f64": torch.float64, "c128": torch.complex128, "u8": torch.uint8,
            "u32": torch.int32}[dtype_name]
    if x.dtype != want:
        raise TypeError(f"{what} must have dtype {want}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{what} must be a device (cuda) tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if x.numel() < need:
        raise ValueError(f"{what} holds {x.numel()} elements, the call needs {need}")
    return ctypes.c_void_p(x.data_ptr())


class Operand:
    """A prepared operand (oz2_operand_create): the exponents and residue
    planes of op(A) (side 'A') or op(B) (side 'B') kept on the device."""

    def __init__(self, ptr, side, cplx, trans, rows, k, s):
        self._p = ptr
        self.side, self.cplx, self.trans, self.rows, self.k, self.s = side, cplx, trans, rows, k, s

    def close(self) -> None:
        if self._p is not None and self._p.value:
            _raw().oz2_operand_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class ChainPlan:
    """A planned persistent tensor-mode chain (oz2_chain_plan_create):
    significand bits b, drop counts g and the operators' residues on the
    device, reusable for any number of tensor batches."""

    MAX_DEPTH = 8

    def __init__(self, ptr, n, s):
        self._p = ptr
        self.n, self.s = n, s
        d = ctypes.c_int()
        b = ctypes.c_int()
        g = (ctypes.c_int * self.MAX_DEPTH)()
        _check("oz2_chain_plan_info", _raw().oz2_chain_plan_info(ptr, ctypes.byref(d), ctypes.byref(b), g))
        self.depth, self.b, self.g = d.value, b.value, tuple(g[:d.value])

    def close(self) -> None:
        if self._p is not None and self._p.value:
            _raw().oz2_chain_plan_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class Handle:
    """An oz2 handle bound to the current device; work goes to torch's
    current stream at the time of each call unless a stream is given."""

    def __init__(self, stream=None):
        h = ctypes.c_void_p()
        _check("oz2_create", _raw().oz2_create(ctypes.byref(h)))
        self._h = h
        self._stream = stream

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _raw().oz2_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---------------------------------------------------------------- config
    def _bind_stream(self) -> None:
        import torch
        st = self._stream if self._stream is not None else torch.cuda.current_stream()
        _raw().oz2_set_stream(self._h, ctypes.c_void_p(st.cuda_stream))

    def set_memory_limit(self, nbytes: int) -> None:
        _check("oz2_set_memory_limit", _raw().oz2_set_memory_limit(self._h, nbytes))

    def workspace_size(self) -> int:
        v = ctypes.c_size_t()
        _check("oz2_get_workspace_size", _raw().oz2_get_workspace_size(self._h, ctypes.byref(v)))
        return v.value

    def set_timing(self, enable: bool) -> None:
        _check("oz2_set_timing", _raw().oz2_set_timing(self._h, int(enable)))

    def phase_times(self) -> list:
        arr = (ctypes.c_float * 4)()
        _check("oz2_get_phase_times", _raw().oz2_get_phase_times(self._h, arr))
        return list(arr)

    def tile_plan(self) -> dict:
        """Blocking of the last product (oz2_get_tile_plan): block sides and
        which operand's encoded block was kept ('untiled', 'A', 'B', 'prepared')."""
        mb, nb, held = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
        _check("oz2_get_tile_plan", _raw().oz2_get_tile_plan(self._h, ctypes.byref(mb), ctypes.byref(nb),
                                                             ctypes.byref(held)))
        return dict(mb=mb.value, nb=nb.value, held=("untiled", "A", "B", "prepared")[held.value])

    def set_debug(self, enable: bool) -> None:
        _check("oz2_set_debug", _raw().oz2_set_debug(self._h, int(enable)))

    # ------------------------------------------------------------------ BLAS
    @staticmethod
    def _stored(op: str, rows: int, cols: int):
        return (rows, cols) if op.upper() == "N" else (cols, rows)

    def dgemm(self, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s):
        ra, ca = self._stored(transa, m, k)
        rb, cb = self._stored(transb, k, n)
        need_ab = m > 0 and n > 0 and k > 0 and alpha != 0.0
        pa = _dev_ptr(A, "f64", _extent(ra, ca, lda), "A") if need_ab else None
        pb = _dev_ptr(B, "f64", _extent(rb, cb, ldb), "B") if need_ab else None
        pc = _dev_ptr(C, "f64", _extent(m, n, ldc), "C") if m > 0 and n > 0 else None
        self._bind_stream()
        _check("oz2_dgemm", _raw().oz2_dgemm(self._h, transa.encode(), transb.encode(), m, n, k,
                                             float(alpha), pa, lda, pb, ldb, float(beta), pc,
                                             ldc, s))

    def dgemm_noalloc(self, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s):
        """oz2_dgemm_noalloc: the same product with the library's fixed device
        scratch as workspace (no device allocation during the call)."""
        ra, ca = self._stored(transa, m, k)
        rb, cb = self._stored(transb, k, n)
        need_ab = m > 0 and n > 0 and k > 0 and alpha != 0.0
        pa = _dev_ptr(A, "f64", _extent(ra, ca, lda), "A") if need_ab else None
        pb = _dev_ptr(B, "f64", _extent(rb, cb, ldb), "B") if need_ab else None
        pc = _dev_ptr(C, "f64", _extent(m, n, ldc), "C") if m > 0 and n > 0 else None
        self._bind_stream()
        _check("oz2_dgemm_noalloc", _raw().oz2_dgemm_noalloc(self._h, transa.encode(), transb.encode(), m, n,
                                                             k, float(alpha), pa, lda, pb, ldb, float(beta),
                                                             pc, ldc, s))

    def zgemm(self, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s):
        ra, ca = self._stored(transa, m, k)
        rb, cb = self._stored(transb, k, n)
        alpha, beta = complex(alpha), complex(beta)
        need_ab = m > 0 and n > 0 and k > 0 and alpha != 0
        pa = _dev_ptr(A, "c128", _extent(ra, ca, lda), "A") if need_ab else None
        pb = _dev_ptr(B, "c128", _extent(rb, cb, ldb), "B") if need_ab else None
        pc = _dev_ptr(C, "c128", _extent(m, n, ldc), "C") if m > 0 and n > 0 else None
        al = (ctypes.c_double * 2)(alpha.real, alpha.imag)
        be = (ctypes.c_double * 2)(beta.real, beta.imag)
        self._bind_stream()
        _check("oz2_zgemm", _raw().oz2_zgemm(self._h, transa.encode(), transb.encode(), m, n, k,
                                             al, pa, lda, pb, ldb, be, pc, ldc, s))

    def dgemm_strided_batched(self, transa, transb, m, n, k, alpha, A, lda, strideA, B, ldb,
                              strideB, beta, C, ldc, strideC, batch, s):
        ra, ca = self._stored(transa, m, k)
        rb, cb = self._stored(transb, k, n)
        live = batch > 0 and m > 0 and n > 0
        need_ab = live and k > 0 and alpha != 0.0
        last = max(batch - 1, 0)
        pa = _dev_ptr(A, "f64", last * strideA + _extent(ra, ca, lda), "A") if need_ab else None
        pb = _dev_ptr(B, "f64", last * strideB + _extent(rb, cb, ldb), "B") if need_ab else None
        pc = _dev_ptr(C, "f64", last * strideC + _extent(m, n, ldc), "C") if live else None
        self._bind_stream()
        _check("oz2_dgemm_strided_batched",
               _raw().oz2_dgemm_strided_batched(self._h, transa.encode(), transb.encode(), m, n,
                                                k, float(alpha), pa, lda, strideA, pb, ldb,
                                                strideB, float(beta), pc, ldc, strideC, batch, s))

    # ------------------------------------------------------ prepared operands
    def prepare(self, side, trans, rows, k, X, ld, s, cplx=False) -> Operand:
        """Scan and encode op(X) once (oz2_operand_create): side 'A' gives
        op(A) with rows = m, side 'B' gives op(B) with rows = n."""
        side, trans = side.upper(), trans.upper()
        if side == "A":
            r, c = self._stored(trans, rows, k)
        else:
            r, c = self._stored(trans, k, rows)
        px = _dev_ptr(X, "c128" if cplx else "f64", _extent(r, c, ld), "X")
        out = ctypes.c_void_p()
        self._bind_stream()
        _check("oz2_operand_create",
               _raw().oz2_operand_create(self._h, side.encode(), int(cplx), trans.encode(), rows, k,
                                         px, ld, s, ctypes.byref(out)))
        return Operand(out, side, cplx, trans, rows, k, s)

    def update(self, op: Operand, X, ld) -> None:
        """Re-encode new data of the same shape into `op` (oz2_operand_update)."""
        if op.side == "A":
            r, c = self._stored(op.trans, op.rows, op.k)
        else:
            r, c = self._stored(op.trans, op.k, op.rows)
        px = _dev_ptr(X, "c128" if op.cplx else "f64", _extent(r, c, ld), "X")
        self._bind_stream()
        _check("oz2_operand_update", _raw().oz2_operand_update(self._h, op._p, px, ld))

    def gemm_prepared(self, pa: Operand, pb: Operand, alpha, beta, C, ldc) -> None:
        """C <- alpha op(A) op(B) + beta C from two prepared operands."""
        m, n = pa.rows, pb.rows
        alpha, beta = complex(alpha), complex(beta)
        pc = _dev_ptr(C, "c128" if pa.cplx else "f64", _extent(m, n, ldc), "C")
        al = (ctypes.c_double * 2)(alpha.real, alpha.imag)
        be = (ctypes.c_double * 2)(beta.real, beta.imag)
        self._bind_stream()
        _check("oz2_gemm_prepared", _raw().oz2_gemm_prepared(self._h, pa._p, pb._p, al, be, pc, ldc))

    # ------------------------------------------------- persistent chains
    def chain_plan(self, ops, n, s, modes=None) -> ChainPlan:
        """Plan Y = X x_{m1} A1 x_{m2} A2 ... by OzII-RescaleBE
        (oz2_chain_plan_create): ops is a sequence of depth host n x n
        column-major arrays; modes the directions in {1, 2, 3}, by default
        1, 2, 3, 1, ..."""
        mats = [np.ascontiguousarray(np.asarray(M, dtype=np.float64).reshape(-1)) for M in ops]
        for M in mats:
            if M.size < n * n:
                raise ValueError(f"operator holds {M.size} entries, n x n needs {n * n}")
        out = ctypes.c_void_p()
        ptrs = (ctypes.c_void_p * max(1, len(mats)))(*[M.ctypes.data_as(ctypes.c_void_p) for M in mats])
        pm = None
        if modes is not None:
            if len(modes) != len(mats):
                raise ValueError("one mode per operator")
            pm = (ctypes.c_int * len(mats))(*[int(m) for m in modes])
        _check("oz2_chain_plan_create",
               _raw().oz2_chain_plan_create(self._h, n, len(mats), ptrs, pm, s, ctypes.byref(out)))
        return ChainPlan(out, n, s)

    CHAIN_KERNELS = ("auto", "lds", "hbm")

    def set_chain_kernel(self, kernel: str) -> None:
        """Which kernels run persistent chains (oz2_set_chain_kernel): 'auto'
        (LDS for 8 < n <= 16, else HBM), 'lds' or 'hbm'."""
        _check("oz2_set_chain_kernel", _raw().oz2_set_chain_kernel(self._h, self.CHAIN_KERNELS.index(kernel)))

    def set_chain_crt(self, enable: bool) -> None:
        """Base extension of the chain kernels (oz2_set_chain_crt): the CRT
        form where the plan allows it (True, the default) or the mixed-radix
        form after every product (False)."""
        _check("oz2_set_chain_crt", _raw().oz2_set_chain_crt(self._h, 1 if enable else 0))

    def chain_rescale_be(self, plan: ChainPlan, X, Y, batch) -> None:
        """Run a planned chain on `batch` tensors (oz2_chain_rescale_be)."""
        need = batch * plan.n ** 3
        px = _dev_ptr(X, "f64", need, "X") if batch > 0 else None
        py = _dev_ptr(Y, "f64", need, "Y") if batch > 0 else None
        self._bind_stream()
        _check("oz2_chain_rescale_be", _raw().oz2_chain_rescale_be(self._h, plan._p, px, py, batch))

    def tensor_mode_chain(self, X, A, B, C, n, batch, s, Y=None, work=None):
        """Y = X x1 A x2 B x3 C for `batch` independent n x n x n tensors
        (column-major X[i + n j + n^2 k + n^3 b]) and shared n x n operators,
        each mode one emulated product with its own per-fiber and
        per-operator-row scales ("You Only Convert Twice", Sec. 2.1 Eq. (5)
        and Sec. 5.1): mode 1 is A X_(1); modes 2 and 3 are strided batches
        of slice x operator^T.  Returns Y (allocated if not given)."""
        import torch
        n2, n3 = n * n, n * n * n
        total = n3 * batch
        if Y is None:
            Y = torch.empty(total, dtype=torch.float64, device=X.device)
        if work is None:
            work = torch.empty(total, dtype=torch.float64, device=X.device)
        # X -> Y (mode 1) -> work (mode 2) -> Y (mode 3)
        self.dgemm("N", "N", n, n2 * batch, n, 1.0, A, n, X, n, 0.0, Y, n, s)
        self.dgemm_strided_batched("N", "T", n, n, n, 1.0, Y, n, n2, B, n, 0, 0.0, work, n, n2,
                                   n * batch, s)
        self.dgemm_strided_batched("N", "T", n2, n, n, 1.0, work, n2, n3, C, n, 0, 0.0, Y, n2, n3,
                                   batch, s)
        return Y

    # ------------------------------------------------------------ test hooks
    def debug_copy(self, which: int) -> np.ndarray:
        """Intermediate buffer `which` of the last call, copied to the host
        (see oz2_debug_copy in include/oz2.h for the layouts)."""
        nbytes = ctypes.c_size_t()
        dims = (ctypes.c_int64 * 5)()
        _check("oz2_debug_copy", _raw().oz2_debug_copy(self._h, which, None, 0,
                                                       ctypes.byref(nbytes), dims))
        dtype = {0: np.uint64, 1: np.uint64, 2: np.int8, 3: np.int8, 4: np.uint8, 5: np.uint32}[which]
        out = np.empty(nbytes.value // np.dtype(dtype).itemsize, dtype=dtype)
        _check("oz2_debug_copy", _raw().oz2_debug_copy(self._h, which, out.ctypes.data_as(ctypes.c_void_p),
                                                       out.nbytes, ctypes.byref(nbytes), dims))
        d = [int(x) for x in dims]
        if which in (2, 3):
            # k-panels [sets][s][k_pad/64][rows_pad][64] -> [sets][s][rows_pad][k_pad]
            panels = out.reshape(d[0], d[1], d[2], d[3], d[4])
            return np.ascontiguousarray(panels.transpose(0, 1, 3, 2, 4)).reshape(d[0], d[1], d[3], d[2] * d[4])
        if which == 4:
            return out.reshape(d[4], d[0], d[1], d[2], d[3])
        if which == 5:
            return out.reshape(d[0], d[2], d[3], d[4])
        return out

    def test_crt(self, residues, s: int, words) -> None:
        """CRT of residues (uint8 device tensor [s][count]) into N_L int32
        words per entry (int32 device tensor [count][N_L])."""
        count = residues.numel() // s
        nl = plan_info(s, 1)["NL"]
        pr = _dev_ptr(residues, "u8", s * count, "residues")
        pw = _dev_ptr(words, "u32", count * nl, "words")
        self._bind_stream()
        _check("oz2_test_crt", _raw().oz2_test_crt(self._h, count, s, pr, pw))
