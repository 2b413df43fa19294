"""The C-ABI libraries load and export every symbol include/*.h declares, and
its host planner agrees with the independently written oracle (no GPU)."""
import os
import re

import pytest

import complex_gemm_emulation_amd as oz2
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "oz2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oz2_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_match_binding_list():
    assert _declared_symbols() == sorted(oz2.EXPORTED_SYMBOLS)


def test_stream_library_exports_its_header():
    # include/oz2_stream.h: the stream kernels the bench times as HBM ceilings
    import ctypes
    text = open(os.path.join(ROOT, "include", "oz2_stream.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(oz2_[a-z0-9_]+)\s*\(", text)))
    assert names == ["oz2_stream_run"]
    lib = ctypes.CDLL(os.path.join(ROOT, "complex_gemm_emulation_amd", "liboz2_stream.so"))
    for name in names:
        assert hasattr(lib, name), name
    # argument checks return before any launch (no GPU needed)
    fn = lib.oz2_stream_run
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(7, None, None, 16, 1, 2, 0, None) == -1
    assert fn(1, None, None, 16, 1, 2, 0, None) == -3
    assert fn(1, None, ctypes.c_void_p(16), 17, 1, 2, 0, None) == -4
    assert fn(1, None, ctypes.c_void_p(16), 16, 1, 3, 0, None) == -6


def test_library_exports_every_declared_symbol():
    import ctypes
    lib = ctypes.CDLL(oz2.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("s", range(2, 25))
def test_planner_matches_oracle(s):
    # two independent searches for the max-product moduli set, and two
    # independent t(s, k) computations, must agree
    for k in (1, 16, 256, 4096, 8192, 131071, 300000):
        for cplx in (False, True):
            info = oz2.plan_info(s, k, cplx)
            assert info["moduli"] == oracle.max_product_moduli(s)
            # the encoders pack the first plane as the low byte of a_hat
            assert info["moduli"][0] == 256
            assert info["NL"] == oracle.n_limbs(s)
            t = oracle.scaling_width(s, k, cplx)
            assert info["t"] == t, (s, k, cplx)
            assert abs(info["log2M"] - oracle.log2_M(s)) < 1e-9


def test_moduli_for_bits_matches_oracle():
    for k in (16, 256, 4096, 65536, 1 << 20):
        for bits in (24, 40, 53, 70):
            assert oz2.moduli_for_bits(k, bits) == oracle.moduli_for_bits(k, bits)


def test_plan_info_rejects_bad_s():
    with pytest.raises(oz2.Oz2Error):
        oz2.plan_info(1, 10)
    with pytest.raises(oz2.Oz2Error):
        oz2.plan_info(25, 10)


def test_status_strings():
    lib = oz2.lib()
    assert lib.oz2_status_string(0) == b"success"
    assert b"scaling width" in lib.oz2_status_string(3)
    assert lib.oz2_status_string(-3) == b"invalid argument"


def test_prepared_operand_entry_points_reject_null_handles():
    # no GPU needed: argument checks run before any HIP call
    lib = oz2.lib()
    assert lib.oz2_operand_create(None, b"A", 0, b"N", 1, 1, None, 1, 8, None) == -1
    assert lib.oz2_operand_update(None, None, None, 1) == -1
    assert lib.oz2_operand_destroy(None) == -1
    assert lib.oz2_gemm_prepared(None, None, None, None, None, None, 1) == -1


def test_chain_controls_reject_null_handles():
    # no GPU needed: argument checks run before any HIP call
    lib = oz2.lib()
    assert lib.oz2_set_chain_kernel(None, 0) == -1
    assert lib.oz2_set_chain_crt(None, 1) == -1
    assert lib.oz2_chain_plan_info(None, None, None, None) == -1
