"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (no GPU).

The oracle's C part (128- and 256-bit integer arithmetic, sampled entry
lists, the encoder and residues) and the library's host planners (UBig, the
moduli plans, the persistent chain's planner) are compiled with gcc/g++
-fsanitize=address,undefined and driven over small inputs that reach their
wide-integer and edge paths (tests/sanitize/*_driver.*).  Any sanitizer
report aborts the driver (-fno-sanitize-recover=all), failing the test.
Host code only: the GPU kernels are not built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "complex_gemm_emulation_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd_build, exe):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    return report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_c_part_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = (["gcc"] + SAN + ["-Wno-unknown-pragmas", os.path.join(HERE, "oracle_driver.c"),
                            os.path.join(ROOT, "oracle", "oz2_oracle.c"), "-lm", "-o", exe])
    assert "0 failing calls" in _run(cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_host_planners_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "planner_driver")
    cmd = (["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                                          os.path.join(HERE, "planner_driver.cpp"),
                                          os.path.join(CSRC, "oz2_plan.cpp"),
                                          os.path.join(CSRC, "oz2_chain_plan.cpp"), "-o", exe])
    assert "0 unexpected results" in _run(cmd, exe)
