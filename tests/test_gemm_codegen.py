"""Generated-code checks of the residue GEMM kernel (no GPU: hipcc
cross-compiles gfx950 assembly here).

The kernel issues its global->LDS loads from inline assembly that writes M0,
a register the compiler reserves.  That is sound only while the compiler
itself uses M0 nowhere in these kernels; and the point of issuing the loads
that way is that the wait before each k step's barrier leaves the loads of
the two following steps in flight (vmcnt(2 steps), not vmcnt(0)).  Both are
properties of the compiler's output, checked here on every kernel instance.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "complex_gemm_emulation_amd", "csrc", "oz2_gemm.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "oz2_gemm.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _kernels(asm):
    bodies = {}
    for m in re.finditer(r"^(_Z\w*residue_gemm16s?_kernel\w*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        lines = [l.split(";")[0].strip() for l in asm[m.end():end].split("\n")]
        bodies[m.group(1)] = [l for l in lines if l and not l.startswith(".")]
    return bodies


def test_m0_written_only_by_the_load_sequence(gemm_asm):
    kernels = _kernels(gemm_asm)
    assert len(kernels) == 4  # {256 x 256 four stages, 128 x 128 two stages} x {real, complex}
    for name, lines in kernels.items():
        for i, l in enumerate(lines):
            if re.search(r"\bm0\b", l):
                # only the inline sequence: s_mov_b32 m0, sX ; s_nop 0 ; global_load_lds_dwordx4
                assert l.startswith("s_mov_b32 m0,"), (name, l)
                assert lines[i + 1] == "s_nop 0", (name, lines[i + 1])
                assert lines[i + 2].startswith("global_load_lds_dwordx4"), (name, lines[i + 2])
        loads = [l for l in lines if l.startswith("global_load_lds")]
        writes = [l for l in lines if l.startswith("s_mov_b32 m0,")]
        assert loads and len(loads) == len(writes), name


def _shape(name):
    # residue_gemm16_kernel<CPLX>: the 256 x 256 tile, 8 waves, four stages;
    # residue_gemm16s_kernel<CPLX>: the 128 x 128 tile, 4 waves, two stages
    return (256, 256, 8, 4) if "residue_gemm16_kernel" in name else (128, 128, 4, 2)


def test_main_loop_keeps_loads_in_flight(gemm_asm):
    kernels = _kernels(gemm_asm)
    assert {_shape(n)[3] for n in kernels} == {2, 4}
    for name, lines in kernels.items():
        bm, bn, nw, nst = _shape(name)
        loads = (bm + bn) * 4 // (64 * nw)  # 1 KiB loads per wave and step
        before_barrier = [lines[i - 1] for i, l in enumerate(lines) if l == "s_barrier"]
        counts = [int(m.group(1)) for w in before_barrier for m in [re.search(r"vmcnt\((\d+)\)", w)] if m]
        assert len(counts) == len(before_barrier), (name, before_barrier)
        if nst == 4:
            # ping-pong: loads are issued three steps ahead, so every barrier
            # (prologue, the staggering ones, 2 per unrolled step) waits with
            # the loads of two later steps in flight; one drain before the epilogue
            assert counts.count(0) == 1 and counts.count(2 * loads) == len(counts) - 1, (name, counts)
            assert len(counts) == 1 + 2 + 2 * 4 + 1, (name, counts)
        else:
            # two stages: the loads of step k + 1 are issued after the barrier
            # that opens step k, so each barrier waits for all loads (vmcnt(0)):
            # two per unrolled loop trip and the drain
            assert counts == [0] * len(counts) and len(counts) == 3, (name, counts)
        assert all(l.startswith("v_mfma_i32_16x16x64_i8") for l in lines if l.startswith("v_mfma")), name


def test_ping_pong_phases(gemm_asm):
    # in the main loop of the 256 x 256 tile, consecutive barriers enclose
    # either a memory phase (a k step's 12 LDS fragment reads and its loads,
    # no MFMA) or a compute phase (the step's 32 16x16x64 MFMAs, no LDS read)
    for name, lines in _kernels(gemm_asm).items():
        if _shape(name)[3] != 4:
            continue
        bars = [i for i, l in enumerate(lines) if l == "s_barrier"]
        phases = []
        for a, b in zip(bars, bars[1:]):
            seg = lines[a + 1:b]
            mf = sum(l.startswith("v_mfma") for l in seg)
            rd = sum(l.startswith("ds_read") for l in seg)
            if mf or rd:
                phases.append((mf, rd))
        loop = [p for p in phases if p in ((32, 0), (0, 12))]
        assert len(loop) >= 8, (name, phases)
        assert all(p in ((32, 0), (0, 12)) for p in phases), (name, phases)
