"""ISA-level guards for the GEMM kernels (host-only: compiles to gfx950 assembly, runs nothing).

The direct-to-LDS loads are inline asm that writes m0 (listed as clobbered).  That is only safe
while no compiler-generated instruction in the translation unit relies on m0; this test
compiles gemm.hip with exactly the flags the shipped library is built with (``build.FLAGS``)
and checks that every m0 reference sits inside one of those asm blocks.  It also checks the
occupancy the compiler reports for every GEMM instantiation against the waves per SIMD that the
persistent grid and the tile rules assume for its tile shape.
"""

import os
import shutil
import subprocess

import pytest

from fp8_quantized_generative_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_quantized_generative_amd", "csrc")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    """gemm.hip compiled to gfx950 assembly once for the module's tests."""
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    asm = str(tmp_path_factory.mktemp("isa") / "gemm.s")
    subprocess.check_call([lib_build.HIPCC, *lib_build.FLAGS, "-Wno-inline-asm",
                           "-S", "--cuda-device-only", "-o", asm, os.path.join(CSRC, "gemm.hip")],
                          stderr=subprocess.DEVNULL)
    return asm


def test_gemm_m0_only_in_lds_dma_asm(gemm_asm):
    asm = gemm_asm
    inside = outside = 0
    in_asm = False
    for line in open(asm):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        if "m0" in t.split(";")[0]:
            if in_asm:
                inside += 1
            else:
                outside += 1
    assert inside > 0
    assert outside == 0, "compiler-generated code uses m0"


# Waves per SIMD each tile shape must reach (its workgroups per CU times its wavefronts per
# workgroup, over 4 SIMDs): the persistent grid and the grouped tile rule assume these.
_OCCUPANCY = {"Li256ELi256E": 2, "Li256ELi128E": 2, "Li128ELi128E": 2, "Li64ELi128E": 3, "Li64ELi256E": 2,
              "Li256ELi192E": 2}


def test_gemm_occupancy(gemm_asm):
    name, seen = None, 0
    for line in open(gemm_asm):
        if line.startswith("_ZN2rq") and "gemm_fp8_kernel" in line and line.split(";")[0].rstrip().endswith(":"):
            name = line
        elif line.startswith("; Occupancy:") and name is not None:
            shape = [k for k in _OCCUPANCY if "CfgI" + k in name]
            assert len(shape) == 1, name
            assert int(line.split(":")[1]) >= _OCCUPANCY[shape[0]], (name, line)
            name, seen = None, seen + 1
    assert seen >= 5 * 8
