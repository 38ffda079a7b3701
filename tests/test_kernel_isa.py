"""ISA-level guards for the GEMM kernels (host-only: compiles to gfx950 assembly, runs nothing).

The direct-to-LDS loads are inline asm that writes m0 (listed as clobbered).  That is only safe
while no compiler-generated instruction in the translation unit relies on m0; this test
compiles gemm.hip with exactly the flags the shipped library is built with (``build.FLAGS``)
and checks that every m0 reference sits inside one of those asm blocks.
"""

import os
import shutil
import subprocess

import pytest

from fp8_quantized_generative_amd import build as lib_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_quantized_generative_amd", "csrc")


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_gemm_m0_only_in_lds_dma_asm(tmp_path):
    asm = str(tmp_path / "gemm.s")
    subprocess.check_call([lib_build.HIPCC, *lib_build.FLAGS, "-Wno-inline-asm",
                           "-S", "--cuda-device-only", "-o", asm, os.path.join(CSRC, "gemm.hip")],
                          stderr=subprocess.DEVNULL)
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
