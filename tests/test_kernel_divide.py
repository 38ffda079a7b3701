"""The row quantizer's 3-operation quotient equals IEEE FP32 division on its whole domain.

The kernel's arithmetic is replayed in C on the host for every FP16 |x| and every FP16 amax
(5.0e8 pairs); see tests/native/quotient_check.c.  This pins the kernel's algorithm; the GPU
parity tests then pin the kernel's bytes against the oracle.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_markstein_quotient_is_exact(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                           os.path.join(HERE, "native", "quotient_check.c"), "-lm"])
    out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=300)
    assert out.returncode == 0, out.stdout
    assert "mismatches 0" in out.stdout
    assert "pairs 503856640" in out.stdout
