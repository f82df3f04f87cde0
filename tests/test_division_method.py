"""Host check of the divisions the kernels replace: the reciprocal-and-
correction division of the int8 activation quantisers (bl_device.h,
quant_code_fast) and the binary64 product used for the division by 127 in
the GEMM epilogue (gemm_tiles.h, dequant_f64).  Both must give the IEEE-rounded
binary32 quotient, hence the same codes and outputs as a plain division."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_markstein_division_matches_ieee_quotient():
    with tempfile.TemporaryDirectory() as td:
        exe = os.path.join(td, "mk")
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                        os.path.join(HERE, "csrc", "markstein_check.c"), "-lm"], check=True)
        out = subprocess.run([exe, "20000000"], check=True, capture_output=True, text=True).stdout
    n, bad = map(int, out.split())
    assert n == 20000000 and bad == 0
