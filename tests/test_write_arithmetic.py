"""Host check of an arithmetic identity the write kernel relies on: its scale
(max - min) / levels is computed as a product with the rounded reciprocal plus one fused
multiply-add correction, which must equal the correctly rounded division for every input
(the quantiser's scale is the range over 15 levels, or 3 at 2 bits: wispaper.ai blog,
section 3, the token-wise quantiser of the core formula).  Exhaustive over all 2^31
non-negative finite binary32 values; the C program is compiled here with gcc."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_scale_division_identity_exhaustive(tmp_path):
    exe = str(tmp_path / "exact_division")
    subprocess.check_call(["gcc", "-O3", "-march=native", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           os.path.join(HERE, "exact_division.c"), "-o", exe, "-lm"])
    r = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "d=15 mismatches=0" in r.stdout and "d=3 mismatches=0" in r.stdout, r.stdout
