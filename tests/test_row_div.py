"""Host check of the reciprocal-corrected quotient that the GPU epilogues use
to quantise h (one correctly rounded reciprocal per row, then an FMA
correction per value): its E4M3 codes must equal those of the IEEE division
v / (amax / 448) for every |v| <= amax when amax >= 2^-80.  The C checker
walks a strided subset of all float bit patterns for fixed and random amax
(the full walk, stride 1, also passes but takes minutes per amax)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_row_div_codes_match_division(tmp_path):
    exe = tmp_path / "row_div_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "row_div_check.c"), "-lm"],
                   check=True)
    r = subprocess.run([str(exe), "251", "8"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 code mismatches" in r.stdout
