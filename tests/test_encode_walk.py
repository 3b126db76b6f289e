"""The oracle's FP32 -> E4M3 encoder over all 2^32 FP32 bit patterns against
an independent nearest-code search (tests/encode_walk.c: binary search over
the 127 non-negative E4M3 values built from the closed form, ties to the
even code, saturation at 448, sign kept, NaN to +0).  CPU only; about ten
seconds on eight cores."""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_encode_all_fp32_patterns(tmp_path):
    lib = oracle.build(force=False)
    exe = tmp_path / "encode_walk"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "encode_walk.c"), "-ldl", "-lm"], check=True)
    r = subprocess.run([str(exe), lib], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("0 mismatches over 4294967296 patterns"), r.stdout
