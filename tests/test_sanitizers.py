"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code, run
on the CPU: the oracle and the input generator (gcc, tests/sanitize_oracle.c
drives every exported routine on small layers and edge cases), and the
library's host side (hipcc with the sanitizers on the host pass only; the
kernels are compiled but never launched; tests/sanitize_api.cpp drives
validation, size queries, error strings, create() without a usable device
and every entry point with null handles).  Leak detection is on."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = tmp_path / "san_oracle"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "gen", "gen.c"), "-lm"], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_api_under_sanitizers(tmp_path):
    exe = tmp_path / "san_api"
    src = os.path.join(ROOT, "fp8_blockwise_routed_amd", "csrc")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "sanitize_api.cpp"),
           os.path.join(src, "moe_api.cpp"), os.path.join(src, "moe_kernels.hip"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    # the check for a usable device is what create() exercises here: hide any
    env = dict(ENV, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
