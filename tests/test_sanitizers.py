"""The CPU oracle, the input generator and the launch index arithmetic built
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc and g++, host code
only) and run on small cases: no out-of-bounds access, leak or undefined
operation, every call succeeding."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _have(tool):
    return shutil.which(tool) is not None


@pytest.mark.skipif(not _have("gcc"), reason="gcc not available")
def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = tmp_path / "sanitize_driver"
    subprocess.run(["gcc", *SAN, "-std=c11", "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "native", "sanitize_driver.c"),
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(ROOT, "synth", "gen.c"),
                    "-lm", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "sanitized run ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(not _have("g++"), reason="g++ not available")
def test_launch_index_math_under_sanitizers(tmp_path):
    exe = tmp_path / "index_check"
    subprocess.run(["g++", *SAN, "-std=c++17", "-include", "algorithm",
                    "-I", os.path.join(ROOT, "mixture_experts_layer_gemv_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "index_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "index check ok" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
