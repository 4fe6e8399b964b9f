"""Host-side check of the decode FFN's launch index arithmetic: the header the
kernel includes is compiled with g++ and checked exhaustively (work items
cover every (column group, slice, expert chunk) exactly once, rows stay inside
their expert's segment, reduction slices partition the units)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_skinny_launch_index_math(tmp_path):
    exe = tmp_path / "index_check"
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-include", "algorithm",
                    "-I", os.path.join(ROOT, "mixture_experts_layer_gemv_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "index_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "index check ok" in r.stdout
