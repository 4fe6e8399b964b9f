"""The grouped GEMM issues its matrix products as inline assembly (so the
compiler keeps the accumulators in place), which also means the compiler
inserts none of the wait states a matrix instruction needs after a vector
ALU instruction that wrote one of its source registers (two on gfx950).
The kernel adds them itself where it converts weights in registers; this
test compiles the kernel for gfx950 and checks every variant's code for a
vector ALU write followed, within two instructions and with no s_nop
between, by a matrix product that reads the written register.  CPU only:
hipcc cross-compiles without a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_gemv_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", text):
        out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _instructions(body):
    for line in body.split("\n"):
        s = line.strip()
        if s and not s.startswith((".", ";")) and not s.endswith(":"):
            yield s.split(";")[0].strip()


def hazards(asm_text):
    """{kernel: number of VALU-write -> MFMA-read pairs closer than 2 instructions}."""
    found = {}
    for fn in re.findall(r"^(_Z\w+):", asm_text, flags=re.M):
        body = re.split(r"^\.Lfunc_end\d+:", asm_text.split(fn + ":", 1)[1], maxsplit=1, flags=re.M)[0]
        ins = list(_instructions(body))
        bad = 0
        for i, op in enumerate(ins):
            if not op.startswith("v_mfma"):
                continue
            srcs = _regs(",".join(op.split(None, 1)[1].split(",")[1:]))
            for d in (1, 2):
                prev = ins[i - d]
                if prev.startswith("s_nop"):
                    break
                if prev.startswith("v_") and not prev.startswith("v_mfma"):
                    if _regs(prev.split(None, 1)[1].split(",")[0]) & srcs:
                        bad += 1
        found[fn] = bad
    return found


def test_scanner_finds_a_planted_hazard():
    planted = """_Zk:
\tv_perm_b32 v225, v225, v178, s46
\tv_mfma_f32_16x16x32_bf16 v[126:129], v[182:185], v[224:227], v[126:129]
\ts_endpgm
.Lfunc_end0:
_Zok:
\tv_perm_b32 v225, v225, v178, s46
\ts_nop 1
\tv_mfma_f32_16x16x32_bf16 v[126:129], v[182:185], v[224:227], v[126:129]
\ts_endpgm
.Lfunc_end1:
"""
    assert hazards(planted) == {"_Zk": 1, "_Zok": 0}


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not available")
def test_grouped_gemm_has_no_valu_to_mfma_hazard(tmp_path):
    out = tmp_path / "gemm.s"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only",
           "-S", os.path.join(CSRC, "moe_ffn_gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    found = hazards(out.read_text())
    gemm = {k: v for k, v in found.items() if "k_ffn_gemm" in k}
    assert len(gemm) >= 18, sorted(found)
    assert all(v == 0 for v in gemm.values()), {k: v for k, v in gemm.items() if v}
