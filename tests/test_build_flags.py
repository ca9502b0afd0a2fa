"""The device code of the built library (no GPU needed): the gfx950 code
object carries no packed-fp32 arithmetic, and the build flag that turns it
off is what keeps it out (a small float2 kernel compiled with and without
the flag)."""
import os
import re
import shutil
import subprocess

import pytest

import linear_attention_decode_replay_amd as rs
from linear_attention_decode_replay_amd import build as rs_build

LLVM = "/opt/rocm/llvm/bin"
PACKED_F32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")


def _tools():
    need = [shutil.which("objcopy"), os.path.join(LLVM, "clang-offload-bundler"), os.path.join(LLVM, "llvm-objdump")]
    if not all(t and os.path.exists(t) for t in need):
        pytest.skip("binutils / ROCm LLVM tools not found")
    return need


def _disassemble_library(tmp_path):
    objcopy, bundler, objdump = _tools()
    fatbin = tmp_path / "fatbin.bin"
    code = tmp_path / "gfx950.co"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fatbin}", rs.LIBRARY_PATH, str(tmp_path / "lib.tmp")],
                   check=True)
    subprocess.run([bundler, "--unbundle", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--input={fatbin}", f"--output={code}"], check=True)
    return subprocess.run([objdump, "-d", str(code)], check=True, capture_output=True, text=True).stdout


def test_library_has_no_packed_fp32_instructions(tmp_path):
    dis = _disassemble_library(tmp_path)
    assert "k_replay_step" in dis and "k_conventional_step" in dis
    found = PACKED_F32.findall(dis)
    assert not found, f"{len(found)} packed-fp32 instructions in the gfx950 code"


def test_feature_flag_removes_packed_fp32(tmp_path):
    """Without the flag hipcc -O3 turns float2 arithmetic into packed-fp32
    instructions; with the flags build.py passes, it does not."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    src = tmp_path / "probe.hip"
    src.write_text(
        "#include <hip/hip_runtime.h>\n"
        "typedef float f2 __attribute__((ext_vector_type(2)));\n"
        "__global__ void probe(f2* a, const f2* b, const f2* c, int n) {\n"
        "  int i = blockIdx.x * blockDim.x + threadIdx.x;\n"
        "  if (i < n) { f2 x = a[i]; x = x * b[i] + c[i]; x += b[i]; a[i] = x; }\n"
        "}\n")
    i = rs_build.HIPCC_FLAGS.index("-packed-fp32-ops")
    feature = rs_build.HIPCC_FLAGS[i - 3:i + 1]
    assert feature == ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    counts = []
    for extra in ([], feature):
        out = tmp_path / "probe.s"
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", *extra, "--cuda-device-only", "-S", "-o", str(out),
                        str(src)], check=True, capture_output=True)
        counts.append(len(PACKED_F32.findall(out.read_text())))
    assert counts[0] > 0 and counts[1] == 0, counts
