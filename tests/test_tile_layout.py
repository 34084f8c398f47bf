"""The LDS tile layout the kernels share, checked on the host (no GPU).

Compiles tests/csrc/check_tile_layout.cpp against the kernels' own header
with hipcc (host code only) and runs it: the direct-load map and the read map
must agree, and both read patterns must be free of LDS bank conflicts.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not found")
def test_tile_layout(tmp_path):
    exe = tmp_path / "check_tile_layout"
    src = os.path.join(ROOT, "tests", "csrc", "check_tile_layout.cpp")
    inc = os.path.join(ROOT, "tiled_attention_memory_amd", "csrc")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "-x", "hip", "--offload-arch=gfx950",
           "-std=c++17", "-O1", f"-I{inc}", src, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
