"""The work-unit scheduler the kernels share, checked on the host (no GPU).

Compiles tests/csrc/check_sched.cpp against the kernels' own header with hipcc
(host code only) and runs it: every unit is dispatched once, all XCDs get work
and each XCD walks its units heaviest first.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not found")
def test_scheduler(tmp_path):
    exe = tmp_path / "check_sched"
    src = os.path.join(ROOT, "tests", "csrc", "check_sched.cpp")
    inc = os.path.join(ROOT, "tiled_attention_memory_amd", "csrc")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "-x", "hip", "--offload-arch=gfx950",
           "-std=c++17", "-O1", f"-I{inc}", src, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
