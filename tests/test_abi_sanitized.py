"""The C ABI tests again, on a build with AddressSanitizer and UndefinedBehaviorSanitizer
on the host side (tests/asan_build.py), in a child process that preloads the ASan
runtime. Any sanitizer report fails the run. CPU only: every call in those tests is
rejected, or sized, before the library touches a GPU."""
import os
import subprocess
import sys

import pytest

import asan_build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                    reason="a library is already preloaded in this environment; it is left alone")
def test_abi_under_host_sanitizers():
    lib = asan_build.build()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan_build.asan_runtime(),
        "TAM_LIBATTN_PATH": lib,
        # the interpreter itself is not built for leak checking
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    # the child really runs the sanitized library with the runtime in place
    probe = ("import ctypes, sys; sys.path.insert(0, '.'); import tiled_attention_memory_amd as t; "
             "t.load(); g = ctypes.CDLL(None); print(t.LIB_PATH, hasattr(g, '__asan_init'))")
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(HERE))
    assert r.returncode == 0 and r.stdout.split() == [lib, "True"], r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], env=env, capture_output=True, text=True,
                       timeout=900, cwd=os.path.dirname(HERE))
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert r.returncode == 0
    assert " passed" in r.stdout
