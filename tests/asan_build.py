"""Host-sanitizer build of libattn.so for the ABI tests (CPU only, never run on a GPU).

Every source is compiled as for the product, plus AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (each -fsanitize= goes to
the host pass through -Xarch_host; the gfx950 code is unchanged). The result,
_build/asan/libattn.so, is loaded by a Python process that preloads clang's
ASan runtime; it exercises the argument checks and the host-side size and
plan computations, which run before any GPU call.

    python tests/asan_build.py      # prints the library path
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from tiled_attention_memory_amd import build as B  # noqa: E402

OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libattn.so")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """clang's shared ASan runtime, which the loading process must preload."""
    rt = glob.glob(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm", "lib", "clang", "*",
                                "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not rt:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under the ROCm clang")
    return rt[0]


def _sources_hash() -> str:
    h = hashlib.sha256(" ".join(SAN).encode())
    for name in B.SOURCES:
        with open(os.path.join(B.CSRC, name), "rb") as f:
            h.update(f.read())
    for name in sorted(os.listdir(B.CSRC)) + sorted(os.listdir(B.INCLUDE)):
        if name.endswith(".h"):
            d = B.CSRC if os.path.exists(os.path.join(B.CSRC, name)) else B.INCLUDE
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f for f in B.COMMON if f != "-O3"]
    cmd = [B.hipcc(), *flags, "-O1", "-g", *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    stamp = os.path.join(OUT, "sources.sha")
    want = _sources_hash()
    if os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == want:
        return LIB
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    cmd = [B.hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *SAN, *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    with open(stamp, "w") as f:
        f.write(want)
    return LIB


if __name__ == "__main__":
    print(build())
