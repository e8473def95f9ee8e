"""Builds a copy of ``libdmuon.so`` whose host code runs under AddressSanitizer
and UndefinedBehaviorSanitizer, for checking the planner and the C ABI's
validation on the CPU.  The device code is built as usual (no GPU sanitizer).

Run ``python -m newton_schulz_dmuon_amd.build_sanitized``; the library goes to
``_san/libdmuon.so`` at the repository root.  Load it through ``DMUON_LIB``,
with the clang ASan runtime preloaded, for example::

    DMUON_LIB=$PWD/_san/libdmuon.so ASAN_OPTIONS=detect_leaks=0 \\
    LD_PRELOAD=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so)${LD_PRELOAD:+:$LD_PRELOAD} \\
    python -m pytest tests/test_plan.py tests/test_abi.py -m "not gpu"
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from newton_schulz_dmuon_amd.build import ARCH, COMMON, CSRC, ROOT, SOURCES, hipcc

OUT = os.path.join(ROOT, "_san")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    extra = SAN if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    lib = os.path.join(OUT, "libdmuon.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN, "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
