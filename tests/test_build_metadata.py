"""The built library's gfx950 kernels use no scratch memory.

A kernel that spills registers or keeps an array in private memory (for
instance an accumulator indexed at run time) runs many times slower; the
code-object metadata of our own build says so before any GPU run.  Host-only:
reads the device code objects bundled into libdmuon.so with the ROCm LLVM
tools."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "newton_schulz_dmuon_amd", "libdmuon.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernel_metadata(tmp_path):
    fat = tmp_path / "fatbin.bin"
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fat}", LIB], check=True, capture_output=True)
    blob = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), blob)]
    kernels = {}
    for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(blob)])):
        part = tmp_path / f"bundle{n}.bin"
        part.write_bytes(blob[a:b])
        co = tmp_path / f"co{n}.o"
        r = subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={part}",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                           capture_output=True, text=True)
        if r.returncode != 0 or not co.exists() or co.stat().st_size == 0:
            continue
        notes = subprocess.run([TOOLS[2], "--notes", str(co)], capture_output=True, text=True).stdout
        name = None
        for line in notes.splitlines():
            m = re.match(r"\s+\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
                kernels.setdefault(name, {})
                continue
            m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)", line)
            if m and name:
                kernels[name][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="ROCm LLVM tools missing")
def test_kernels_use_no_scratch(tmp_path):
    kernels = kernel_metadata(tmp_path)
    names = " ".join(kernels)
    for k in ("ns_gemm_kernel", "ns_gemm_small_kernel", "momentum_orient_kernel", "adamw_kernel",
              "pack_copy_kernel"):
        assert k in names, f"{k} missing from the code objects"
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)}
    assert not bad, f"kernels using scratch: {bad}"
