"""Resource checks of the built gfx950 library (CPU only; needs the ROCm
LLVM tools of the image): no attention or projection kernel keeps per-lane
state in scratch memory beyond its known register spills.

A kernel whose wave state or staging registers end up in scratch (for
instance when a helper lambda is not inlined) still computes the right
results, so the parity tests cannot see it, but it runs several times
slower.  The kernel metadata of the library's code objects states each
kernel's private segment size; this test reads it from the library built in
this tree.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from long_context_tabular_amd import binding as B

LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# (kernel name pattern, largest private segment in bytes): the FP16 two-group
# context kernel sits at the register limit and spills 28 registers outside
# its tile loop, and the GatedLogScale projection (at the 168-register budget
# of three workgroups per CU) a handful around its K loop; every other kernel
# keeps everything in registers
LIMITS = [
    (r"attention_kernelILi0ELi2ELb0E", 128),
    (r"qkv_project_kernelILi2E", 32),
    (r"attention_kernel", 0),
    (r"qkv_project_kernel", 0),
    (r"combine_kernel", 0),
    (r"(scale_queries|amax|pack_kv|scales|fill_)", 0),
]


def _kernel_private_sizes(lib_path: str) -> dict:
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools are not available")
    objcopy, bundler, readelf = tools
    sizes = {}
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin.bin")
        subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", lib_path, os.path.join(d, "lib.so")],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        assert starts, "no offload bundle in the library"
        for i, s in enumerate(starts):
            part = os.path.join(d, f"b{i}.bin")
            with open(part, "wb") as f:
                f.write(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
            co = os.path.join(d, f"b{i}.o")
            r = subprocess.run([bundler, "--type=o", "--unbundle", f"--input={part}",
                                "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                               capture_output=True)
            if r.returncode != 0 or not os.path.getsize(co):
                continue
            notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
            name = None
            for line in notes.splitlines():
                m = re.search(r"^\s+\.name:\s+(\S+)", line)
                if m:
                    name = m.group(1)
                m = re.search(r"\.private_segment_fixed_size:\s+(\d+)", line)
                if m and name:
                    sizes[name] = int(m.group(1))
    return sizes


def test_no_kernel_keeps_state_in_scratch():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    if shutil.which(os.path.join(LLVM, "llvm-readelf")) is None:
        pytest.skip("llvm-readelf missing")
    sizes = _kernel_private_sizes(B.LIB_PATH)
    kernels = [k for k in sizes if "attention_kernel" in k]
    assert len(kernels) >= 7 and any("qkv_project_kernel" in k for k in sizes), sorted(sizes)
    for name, size in sizes.items():
        limit = next((lim for pat, lim in LIMITS if re.search(pat, name)), 0)
        assert size <= limit, f"{name} uses {size} bytes of scratch (limit {limit})"
