"""Checks on the built gfx950 code (CPU only): the device code objects inside the library are
disassembled with the ROCm LLVM tools and scanned.

On gfx950 a 16x16x16 bf16 MFMA occupies the matrix core as long as the 16x16x32 form, and the
compiler's wait states after it were too short for a dependent read (a forward kernel read
stale accumulators for a few rows), so no kernel may contain one."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "triangular_attention_amd", "libtri_attn.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _device_asm(tmp_path):
    bundler = os.path.join(LLVM, "clang-offload-bundler")
    objdump = os.path.join(LLVM, "llvm-objdump")
    if not (os.path.exists(LIB) and os.path.exists(bundler) and os.path.exists(objdump) and shutil.which("objcopy")):
        pytest.skip("library or ROCm LLVM tools not available")
    fat = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fat)], check=True)
    data = fat.read_bytes()
    starts = []
    i = data.find(MAGIC)
    while i >= 0:
        starts.append(i)
        i = data.find(MAGIC, i + 1)
    assert starts, "no offload bundle in the library"
    asm = []
    for n, s in enumerate(starts):
        end = starts[n + 1] if n + 1 < len(starts) else len(data)
        part = tmp_path / f"b{n}.bin"
        part.write_bytes(data[s:end])
        co = tmp_path / f"b{n}.co"
        r = subprocess.run([bundler, "--unbundle", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                            f"--input={part}", f"--output={co}"], capture_output=True)
        if r.returncode != 0 or not co.exists() or co.stat().st_size == 0:
            continue
        asm.append(subprocess.run([objdump, "-d", str(co)], capture_output=True, text=True, check=True).stdout)
    return "\n".join(asm)


def test_no_16x16x16_products(tmp_path):
    asm = _device_asm(tmp_path)
    assert asm.count("v_mfma_f32_16x16x32_bf16") > 1000, "device code not found"
    assert "v_mfma_f32_16x16x16" not in asm
