"""Checks on the built gfx950 code (CPU only): the device code objects inside the library are
disassembled with the ROCm LLVM tools and scanned.

On gfx950 a 16x16x16 bf16 MFMA occupies the matrix core as long as the 16x16x32 form, and the
compiler's wait states after it were too short for a dependent read (a forward kernel read
stale accumulators for a few rows), so no kernel may contain one.  The direct global->LDS loads
are checked for the wait states that a VALU write of their descriptor SGPRs needs before them
(a build without them read a descriptor word that v_readlane had restored 3 wait states earlier)."""
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


def _sgprs(tok):
    tok = tok.rstrip(",")
    if tok == "m0":
        return {"m0"}
    if tok.startswith("s[") and ":" in tok:
        a, b = tok[2:-1].split(":")
        return set(range(int(a), int(b) + 1))
    if tok.startswith("s") and tok[1:].isdigit():
        return {int(tok[1:])}
    return set()


def test_direct_loads_wait_after_valu_sgpr_writes(tmp_path):
    """On GFX9 a vector-memory instruction that reads an SGPR written by a VALU instruction
    (v_readlane restoring a spilled SGPR, v_readfirstlane, a VOP3 compare) needs 5 wait states
    after that write.  The direct global->LDS loads issued as inline assembly are not padded by
    the compiler's hazard recognizer, so they carry their own s_nop 4; the ones the compiler
    emits itself (from the buffer-to-LDS builtin) it pads.  Every direct load is checked on its
    straight-line predecessors: no VALU write of its descriptor SGPRs or of M0 in the 5 wait
    states before it."""
    asm = _device_asm(tmp_path)
    lines = [ln.split("//")[0].strip() for ln in asm.split("\n")]
    lines = [ln for ln in lines if ln and not ln.endswith(":")]
    loads = [i for i, ln in enumerate(lines) if ln.startswith("buffer_load") and ln.endswith(" lds")]
    assert len(loads) > 100, "direct loads not found"
    asm_form = 0
    bad = []
    for i in loads:
        ops = lines[i].replace(",", " ").split()
        need = set().union(*(_sgprs(t) for t in ops[1:])) | {"m0"}
        prev0 = lines[i - 1].split()
        if prev0[0] == "s_nop" and int(prev0[1], 0) >= 4:
            asm_form += 1
        states = 0
        for j in range(i - 1, max(i - 16, -1), -1):
            if states >= 5 or not need:
                break
            t = lines[j].split()
            dst = _sgprs(t[1]) if len(t) > 1 else set()
            hit = dst & need
            if hit and t[0].startswith("v_"):
                bad.append(" | ".join(lines[j:i + 1]))
                break
            need -= hit
            states += int(t[1], 0) + 1 if t[0] == "s_nop" else 1
    assert asm_form > 100, "the inline-assembly direct loads lost their s_nop"
    assert not bad, f"{len(bad)} direct loads within 5 wait states of a VALU write of their SGPRs: {bad[:3]}"
