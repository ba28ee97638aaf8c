"""Build the gfx950 HIP library ``libtri_attn.so`` in-tree with hipcc.

Every source under ``csrc/`` is compiled for gfx950 only; the shared library is
written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libtri_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "bwd_q.hip", "delta_reduce.hip", "block.hip", "block_api.hip", "trimul.hip",
           "trimul_api.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed FP32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# Per-source extra flags.  Both kernels do VALU work on most MFMA results, so MFMA
# results are formed in VGPRs (the register file is unified on gfx950: AGPRs would
# not add capacity, only copies).
EXTRA = {
    "fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "bwd_q.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libtri_attn.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
