"""ctypes binding of ``libtri_attn.so`` (the C ABI declared in include/tri_attn.h,
include/tri_attn_block.h and include/tri_mul.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Loading fails loudly when the library has not been
built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# TRI_ATTN_LIBRARY points the binding at another build of the same sources (the host-sanitizer
# build of the CPU checks); by default the in-tree library
LIB_PATH = os.environ.get("TRI_ATTN_LIBRARY") or os.path.join(HERE, "libtri_attn.so")

STATUS = {
    0: "TRI_ATTN_OK",
    1: "TRI_ATTN_ERR_NULL",
    2: "TRI_ATTN_ERR_SHAPE",
    3: "TRI_ATTN_ERR_UNSUPPORTED",
    4: "TRI_ATTN_ERR_ALIGN",
    5: "TRI_ATTN_ERR_LAUNCH",
    6: "TRI_ATTN_ERR_WORKSPACE",
}

#: every symbol include/tri_attn.h declares
EXPORTS = (
    "tri_attn_fwd",
    "tri_attn_bwd_delta",
    "tri_attn_bwd",
    "tri_attn_reduce_dq",
    "tri_attn_reduce_dbias",
    "tri_attn_bwd_bf16p",
    "tri_attn_reduce_dq_bf16p",
    "tri_attn_reduce_dbias_bf16p",
    "tri_attn_bwd_chunked_workspace",
    "tri_attn_bwd_chunked",
    "tri_attn_bwd_chunked_noalloc",
    "tri_attn_noalloc_scratch_bytes",
    "tri_attn_workspace",
    "tri_attn_workspace_single_pass",
    "tri_attn_status_string",
    "tri_attn_version",
)

#: every symbol include/tri_attn_block.h declares
BLOCK_EXPORTS = (
    "tri_block_workspace",
    "tri_block_ln_proj",
    "tri_block_gate_out",
    "tri_block_gate_out_bwd",
    "tri_block_proj_bwd_dz",
    "tri_block_proj_bwd_dw",
    "tri_block_reduce_wgrad",
)

#: every symbol include/tri_mul.h declares
TRIMUL_EXPORTS = (
    "tri_mul_workspace",
    "tri_mul_in_fwd",
    "tri_mul_contract",
    "tri_mul_out_fwd",
    "tri_mul_out_bwd",
    "tri_mul_contract_bwd",
    "tri_mul_in_bwd",
    "tri_mul_in_bwd_dz",
    "tri_mul_in_bwd_dw",
    "tri_mul_reduce_wgrad",
)


class Dims(ctypes.Structure):
    """Mirror of ``tri_attn_dims``."""
    _fields_ = [
        ("B", ctypes.c_int64),
        ("N_o", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("scale", ctypes.c_float),
    ]


class BlockDims(ctypes.Structure):
    """Mirror of ``tri_block_dims``."""
    _fields_ = [
        ("B", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("C_z", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("ending", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class MulDims(ctypes.Structure):
    """Mirror of ``tri_mul_dims``."""
    _fields_ = [
        ("B", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("C_z", ctypes.c_int64),
        ("c", ctypes.c_int64),
        ("incoming", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class TriAttnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m triangular_attention_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
    dp = ctypes.POINTER(Dims)
    sig = {
        "tri_attn_fwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "tri_attn_bwd_delta": [dp, vp, vp, vp, vp, vp],
        "tri_attn_bwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "tri_attn_reduce_dq": [dp, vp, vp, vp],
        "tri_attn_reduce_dbias": [dp, vp, vp, vp],
        "tri_attn_bwd_bf16p": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "tri_attn_reduce_dq_bf16p": [dp, vp, vp, vp],
        "tri_attn_reduce_dbias_bf16p": [dp, vp, vp, vp],
        "tri_attn_workspace": [dp, i64p, i64p, i64p, i64p, i64p, i64p],
        "tri_attn_workspace_single_pass": [dp, i64p, i64p, i64p, i64p, i64p, i64p],
        "tri_attn_bwd_chunked_workspace": [dp, ctypes.c_int64, i64p, i64p],
        "tri_attn_bwd_chunked": [dp] + [vp] * 13 + [ctypes.c_int64, vp],
        "tri_attn_bwd_chunked_noalloc": [dp] + [vp] * 13,
    }
    bp = ctypes.POINTER(BlockDims)
    sig.update({
        "tri_block_workspace": [bp, i64p, i64p, i64p],
        "tri_block_ln_proj": [bp] + [vp] * 12,
        "tri_block_gate_out": [bp] + [vp] * 5,
        "tri_block_gate_out_bwd": [bp] + [vp] * 8,
        "tri_block_proj_bwd_dz": [bp] + [vp] * 13,
        "tri_block_proj_bwd_dw": [bp] + [vp] * 11,
        "tri_block_reduce_wgrad": [bp] + [vp] * 9,
    })
    mp = ctypes.POINTER(MulDims)
    sig.update({
        "tri_mul_workspace": [mp, i64p, i64p, i64p, i64p],
        "tri_mul_in_fwd": [mp] + [vp] * 9,
        "tri_mul_contract": [mp] + [vp] * 4,
        "tri_mul_out_fwd": [mp] + [vp] * 8,
        "tri_mul_out_bwd": [mp] + [vp] * 12,
        "tri_mul_contract_bwd": [mp] + [vp] * 6,
        "tri_mul_in_bwd": [mp] + [vp] * 9,
        "tri_mul_in_bwd_dz": [mp] + [vp] * 9,
        "tri_mul_in_bwd_dw": [mp] + [vp] * 8,
        "tri_mul_reduce_wgrad": [mp] + [vp] * 11,
    })
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.tri_attn_status_string.argtypes = [ctypes.c_int]
    lib.tri_attn_status_string.restype = ctypes.c_char_p
    lib.tri_attn_noalloc_scratch_bytes.argtypes = []
    lib.tri_attn_noalloc_scratch_bytes.restype = ctypes.c_int64
    lib.tri_attn_version.argtypes = []
    lib.tri_attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(fn: str, code: int) -> None:
    if code != 0:
        msg = load().tri_attn_status_string(code).decode()
        raise TriAttnError(fn, code, msg)


def dims(B: int, N_o: int, H: int, N: int, D: int, scale: float) -> Dims:
    return Dims(int(B), int(N_o), int(H), int(N), int(D), float(scale))
