"""MI355X (gfx950) triangular attention: HIP kernels behind a C ABI.

The library ``libtri_attn.so`` (built from ``csrc/`` by ``build.py``) exports
``tri_attn_fwd``, ``tri_attn_bwd_delta``, ``tri_attn_bwd``,
``tri_attn_reduce_dq`` and ``tri_attn_reduce_dbias``; this package binds them
with ctypes under the same names and offers ``triangular_attention`` as an
autograd function.
"""
from ._lib import EXPORTS, LIB_PATH, Dims, TriAttnError, load  # noqa: F401
from .api import (  # noqa: F401
    backward,
    dims_of,
    forward,
    tri_attn_bwd,
    tri_attn_bwd_delta,
    tri_attn_fwd,
    tri_attn_reduce_dbias,
    tri_attn_reduce_dq,
    triangular_attention,
    workspace,
)
