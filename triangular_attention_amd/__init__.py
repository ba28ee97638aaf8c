"""MI355X (gfx950) triangular attention: HIP kernels behind a C ABI.

The library ``libtri_attn.so`` (built from ``csrc/`` by ``build.py``) exports
``tri_attn_fwd``, ``tri_attn_bwd_delta``, ``tri_attn_bwd``,
``tri_attn_reduce_dq`` and ``tri_attn_reduce_dbias``; this package binds them
with ctypes under the same names and offers ``triangular_attention`` as an
autograd function.  ``block`` binds the triangle-attention block around it
(``tri_block_*``, include/tri_attn_block.h) and offers ``triangle_attention_block``;
``trimul`` binds the triangle multiplicative update (``tri_mul_*``, include/tri_mul.h) and
offers ``triangle_multiplication``.
"""
from ._lib import BLOCK_EXPORTS, EXPORTS, LIB_PATH, TRIMUL_EXPORTS, BlockDims, Dims, MulDims, TriAttnError, load  # noqa: F401
from .api import (  # noqa: F401
    backward,
    backward_chunked,
    chunked_workspace,
    dims_of,
    forward,
    tri_attn_bwd,
    tri_attn_bwd_chunked,
    tri_attn_bwd_chunked_noalloc,
    tri_attn_bwd_delta,
    tri_attn_fwd,
    tri_attn_reduce_dbias,
    tri_attn_reduce_dq,
    triangular_attention,
    workspace,
)
from .block import (  # noqa: F401
    block_backward,
    block_dims,
    block_forward,
    block_workspace,
    triangle_attention_block,
)
from .trimul import (  # noqa: F401
    mul_dims,
    mul_workspace,
    triangle_multiplication,
    trimul_backward,
    trimul_forward,
)
