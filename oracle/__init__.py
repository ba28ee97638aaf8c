"""FP64 CPU oracle for triangular attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The GPU library never calls it and shares no code
with it.

Source: "TurboPairFormer: Fast and Stable Protein Folding Model Training with
an Optimized Triangle Attention Kernel" -- Figure 1(a), Figure 6, Figure 7(b)
and the notation table (Table 1) for what is computed; Figure 7(d) and
Figure 11(a) for the reductions.  The method is an exact reorganisation of
plain triangular attention (one probability evaluation, partial sums
reordered), so the oracle is the plain definition written out in float64,
not the tiled algorithm.

``oracle.block_fp64`` extends it to the whole triangle-attention block
(normalisation, projections, gate, output projection; starting and ending
node), pinned by ``tests/test_oracle_block.py``; ``oracle.trimul_fp64`` is the triangle
multiplicative update (Figure 12), pinned by ``tests/test_oracle_trimul.py``.

Every function here is pinned by ``tests/test_oracle.py`` against something
other than itself (brute force, finite differences, a library special case,
closed forms, invariants, or the indices of the worked example).
"""
from .tri_attn_fp64 import (  # noqa: F401
    forward,
    backward,
    backward_slices,
    dbias_rows,
    probabilities,
    compensated_delta,
    sum_partials,
    bf16_round,
    rel_rmse,
    abs_rmse,
)
