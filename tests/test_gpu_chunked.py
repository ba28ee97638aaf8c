"""The chunked backward (tri_attn_bwd_chunked; TurboPairFormer, Figure 7(d) and Table 2:
partial buffers reused once consumed, so only one chunk of outer groups has partials at a
time) runs the single-pass key-tile kernel.  For every chunk size it is bitwise equal to the
same kernel run as one chunk (all outer groups) and, where the default backward is that kernel
(D = 64; D = 16 up to N = 640), to the three unchunked calls; including ragged last chunks, ragged
last outer groups, B > 1, odd N (scalar reduction path), D = 16 (outer group 6) and D = 64
(outer group 2); and at full size, where it is also checked against the oracle on sampled
outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import inputs, np64, require_gpu, row_ratio, to_dev, workload

pytestmark = pytest.mark.gpu

TOL_G = 1.5e-2


def _bits(t):
    return t.view(torch.int16)


def _both(ta, dev, scale, chunk_groups):
    """The chunked backward at each chunk size, and its reference: the same kernel as one chunk
    where the default backward runs two kernels (D = 32; D = 16 past N = 640), else the three
    unchunked calls (the same kernel)."""
    o, o_res, lse = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], scale)
    args = (dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], scale, o, o_res, lse, dev["do"])
    D, N = dev["q"].shape[-1], dev["q"].shape[-2]
    if D == 32 or (D == 16 and N > 640):
        ref = ta.backward_chunked(*args)          # one chunk of all outer groups
    else:
        ref = ta.backward(*args)
    out = {}
    for C in chunk_groups:
        d = ta.dims_of(dev["q"], scale)
        nbytes = ta.chunked_workspace(d, C)["bytes"]
        buf = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")     # NaN-poisoned partials
        out[C] = ta.backward_chunked(*args, buffer=buf)
    torch.cuda.synchronize()
    return ref, out


# (N_o, N, H, D, mask_p, bias_std, B)
CASES = [
    (9, 72, 3, 32, 0.1, 1.0, 1),      # L = 3 groups of 4 (last ragged)
    (5, 100, 2, 32, 0.3, 2.0, 2),     # B = 2, 4-byte bias loads
    (13, 200, 2, 16, 0.1, 1.0, 1),    # D = 16: groups of 6, ragged
    (9, 67, 2, 32, 0.2, 1.0, 1),      # odd N: scalar reduction path
    (7, 72, 2, 64, 0.1, 1.0, 2),      # D = 64: groups of 2, B = 2
    (3, 63, 1, 16, 0.1, 1.0, 3),      # odd N, D = 16, B = 3
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "No{}_N{}_H{}_D{}_m{}_b{}_B{}".format(*c))
def test_chunked_bitwise_equals_unchunked(case):
    ta = require_gpu()
    N_o, N, H, D, mask_p, bstd, B = case
    w, _ = workload(N_o, N, H, D, mask_p, bstd, B=B)
    x = inputs(w, seed=N + 3 * D, mask_p=mask_p)
    dev = to_dev(x)
    L = ta.workspace(ta.dims_of(dev["q"], w.scale), single_pass=True)["l"]
    sizes = sorted({1, 2, max(1, L - 1), L})
    print(f"chunked {case}: L = {L}, chunk sizes {sizes}", flush=True)
    ref, out = _both(ta, dev, w.scale, sizes)
    for C, got in out.items():
        for n, a, b in zip(("dq", "dk", "dv", "dbias"), got, ref):
            assert torch.equal(_bits(a), _bits(b)), (C, n)
    # and the result is the oracle's (the unchunked path's own parity, restated here)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    for n, a in zip(("dq", "dk", "dv", "dbias"), out[1]):
        assert oracle.rel_rmse(np64(a), g[n]) <= TOL_G, n


def test_chunked_workspace_too_small_is_an_error():
    ta = require_gpu()
    w, _ = workload(9, 72, 2, 32)
    x = inputs(w, seed=1)
    dev = to_dev(x)
    d = ta.dims_of(dev["q"], w.scale)
    need = ta.chunked_workspace(d, 1)["bytes"]
    buf = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    o, o_res, lse = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], w.scale)
    with pytest.raises(ta.TriAttnError) as e:
        ta.backward_chunked(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], w.scale, o, o_res, lse,
                            dev["do"], buffer=buf)
    assert e.value.code == 6


@pytest.mark.parametrize("name,chunks", [("n768_d32_mask", (10, 48)), ("n640_d16", (13,)),
                                         ("n768_d64_mask", (40,))])
def test_chunked_full_size(name, chunks):
    """Full size: the chunked backward with chunks whose partials fit the 256 MB last-level
    cache (C = 10 at N = 768, D = 32: 189 MB) and with four chunks, bitwise equal to the
    unchunked calls and within the tolerance of the oracle on sampled outputs."""
    ta = require_gpu()
    w = synth.get(name)
    print(f"chunked full size {name} {chunks}", flush=True)
    x = synth.make_inputs(w, 0)
    dev = to_dev(x)
    ref, out = _both(ta, dev, w.scale, chunks)
    for C, got in out.items():
        for n, a, b in zip(("dq", "dk", "dv", "dbias"), got, ref):
            assert torch.equal(_bits(a), _bits(b)), (C, n)
    from test_gpu_full import as64, oracle_at, sample_points
    slices, rows = sample_points(w, n_slices=6, n_rows=24)
    r = oracle_at(w, as64(x), slices, rows)
    got = dict(zip(("dq", "dk", "dv", "dbias"), out[chunks[0]]))
    for n in ("dq", "dk", "dv"):
        g = np.stack([np64(got[n][b, o]) for (b, o) in slices])
        assert oracle.rel_rmse(g, r[n]) <= TOL_G, n
        assert row_ratio(g, r[n], TOL_G) <= 3.0, n
    g = np.stack([np64(got["dbias"][b, h, i]) for (b, h, i) in rows])
    assert oracle.rel_rmse(g, r["dbias"]) <= TOL_G
