"""The allocation-free backward (tri_attn_bwd_chunked_noalloc): its chunk buffers live in the
library's static scratch array.  Checked through the C ABI against the entry point it is a
variant of, which takes a caller workspace (tri_attn_bwd_chunked): bitwise equal, on two calls
in a row (the second with a smaller input, so the scratch holds the first call's contents when
the second starts).  Both run the single-pass key-tile kernel; the default five calls
(tri_attn_bwd + the two reductions, two kernels at D = 32) give the same gradients up to
rounding order, which is checked too, and the small case is checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import inputs, np64, require_gpu, to_dev, workload

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16)


def _prepare(ta, dev, scale):
    o, o_res, lse = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], scale)
    d = ta.dims_of(dev["q"], scale)
    delta = torch.empty_like(lse)
    ta.tri_attn_bwd_delta(d, o, o_res, dev["do"], delta)
    return d, lse, delta


def _noalloc(ta, d, dev, lse, delta):
    out = [torch.full_like(dev[n], float("nan")) for n in ("q", "k", "v", "bias")]
    ta.tri_attn_bwd_chunked_noalloc(d, dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], dev["do"], lse, delta,
                                    *out)
    return out


def _with_workspace(ta, d, dev, lse, delta):
    out = [torch.full_like(dev[n], float("nan")) for n in ("q", "k", "v", "bias")]
    nbytes = ta._lib.load().tri_attn_noalloc_scratch_bytes()
    buf = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    ta.tri_attn_bwd_chunked(d, dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], dev["do"], lse, delta,
                            *out, buf)
    return out


def _unchunked(ta, d, dev, lse, delta):
    ws = ta.workspace(d)
    dqp = torch.empty(ws["dq_partial_elems"], device="cuda")
    dbp = torch.empty(ws["dbias_partial_elems"], device="cuda")
    dq, dk, dv, dbias = (torch.empty_like(dev[n]) for n in ("q", "k", "v", "bias"))
    ta.tri_attn_bwd(d, dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], dev["do"], lse, delta, dk, dv,
                    dqp, dbp)
    ta.tri_attn_reduce_dbias(d, dbp, dbias)
    ta.tri_attn_reduce_dq(d, dqp, dq)
    return [dq, dk, dv, dbias]


def test_noalloc_matches_workspace_entry_points_twice():
    ta = require_gpu()
    # first call: the headline workload (many chunks of the 128 MiB array); second: a smaller,
    # ragged case (B = 2, odd N, masked) run straight after it on the same array
    big = synth.get("n768_d32_mask")
    small, _ = workload(9, 67, 3, 32, 0.2, 2.0, B=2)
    runs = [(big, synth.make_inputs(big, 3)), (small, inputs(small, seed=11, mask_p=0.2))]
    for w, x in runs:
        print(f"no-alloc backward: B={w.B} N_o={w.N_o} N={w.N} H={w.H} D={w.D}", flush=True)
        dev = to_dev(x)
        d, lse, delta = _prepare(ta, dev, w.scale)
        got = _noalloc(ta, d, dev, lse, delta)
        ref_ws = _with_workspace(ta, d, dev, lse, delta)
        ref = _unchunked(ta, d, dev, lse, delta)
        torch.cuda.synchronize()
        for n, a, b, c in zip(("dq", "dk", "dv", "dbias"), got, ref_ws, ref):
            assert torch.isfinite(a.float()).all(), n
            assert torch.equal(_bits(a), _bits(b)), n
            # the default calls: same gradients, other summation order (dK, dV: same kernel code)
            rel = float(((a.float() - c.float()).norm() / c.float().norm().clamp_min(1e-30)))
            assert rel <= 4e-3, (n, rel)
        if w.N <= 100:
            # the small case whole against the oracle
            r = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
            for n, a in zip(("dq", "dk", "dv", "dbias"), got):
                assert oracle.rel_rmse(np64(a), r[n]) <= 1.5e-2, n


def test_noalloc_rejects_shapes_past_the_scratch_size():
    ta = require_gpu()
    w, _ = workload(8, 4096, 4, 32)
    q = torch.zeros((1, 8, 4, 4096, 32), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((1, 4, 4096, 4096), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 8, 4, 4096), device="cuda")
    d = ta.dims_of(q, w.scale)
    with pytest.raises(ta.TriAttnError) as e:
        ta.tri_attn_bwd_chunked_noalloc(d, q, q, q, bias, None, q, lse, lse, q.clone(), q.clone(), q.clone(),
                                        bias.clone())
    assert e.value.code == 6
