"""GPU parity of the triangle-attention block (C ABI: include/tri_attn_block.h) against the FP64
block oracle (``oracle.block_fp64``), on seeded inputs: small and ragged sizes compared element by
element over every output, the full-size workload (N = 768) on sampled pair rows, and bitwise
repeatability.

Tolerances (relative RMSE against the FP64 oracle): the projections Q, K, V, gate and bias 5e-3
(the bound of the attention output: Zln and the projection are each rounded to bf16 once); the
update Y 1e-2, twice the attention output's bound, because the attention's own inputs now carry
those roundings and Y adds two more (the gated output and Y itself), each up to about 1.6e-3
relative RMS; every gradient 1.5e-2, the bound of the attention gradients.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import np64, require_gpu
from oracle import block_fp64 as blk
from oracle import rel_rmse

TOL_P, TOL_Y, TOL_G = 5e-3, 1e-2, 1.5e-2
GRADS = ("dz", "dw_qkvg", "dw_b", "dw_o", "dgamma", "dbeta")

# (B, N, H, ending, w_std): ragged pair counts against the 128- and 64-pair tiles, a case below one
# tile, and N = 182 (33124 pairs: more tiles than workgroups, so workgroups loop)
CASES = [
    (1, 12, 4, False, 0.1),
    (1, 9, 8, False, 0.1),
    (2, 23, 8, True, 0.1),
    (1, 40, 4, True, 0.1),
    (1, 182, 4, False, 0.08),
    (1, 182, 8, True, 0.08),
    (2, 128, 4, True, 0.08),     # B = 2 with whole-row tiles: the division-free index path at b = 1
]


def _dev(x):
    out = {}
    for n in ("z", "dy", "w_qkvg", "w_b", "w_o"):
        out[n] = x[n].to(torch.bfloat16).cuda()
    out["gamma"] = x["gamma"].float().cuda()
    out["beta"] = x["beta"].float().cuda()
    return out


def _run(ta, dv, H, D, ending):
    y, saved = ta.block_forward(dv["z"], dv["gamma"], dv["beta"], dv["w_qkvg"], dv["w_b"], dv["w_o"], H, D,
                                ending=ending)
    g = ta.block_backward(dv["z"], dv["gamma"], dv["beta"], dv["w_qkvg"], dv["w_b"], dv["w_o"], saved, dv["dy"])
    torch.cuda.synchronize()
    g["y"] = y
    for n in ("q", "k", "v", "g", "bias"):
        g[n] = saved[n]
    return g


def _oracle(x, H, D, ending):
    a = [x[n].double().numpy() for n in ("z", "gamma", "beta", "w_qkvg", "w_b", "w_o")]
    ref = blk.block_backward(*a, x["dy"].double().numpy(), H, D, ending=ending)
    fwd = blk.block_forward(*a, H, D, ending=ending)
    for n in ("q", "k", "v", "g", "bias"):
        ref[n] = fwd[n]
    return ref


def _case_id(c):
    B, N, H, ending, ws = c
    return f"B{B}_N{N}_H{H}_{'end' if ending else 'start'}"


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_block_matches_oracle(case):
    ta = require_gpu()
    B, N, H, ending, ws = case
    D = 128 // H
    print(f"block parity {_case_id(case)}", flush=True)
    w = synth.BlockWorkload("t", B, N, H, D, ending=ending, w_std=ws, ln_std=0.1)
    x = synth.make_block_inputs(w, seed=N + H)
    got = _run(ta, _dev(x), H, D, ending)
    ref = _oracle(x, H, D, ending)
    err = {n: rel_rmse(np64(got[n]), ref[n]) for n in ("y", "q", "k", "v", "g", "bias") + GRADS}
    print(_case_id(case), {k: f"{v:.2e}" for k, v in err.items()}, flush=True)
    assert err["y"] <= TOL_Y, err
    for n in ("q", "k", "v", "g", "bias"):
        assert err[n] <= TOL_P, (n, err)
    for n in GRADS:
        assert err[n] <= TOL_G, (n, err)
    for n in ("y",) + GRADS:
        assert torch.isfinite(got[n].float()).all(), n


@pytest.mark.gpu
@pytest.mark.parametrize("case", [CASES[3], CASES[4]], ids=_case_id)
def test_block_bitwise_repeatable(case):
    """Three calls on the same input: every output bitwise identical (fixed-order partial sums)."""
    ta = require_gpu()
    B, N, H, ending, ws = case
    D = 128 // H
    print(f"block replay {_case_id(case)}", flush=True)
    w = synth.BlockWorkload("t", B, N, H, D, ending=ending, w_std=ws, ln_std=0.1)
    dv = _dev(synth.make_block_inputs(w, seed=5))
    first = _run(ta, dv, H, D, ending)
    for _ in range(2):
        again = _run(ta, dv, H, D, ending)
        for n in ("y",) + GRADS:
            assert torch.equal(first[n], again[n]), n


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(synth.BLOCK_WORKLOADS))
def test_block_full_size_sampled(name):
    """The full-size block (N = 768, weights N(0, 0.02)): Y and dZ of sampled pair rows against the
    oracle's row form; every output finite."""
    ta = require_gpu()
    w = synth.BLOCK_WORKLOADS[name]
    print(f"block full-size parity {name}", flush=True)
    x = synth.make_block_inputs(w, seed=0)
    got = _run(ta, _dev(x), w.H, w.D, w.ending)
    rows = [(0, 0), (0, 385), (0, w.N - 1)]
    a = [x[n].double().numpy() for n in ("z", "gamma", "beta", "w_qkvg", "w_b", "w_o")]
    ref = blk.block_rows(*a, x["dy"].double().numpy(), w.H, w.D, rows, ending=w.ending)
    y, dz = np64(got["y"]), np64(got["dz"])
    pick = (lambda t, b, r: t[b, :, r]) if w.ending else (lambda t, b, r: t[b, r])
    gy = np.stack([pick(y, b, r) for (b, r) in rows])
    gz = np.stack([pick(dz, b, r) for (b, r) in rows])
    ey, ez = rel_rmse(gy, ref["y"]), rel_rmse(gz, ref["dz"])
    print(name, f"y {ey:.2e} dz {ez:.2e}", flush=True)
    assert ey <= TOL_Y and ez <= TOL_G, (ey, ez)
    for n in ("y",) + GRADS:
        assert torch.isfinite(got[n].float()).all(), n
