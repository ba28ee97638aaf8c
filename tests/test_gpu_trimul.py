"""GPU parity of the triangle multiplicative update (C ABI: include/tri_mul.h) against the FP64
oracle (``oracle.trimul_fp64``) on seeded inputs, element by element over every output, from a
single tile up to the full N = 768, 128-channel size; and bitwise repeatability.

Tolerances (relative RMSE against the FP64 oracle): the update 1e-2 and every gradient 1.5e-2,
the bounds of the triangle-attention block: the update passes through bf16 roundings of Zln, the
gated branch operands, the contraction, its normalisation and the output, each about 1.1-1.6e-3
relative RMS.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import np64, require_gpu
from oracle import rel_rmse
from oracle import trimul_fp64 as tm

TOL_OUT, TOL_G = 1e-2, 1.5e-2
GRADS = ("dz", "dw_in", "dw_o", "dgamma", "dbeta", "dgamma_o", "dbeta_o")
PARAMS = ("gamma", "beta", "w_in", "gamma_o", "beta_o", "w_o")

# (B, N, c, incoming, w_std): one tile, ragged tiles of every kernel, B = 2, both channel counts,
# and N = 136 (18496 pairs: more tiles than workgroups in every persistent kernel; 2 x 2
# contraction tiles with an 8-wide ragged edge)
CASES = [
    (1, 8, 64, False, 0.1),
    (1, 16, 128, True, 0.1),
    (2, 24, 64, True, 0.1),
    (1, 40, 128, False, 0.1),
    (1, 136, 128, False, 0.08),
    (1, 136, 64, True, 0.08),
    (2, 128, 64, False, 0.08),   # B = 2 with whole-row tiles: the division-free index path at b = 1
]


def _dev(x):
    out = {}
    for n in ("z", "dout", "w_in", "w_o"):
        out[n] = x[n].to(torch.bfloat16).cuda()
    for n in ("gamma", "beta", "gamma_o", "beta_o"):
        out[n] = x[n].float().cuda()
    return out


def _run(ta, dv, c, inc):
    p = [dv[n] for n in PARAMS]
    out, saved = ta.trimul_forward(dv["z"], *p, c, incoming=inc)
    g = ta.trimul_backward(dv["z"], *p, saved, dv["dout"])
    torch.cuda.synchronize()
    g["out"] = out
    return g


def _oracle(x, c, inc):
    a = [x[n].double().numpy() for n in ("z",) + PARAMS]
    return tm.trimul_backward(*a, x["dout"].double().numpy(), c, incoming=inc)


def _case_id(cs):
    B, N, c, inc, ws = cs
    return f"B{B}_N{N}_c{c}_{'in' if inc else 'out'}"


def _check(got, ref, tag):
    err = {n: rel_rmse(np64(got[n]), ref[n]) for n in ("out",) + GRADS}
    print(tag, {k: f"{v:.2e}" for k, v in err.items()}, flush=True)
    assert err["out"] <= TOL_OUT, err
    for n in GRADS:
        assert err[n] <= TOL_G, (n, err)
    for n in ("out",) + GRADS:
        assert torch.isfinite(got[n].float()).all(), n


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_trimul_matches_oracle(case):
    ta = require_gpu()
    B, N, c, inc, ws = case
    print(f"trimul parity {_case_id(case)}", flush=True)
    w = synth.TrimulWorkload("t", B, N, c, incoming=inc, w_std=ws, ln_std=0.1)
    x = synth.make_trimul_inputs(w, seed=N + c)
    _check(_run(ta, _dev(x), c, inc), _oracle(x, c, inc), _case_id(case))


@pytest.mark.gpu
@pytest.mark.parametrize("case", [CASES[3], CASES[5]], ids=_case_id)
def test_trimul_bitwise_repeatable(case):
    """Three calls on the same input: every output bitwise identical (fixed-order partial sums)."""
    ta = require_gpu()
    B, N, c, inc, ws = case
    print(f"trimul replay {_case_id(case)}", flush=True)
    w = synth.TrimulWorkload("t", B, N, c, incoming=inc, w_std=ws, ln_std=0.1)
    dv = _dev(synth.make_trimul_inputs(w, seed=3))
    first = _run(ta, dv, c, inc)
    for _ in range(2):
        again = _run(ta, dv, c, inc)
        for n in ("out",) + GRADS:
            assert torch.equal(first[n], again[n]), n


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["trimul_n768_c128_out", "trimul_n768_c128_in"])
def test_trimul_full_size(name):
    """The pages' largest update (N = 768, 128 channels, weights N(0, 0.02)): every element of the
    update and of all gradients against the FP64 oracle."""
    ta = require_gpu()
    w = synth.TRIMUL_WORKLOADS[name]
    print(f"trimul full-size parity {name}", flush=True)
    x = synth.make_trimul_inputs(w, seed=0)
    got = _run(ta, _dev(x), w.c, w.incoming)
    got = {n: got[n] for n in ("out",) + GRADS}
    torch.cuda.empty_cache()
    _check(got, _oracle(x, w.c, w.incoming), name)
