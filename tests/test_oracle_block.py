"""Pins of the FP64 block oracle (``oracle.block_fp64``) against things other than itself (CPU).

The block follows "TurboPairFormer: Fast and Stable Protein Folding Model
Training with an Optimized Triangle Attention Kernel", Table 1 and Figure 6
(which pair feeds which query, key, value and bias; the normalisation before
the projections).  Checks:

* LayerNorm against torch's ``layer_norm`` in float64 (a library routine);
* every gradient against central finite differences of ``L = sum(y * dy)``;
* every gradient against torch float64 autograd of the block written with
  torch's own ``layer_norm``, ``softmax`` and ``sigmoid`` (an independent
  derivation of the backward);
* the dependency pattern of the worked example (Figure 6): output pair (o, q)
  depends on pair rows o and q of Z only (columns for the ending node);
* closed forms: zero query/key/bias maps give uniform attention, a zero gate map
  gives gate 1/2;
* a symmetric Z gives the same update from both nodes up to the axis swap.
"""
import math

import numpy as np
import pytest
import torch

from oracle import block_fp64 as blk


def _params(Cz, H, D, seed, wstd=0.3):
    rng = np.random.default_rng(seed)
    HD = H * D
    return {
        "gamma": 1.0 + 0.2 * rng.standard_normal(Cz),
        "beta": 0.2 * rng.standard_normal(Cz),
        "w_qkvg": wstd * rng.standard_normal((4 * HD, Cz)),
        "w_b": wstd * rng.standard_normal((H, Cz)),
        "w_o": wstd * rng.standard_normal((Cz, HD)),
    }


def _case(B=1, N=5, Cz=6, H=2, D=3, seed=0):
    rng = np.random.default_rng(seed + 100)
    z = rng.standard_normal((B, N, N, Cz))
    dy = rng.standard_normal((B, N, N, Cz))
    return z, dy, _params(Cz, H, D, seed)


def _fwd(z, p, H, D, ending):
    return blk.block_forward(z, p["gamma"], p["beta"], p["w_qkvg"], p["w_b"], p["w_o"], H, D,
                             ending=ending)["y"]


def _bwd(z, p, dy, H, D, ending):
    return blk.block_backward(z, p["gamma"], p["beta"], p["w_qkvg"], p["w_b"], p["w_o"], dy, H, D,
                              ending=ending)


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(3)
    z = 3.0 * rng.standard_normal((4, 7, 16)) + 1.5
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    zln, xhat, rstd = blk.layer_norm(z, g, b, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (16,), torch.from_numpy(g),
                                         torch.from_numpy(b), 1e-5).numpy()
    assert np.max(np.abs(zln - ref)) < 1e-12
    # invariants of the normalised part: zero mean, unit variance up to eps
    assert np.max(np.abs(xhat.mean(-1))) < 1e-12
    var = z.var(-1)
    assert np.allclose((xhat ** 2).mean(-1), var / (var + 1e-5), rtol=0, atol=1e-12)


@pytest.mark.parametrize("ending", [False, True])
def test_gradients_match_finite_differences(ending):
    H, D = 2, 3
    z, dy, p = _case(H=H, D=D, seed=1)
    g = _bwd(z, p, dy, H, D, ending)
    rng = np.random.default_rng(11)
    loss = lambda zz, pp: float(np.sum(_fwd(zz, pp, H, D, ending) * dy))
    eps = 1e-6
    # directional derivatives along random directions, one per input
    for name, grad in [("z", g["dz"]), ("gamma", g["dgamma"]), ("beta", g["dbeta"]),
                       ("w_qkvg", g["dw_qkvg"]), ("w_b", g["dw_b"]), ("w_o", g["dw_o"])]:
        base = z if name == "z" else p[name]
        u = rng.standard_normal(base.shape)

        def at(t):
            if name == "z":
                return loss(z + t * u, p)
            q = dict(p)
            q[name] = p[name] + t * u
            return loss(z, q)

        fd = (at(eps) - at(-eps)) / (2 * eps)
        an = float(np.sum(grad * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    # and a few single entries of dz
    for idx in [(0, 0, 0, 0), (0, 2, 4, 5), (0, 4, 1, 3)]:
        e = np.zeros_like(z)
        e[idx] = 1.0
        fd = (loss(z + eps * e, p) - loss(z - eps * e, p)) / (2 * eps)
        assert abs(fd - g["dz"][idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, g["dz"][idx])


def _torch_block(z, p, H, D, ending):
    """The block with torch's own layer_norm / softmax / sigmoid, for autograd."""
    if ending:
        z = z.transpose(1, 2)
    B, N, _, Cz = z.shape
    HD = H * D
    zln = torch.nn.functional.layer_norm(z, (Cz,), p["gamma"], p["beta"], 1e-5)
    proj = zln @ p["w_qkvg"].T

    def heads(t):                           # [B,N,N,HD] -> [B,N_o,H,N,D]
        return t.reshape(B, N, N, H, D).permute(0, 1, 3, 2, 4)

    q, k, v, g = (heads(proj[..., i * HD:(i + 1) * HD]) for i in range(4))
    bias = (zln @ p["w_b"].T).permute(0, 3, 1, 2)                    # [B,H,N,N]
    s = (q @ k.transpose(-1, -2)) / math.sqrt(D) + bias[:, None]
    o = torch.softmax(s, dim=-1) @ v
    go = (torch.sigmoid(g) * o).permute(0, 1, 3, 2, 4).reshape(B, N, N, HD)
    y = go @ p["w_o"].T
    return y.transpose(1, 2) if ending else y


@pytest.mark.parametrize("ending", [False, True])
def test_matches_torch_autograd(ending):
    H, D = 2, 4
    z, dy, p = _case(B=2, N=6, Cz=8, H=H, D=D, seed=2)
    tz = torch.from_numpy(z).requires_grad_(True)
    tp = {n: torch.from_numpy(v).requires_grad_(True) for n, v in p.items()}
    y = _torch_block(tz, tp, H, D, ending)
    y.backward(torch.from_numpy(dy))
    g = _bwd(z, p, dy, H, D, ending)
    assert np.max(np.abs(g["y"] - y.detach().numpy())) < 1e-12
    pairs = [("dz", tz), ("dgamma", tp["gamma"]), ("dbeta", tp["beta"]),
             ("dw_qkvg", tp["w_qkvg"]), ("dw_b", tp["w_b"]), ("dw_o", tp["w_o"])]
    for name, t in pairs:
        ref = t.grad.numpy()
        err = np.max(np.abs(g[name] - ref)) / max(1e-300, np.max(np.abs(ref)))
        assert err < 1e-11, (name, err)


@pytest.mark.parametrize("ending", [False, True])
def test_dependency_pattern_of_worked_example(ending):
    """Figure 6: the update of pair (o, q) reads pair row o (query, keys, values, gate) and
    pair row q (the bias of query q); nothing else.  For the ending node, columns."""
    N, H, D = 7, 1, 2
    z, _, p = _case(N=N, Cz=4, H=H, D=D, seed=4)
    y0 = _fwd(z, p, H, D, ending)
    a, b = 2, 4
    z1 = z.copy()
    z1[0, a, b, 1] += 0.5                # one feature (a shift of all features is normalised away)
    y1 = _fwd(z1, p, H, D, ending)
    changed = np.any(y1[0] != y0[0], axis=-1)                       # [N, N]
    i, j = np.meshgrid(np.arange(N), np.arange(N), indexing="ij")
    if not ending:
        expect = (i == a) | (j == a)
    else:
        expect = (i == b) | (j == b)
    assert np.array_equal(changed, expect)


def test_closed_form_uniform_attention_half_gate():
    """Zero Q, K and bias maps: every key gets weight 1/N; zero gate map: sigmoid(0) = 1/2.
    Then y[o, q] = 1/2 * mean_k(V[o, k]) @ w_o.T, with V from torch's layer_norm."""
    H, D, Cz, N = 2, 3, 5, 6
    z, _, p = _case(N=N, Cz=Cz, H=H, D=D, seed=5)
    HD = H * D
    p["w_qkvg"][0:2 * HD] = 0.0          # Q and K maps
    p["w_qkvg"][3 * HD:] = 0.0           # gate map
    p["w_b"][:] = 0.0
    y = _fwd(z, p, H, D, False)
    zln = torch.nn.functional.layer_norm(torch.from_numpy(z), (Cz,), torch.from_numpy(p["gamma"]),
                                         torch.from_numpy(p["beta"]), 1e-5).numpy()
    v = zln @ p["w_qkvg"][2 * HD:3 * HD].T                          # [1,N,N,HD]
    vbar = v.mean(axis=2)                                           # mean over keys k
    ref = 0.5 * np.einsum("bof,cf->boc", vbar, p["w_o"])[:, :, None, :].repeat(N, axis=2)
    assert np.max(np.abs(y - ref)) < 1e-12


def test_symmetric_pairs_both_nodes():
    H, D = 2, 2
    z, _, p = _case(N=6, Cz=4, H=H, D=D, seed=6)
    zs = 0.5 * (z + np.swapaxes(z, 1, 2))
    ys = _fwd(zs, p, H, D, False)
    ye = _fwd(zs, p, H, D, True)
    assert np.max(np.abs(ye - np.swapaxes(ys, 1, 2))) < 1e-13


@pytest.mark.parametrize("ending", [False, True])
def test_sampled_rows_match_full_backward(ending):
    """The row-sampling form used at full size agrees with the full backward."""
    H, D = 2, 3
    z, dy, p = _case(B=2, N=7, Cz=5, H=H, D=D, seed=8)
    full = _bwd(z, p, dy, H, D, ending)
    rows = [(0, 0), (1, 3), (1, 6)]
    r = blk.block_rows(z, p["gamma"], p["beta"], p["w_qkvg"], p["w_b"], p["w_o"], dy, H, D, rows,
                       ending=ending)
    for i, (b, a) in enumerate(rows):
        yref = full["y"][b, :, a] if ending else full["y"][b, a]
        dzref = full["dz"][b, :, a] if ending else full["dz"][b, a]
        assert np.max(np.abs(r["y"][i] - yref)) < 1e-12
        assert np.max(np.abs(r["dz"][i] - dzref)) < 1e-12
