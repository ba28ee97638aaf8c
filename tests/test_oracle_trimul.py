"""Pins of the FP64 triangle-multiplication oracle (``oracle.trimul_fp64``) against things other
than itself (CPU).

The update follows "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
Optimized Triangle Attention Kernel", Figure 12 (input normalisation and five projections with
gated branch values, a per-channel contraction, output normalisation, projection and sigmoid
gate).  Checks:

* the per-channel contraction against brute-force loops, both directions;
* every gradient against central finite differences of ``L = sum(out * dout)``;
* every gradient against torch float64 autograd of the update written with torch's own
  ``layer_norm``, ``sigmoid`` and ``einsum``;
* the incoming contraction of Z equals the outgoing contraction of Z with its token axes swapped;
* a closed form: with a zero branch-value map the contraction vanishes, the output normalisation
  returns its shift, and ``out = sigmoid(g) * (beta_o @ w_o.T)``.
"""
import numpy as np
import pytest
import torch

from oracle import trimul_fp64 as tm


def _case(B=1, N=5, Cz=6, c=3, seed=0, wstd=0.4):
    rng = np.random.default_rng(seed)
    p = {
        "gamma": 1.0 + 0.2 * rng.standard_normal(Cz), "beta": 0.2 * rng.standard_normal(Cz),
        "w_in": wstd * rng.standard_normal((4 * c + Cz, Cz)),
        "gamma_o": 1.0 + 0.2 * rng.standard_normal(c), "beta_o": 0.2 * rng.standard_normal(c),
        "w_o": wstd * rng.standard_normal((Cz, c)),
    }
    z = rng.standard_normal((B, N, N, Cz))
    dout = rng.standard_normal((B, N, N, Cz))
    return z, dout, p


NAMES = ("gamma", "beta", "w_in", "gamma_o", "beta_o", "w_o")


def _fwd(z, p, c, inc):
    return tm.trimul_forward(z, *[p[n] for n in NAMES], c, incoming=inc)["out"]


def _bwd(z, p, dout, c, inc):
    return tm.trimul_backward(z, *[p[n] for n in NAMES], dout, c, incoming=inc)


@pytest.mark.parametrize("inc", [False, True])
def test_contraction_matches_loops(inc):
    rng = np.random.default_rng(1)
    B, N, c = 2, 4, 3
    a, b = rng.standard_normal((B, N, N, c)), rng.standard_normal((B, N, N, c))
    ref = np.zeros((B, N, N, c))
    for bb in range(B):
        for i in range(N):
            for j in range(N):
                for ch in range(c):
                    for k in range(N):
                        if inc:
                            ref[bb, i, j, ch] += a[bb, k, i, ch] * b[bb, k, j, ch]
                        else:
                            ref[bb, i, j, ch] += a[bb, i, k, ch] * b[bb, j, k, ch]
    assert np.max(np.abs(tm.contract(a, b, inc) - ref)) < 1e-12


@pytest.mark.parametrize("inc", [False, True])
def test_gradients_match_finite_differences(inc):
    c = 3
    z, dout, p = _case(c=c, seed=2)
    g = _bwd(z, p, dout, c, inc)
    rng = np.random.default_rng(12)
    loss = lambda zz, pp: float(np.sum(_fwd(zz, pp, c, inc) * dout))
    eps = 1e-6
    grads = {"z": g["dz"], "gamma": g["dgamma"], "beta": g["dbeta"], "w_in": g["dw_in"],
             "gamma_o": g["dgamma_o"], "beta_o": g["dbeta_o"], "w_o": g["dw_o"]}
    for name, grad in grads.items():
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


def _torch_trimul(z, p, c, inc):
    Cz = z.shape[-1]
    zln = torch.nn.functional.layer_norm(z, (Cz,), p["gamma"], p["beta"], 1e-5)
    w = p["w_in"]
    a = torch.sigmoid(zln @ w[c:2 * c].T) * (zln @ w[:c].T)
    b = torch.sigmoid(zln @ w[3 * c:4 * c].T) * (zln @ w[2 * c:3 * c].T)
    g = zln @ w[4 * c:].T
    x = torch.einsum("bkic,bkjc->bijc", a, b) if inc else torch.einsum("bikc,bjkc->bijc", a, b)
    xln = torch.nn.functional.layer_norm(x, (c,), p["gamma_o"], p["beta_o"], 1e-5)
    return torch.sigmoid(g) * (xln @ p["w_o"].T)


@pytest.mark.parametrize("inc", [False, True])
def test_matches_torch_autograd(inc):
    c = 4
    z, dout, p = _case(B=2, N=6, Cz=8, c=c, seed=3)
    tz = torch.from_numpy(z).requires_grad_(True)
    tp = {n: torch.from_numpy(v).requires_grad_(True) for n, v in p.items()}
    out = _torch_trimul(tz, tp, c, inc)
    out.backward(torch.from_numpy(dout))
    g = _bwd(z, p, dout, c, inc)
    assert np.max(np.abs(g["out"] - out.detach().numpy())) < 1e-12
    pairs = [("dz", tz), ("dgamma", tp["gamma"]), ("dbeta", tp["beta"]), ("dw_in", tp["w_in"]),
             ("dgamma_o", tp["gamma_o"]), ("dbeta_o", tp["beta_o"]), ("dw_o", tp["w_o"])]
    for name, t in pairs:
        ref = t.grad.numpy()
        err = np.max(np.abs(g[name] - ref)) / max(1e-300, np.max(np.abs(ref)))
        assert err < 1e-11, (name, err)


def test_incoming_is_outgoing_of_swapped_pairs():
    c = 3
    z, _, p = _case(N=6, c=c, seed=4)
    f_in = tm.trimul_forward(z, *[p[n] for n in NAMES], c, incoming=True)
    f_out = tm.trimul_forward(np.swapaxes(z, 1, 2), *[p[n] for n in NAMES], c, incoming=False)
    assert np.max(np.abs(f_in["x"] - f_out["x"])) < 1e-12


def test_closed_form_zero_branch_values():
    c, Cz = 3, 6
    z, _, p = _case(N=5, Cz=Cz, c=c, seed=5)
    p["w_in"][:c] = 0.0                      # branch value map of a: a = 0, so x = 0
    out = _fwd(z, p, c, False)
    zln = torch.nn.functional.layer_norm(torch.from_numpy(z), (Cz,), torch.from_numpy(p["gamma"]),
                                         torch.from_numpy(p["beta"]), 1e-5).numpy()
    g = zln @ p["w_in"][4 * c:].T
    ref = 1.0 / (1.0 + np.exp(-g)) * (p["beta_o"] @ p["w_o"].T)
    assert np.max(np.abs(out - ref)) < 1e-12
