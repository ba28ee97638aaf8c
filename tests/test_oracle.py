"""Pins of the FP64 oracle against things other than itself (CPU only).

Each check names the passage of "TurboPairFormer: Fast and Stable Protein
Folding Model Training with an Optimized Triangle Attention Kernel" (or the
mathematical fact) it rests on:

* brute force in pure-Python loops, no max shift (definition, Figure 6);
* torch float64 autograd of the plain definition (an independent gradient);
* central finite differences of L = sum(O * dO) for Q, K, V and the bias;
* torch scaled_dot_product_attention with zero bias and no mask;
* closed forms (Q = 0, K = 0, V = 1, a single key) and invariants
  (rows of P sum to one, masked keys get zero probability and zero dK/dV,
  rows of dS sum to zero, dbias is the sum over slices of dS, permuting the
  outer slices, shifting a bias row);
* the indices of the worked example (Figure 6): the bias of pair (4, 6) is
  shared by every slice and only touches query 4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _inputs(N_o, N, H, D, seed, mask_p=0.0, bias_std=1.0, scale=None):
    w = synth.Workload("t", 1, N_o, N, H, D, scale if scale is not None else 1.0 / math.sqrt(D),
                       bias_std=bias_std, mask_p=0.0, bf16=True)
    x = synth.make_inputs(w, seed)
    if mask_p > 0:
        x["mask"] = synth.random_mask(1, N_o, N, mask_p, seed + 7)
    return w, {n: (None if t is None else t.double().numpy()) for n, t in x.items()}


# ----------------------------------------------------------------------------- forward


def _bruteforce_forward(q, k, v, bias, mask, scale):
    B, N_o, H, N, D = q.shape
    O = np.zeros_like(q)
    LSE = np.zeros((B, N_o, H, N))
    for b in range(B):
        for o in range(N_o):
            for h in range(H):
                for i in range(N):
                    s = []
                    for j in range(N):
                        dot = sum(q[b, o, h, i, d] * k[b, o, h, j, d] for d in range(D))
                        m = 0.0 if mask is None else mask[b, o, j]
                        s.append(scale * dot + bias[b, h, i, j] + m)
                    e = [math.exp(x) for x in s]          # no max shift: tiny inputs only
                    tot = sum(e)
                    LSE[b, o, h, i] = math.log(tot)
                    for d in range(D):
                        O[b, o, h, i, d] = sum(e[j] / tot * v[b, o, h, j, d] for j in range(N))
    return O, LSE


def test_forward_matches_bruteforce_loops():
    w, x = _inputs(3, 5, 2, 3, seed=11)
    mask = np.zeros((1, 3, 5))
    mask[0, 0, 1] = mask[0, 2, 4] = -30.0       # finite so that exp() without shift stays > 0
    O, LSE = oracle.forward(x["q"], x["k"], x["v"], x["bias"], mask, w.scale)
    Ob, LSEb = _bruteforce_forward(x["q"], x["k"], x["v"], x["bias"], mask, w.scale)
    assert np.max(np.abs(O - Ob)) <= 1e-12 * max(1.0, np.max(np.abs(Ob)))
    assert np.max(np.abs(LSE - LSEb)) <= 1e-12 * max(1.0, np.max(np.abs(LSEb)))


def test_forward_tiny_workload_bruteforce_rows():
    """The tiny workload (fp32 inputs, N=32): a sample of rows against the loop form."""
    w = synth.get("tiny")
    x = {n: (None if t is None else t.double().numpy()) for n, t in synth.make_inputs(w, 0).items()}
    O, LSE = oracle.forward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale)
    rng = np.random.default_rng(0)
    for _ in range(12):
        o, h, i = (int(rng.integers(w.N_o)), int(rng.integers(w.H)), int(rng.integers(w.N)))
        s = [w.scale * float(np.dot(x["q"][0, o, h, i], x["k"][0, o, h, j])) + x["bias"][0, h, i, j]
             for j in range(w.N)]
        e = [math.exp(t) for t in s]
        tot = math.fsum(e)
        assert abs(LSE[0, o, h, i] - math.log(tot)) < 1e-12 * abs(math.log(tot)) + 1e-13
        ref = [math.fsum(e[j] / tot * x["v"][0, o, h, j, d] for j in range(w.N)) for d in range(w.D)]
        assert np.max(np.abs(O[0, o, h, i] - np.array(ref))) < 1e-12


def test_forward_matches_torch_sdpa_without_bias():
    w, x = _inputs(3, 9, 2, 8, seed=3)
    zero = np.zeros_like(x["bias"])
    O, _ = oracle.forward(x["q"], x["k"], x["v"], zero, None, w.scale)
    t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in ("q", "k", "v")}
    Ot = torch.nn.functional.scaled_dot_product_attention(t["q"], t["k"], t["v"], scale=w.scale)
    assert np.max(np.abs(O - Ot.detach().numpy())) < 1e-12
    # gradients through the library route too
    (Ot * torch.tensor(x["do"])).sum().backward()
    g = oracle.backward(x["q"], x["k"], x["v"], zero, None, w.scale, x["do"])
    for n in ("q", "k", "v"):
        assert np.max(np.abs(g["d" + n] - t[n].grad.numpy())) < 1e-11


# ----------------------------------------------------------------------------- gradients


def _torch_grads(x, mask, scale):
    t = {n: torch.tensor(x[n], dtype=torch.float64, requires_grad=True) for n in ("q", "k", "v", "bias")}
    s = scale * torch.einsum("bohqd,bohkd->bohqk", t["q"], t["k"]) + t["bias"][:, None]
    if mask is not None:
        s = s + torch.tensor(mask)[:, :, None, None, :]
    p = torch.softmax(s, dim=-1)
    O = torch.einsum("bohqk,bohkd->bohqd", p, t["v"])
    (O * torch.tensor(x["do"])).sum().backward()
    return {"d" + n: t[n].grad.numpy() for n in t}, O.detach().numpy()


def _close(a, b, tol):
    return np.max(np.abs(a - b)) <= tol * max(1.0, float(np.max(np.abs(b))))


@pytest.mark.parametrize("mask_p,D", [(0.0, 4), (0.3, 4), (0.2, 64)])
def test_grads_match_torch_autograd(mask_p, D):
    w, x = _inputs(4, 6, 2, D, seed=5, mask_p=mask_p)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    tg, O = _torch_grads(x, x["mask"], w.scale)
    assert _close(g["o"], O, 1e-12)
    for n in ("dq", "dk", "dv", "dbias"):
        assert _close(g[n], tg[n], 1e-12), n


def _loss(x, mask, scale):
    O, _ = oracle.forward(x["q"], x["k"], x["v"], x["bias"], mask, scale)
    return float(np.sum(O * x["do"]))


def _fd_max_rel_err(x, mask, scale, grads, n_dirs=4, n_entries=12, eps=1e-5, seed=0):
    """Largest relative error between central differences and <grad, u>."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for name in ("q", "k", "v", "bias"):
        dirs = [rng.standard_normal(x[name].shape) for _ in range(n_dirs)]
        for _ in range(n_entries):
            u = np.zeros(x[name].shape)
            u.reshape(-1)[int(rng.integers(u.size))] = 1.0
            dirs.append(u)
        for u in dirs:
            xp = dict(x); xp[name] = x[name] + eps * u
            xm = dict(x); xm[name] = x[name] - eps * u
            fd = (_loss(xp, mask, scale) - _loss(xm, mask, scale)) / (2 * eps)
            an = float(np.sum(grads["d" + name] * u))
            worst = max(worst, abs(fd - an) / max(1e-3, abs(an)))
    return worst


def test_grads_match_finite_differences():
    w, x = _inputs(3, 5, 2, 4, seed=9, mask_p=0.25)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    assert _fd_max_rel_err(x, x["mask"], w.scale, g) < 1e-6


def test_finite_difference_pin_catches_planted_mistakes():
    """A dropped scale, a transposed bias gradient or a wrong sign must fail the FD pin."""
    w, x = _inputs(3, 5, 2, 4, seed=9, mask_p=0.25)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    for mutate in (lambda g: {**g, "dq": g["dq"] / w.scale},
                   lambda g: {**g, "dbias": np.swapaxes(g["dbias"], -1, -2)},
                   lambda g: {**g, "dk": -g["dk"]},
                   lambda g: {**g, "dv": g["dv"][:, ::-1]}):
        assert _fd_max_rel_err(x, x["mask"], w.scale, mutate(g), n_dirs=2, n_entries=4) > 1e-3


# ----------------------------------------------------------------------------- closed forms


def test_closed_form_zero_queries_gives_bias_softmax():
    from scipy.special import softmax
    w, x = _inputs(3, 7, 2, 4, seed=21, mask_p=0.3)
    x["q"][:] = 0.0
    O, LSE = oracle.forward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale)
    logits = x["bias"][:, None] + x["mask"][:, :, None, None, :]
    P = softmax(logits, axis=-1)
    assert np.max(np.abs(O - P @ x["v"])) < 1e-12
    from scipy.special import logsumexp
    assert np.max(np.abs(LSE - logsumexp(logits, axis=-1))) < 1e-12


def test_closed_form_zero_keys_gives_mean_value():
    w, x = _inputs(2, 6, 2, 4, seed=22)
    x["k"][:] = 0.0
    O, LSE = oracle.forward(x["q"], x["k"], x["v"], np.zeros_like(x["bias"]), None, w.scale)
    assert np.max(np.abs(O - x["v"].mean(axis=-2, keepdims=True))) < 1e-13
    assert np.max(np.abs(LSE - math.log(6))) < 1e-13


def test_closed_form_unit_values_kill_score_gradients():
    w, x = _inputs(3, 6, 2, 4, seed=23, mask_p=0.2)
    x["v"][:] = 1.0
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    assert np.max(np.abs(g["o"] - 1.0)) < 1e-13
    for n in ("dq", "dk", "dbias"):
        assert np.max(np.abs(g[n])) < 1e-12, n
    # dV[k] = sum_q P[q,k] dO[q]; with one key per row P = 1 (checked below separately)


def test_closed_form_single_key():
    w, x = _inputs(4, 1, 2, 8, seed=24)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], None, w.scale, x["do"])
    assert np.max(np.abs(g["o"] - x["v"])) == 0.0
    assert np.max(np.abs(g["dv"] - x["do"])) == 0.0
    for n in ("dq", "dk", "dbias"):
        assert np.max(np.abs(g[n])) == 0.0


# ----------------------------------------------------------------------------- invariants


def test_invariants():
    w, x = _inputs(5, 8, 2, 4, seed=31, mask_p=0.3)
    P = oracle.probabilities(x["q"], x["k"], x["bias"], x["mask"], w.scale)
    assert np.max(np.abs(P.sum(-1) - 1.0)) < 1e-13
    masked = x["mask"] < -1e8                                 # [1, N_o, N]
    assert masked.any() and (~masked).any()
    assert np.all(P[np.broadcast_to(masked[:, :, None, None, :], P.shape)] == 0.0)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    mk = np.broadcast_to(masked[:, :, None, :, None], g["dk"].shape)
    assert np.all(g["dk"][mk] == 0.0) and np.all(g["dv"][mk] == 0.0)
    # every row of dS sums to zero, so every row of dbias does too
    assert np.max(np.abs(g["dbias"].sum(-1))) < 1e-12
    # the softmax correction in both of its forms
    assert np.max(np.abs(g["delta"] - oracle.compensated_delta(g["o"], None, x["do"]))) < 1e-12


def test_dbias_is_sum_over_slices_of_score_gradient():
    """Give every slice its own copy of the bias (torch autograd); their gradients are dS_o."""
    w, x = _inputs(4, 6, 2, 4, seed=33, mask_p=0.2)
    t = {n: torch.tensor(x[n]) for n in ("q", "k", "v", "do")}
    bias_o = torch.tensor(np.broadcast_to(x["bias"][:, None], (1, 4, 2, 6, 6)).copy(), requires_grad=True)
    s = w.scale * torch.einsum("bohqd,bohkd->bohqk", t["q"], t["k"]) + bias_o
    s = s + torch.tensor(x["mask"])[:, :, None, None, :]
    O = torch.einsum("bohqk,bohkd->bohqd", torch.softmax(s, -1), t["v"])
    (O * t["do"]).sum().backward()
    dS = bias_o.grad.numpy()
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    assert np.max(np.abs(g["dbias"] - dS.sum(axis=1))) < 1e-12


def test_outer_slice_permutation():
    w, x = _inputs(5, 6, 2, 4, seed=35, mask_p=0.2)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    perm = np.array([3, 0, 4, 1, 2])
    xp = {n: (x[n][:, perm] if n in ("q", "k", "v", "do", "mask") else x[n]) for n in x}
    gp = oracle.backward(xp["q"], xp["k"], xp["v"], xp["bias"], xp["mask"], w.scale, xp["do"])
    for n in ("o", "dq", "dk", "dv", "lse"):
        assert np.max(np.abs(gp[n] - g[n][:, perm])) < 1e-13, n
    assert np.max(np.abs(gp["dbias"] - g["dbias"])) < 1e-12


def test_bias_row_shift_invariance():
    w, x = _inputs(3, 7, 2, 4, seed=37, mask_p=0.2)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    c = np.random.default_rng(1).standard_normal((1, 2, 7, 1)) * 3
    xs = dict(x); xs["bias"] = x["bias"] + c
    gs = oracle.backward(xs["q"], xs["k"], xs["v"], xs["bias"], xs["mask"], w.scale, xs["do"])
    assert np.max(np.abs(gs["o"] - g["o"])) < 1e-12
    assert np.max(np.abs(gs["lse"] - (g["lse"] + c[:, None, :, :, 0]))) < 1e-12
    for n in ("dq", "dk", "dv", "dbias"):
        assert np.max(np.abs(gs[n] - g[n])) < 1e-11, n


def test_worked_example_bias_index():
    """Figure 6: crop of seven tokens, one head; the bias of pair (4, 6) enters the score of
    query 4 and key 6 in every slice, and nothing else."""
    w, x = _inputs(7, 7, 1, 4, seed=41)
    O0, _ = oracle.forward(x["q"], x["k"], x["v"], x["bias"], None, w.scale)
    xb = x["bias"].copy()
    xb[0, 0, 4, 6] += 0.5
    O1, _ = oracle.forward(x["q"], x["k"], x["v"], xb, None, w.scale)
    diff = np.abs(O1 - O0).max(axis=-1)[0, :, 0, :]            # [o, q]
    assert np.all(diff[:, 4] > 0)                               # query 4 of every slice o
    assert np.all(np.delete(diff, 4, axis=1) == 0.0)            # no other query
    # the query of pair (2, 4) only affects the output of pair (2, 4)
    xq = x["q"].copy(); xq[0, 2, 0, 4] += 0.5
    O2, _ = oracle.forward(xq, x["k"], x["v"], x["bias"], None, w.scale)
    d2 = np.abs(O2 - O0).max(axis=-1)[0, :, 0, :]
    assert d2[2, 4] > 0 and np.count_nonzero(d2) == 1
    # the key of pair (2, 6) affects slice 2 only (all of its queries)
    xk = x["k"].copy(); xk[0, 2, 0, 6] += 0.5
    O3, _ = oracle.forward(x["q"], xk, x["v"], x["bias"], None, w.scale)
    d3 = np.abs(O3 - O0).max(axis=-1)[0, :, 0, :]
    assert np.all(d3[2] > 0) and np.all(np.delete(d3, 2, axis=0) == 0.0)


# ----------------------------------------------------------------------------- helpers


def test_compensated_delta_integers():
    rng = np.random.default_rng(2)
    o = rng.integers(-8, 8, (2, 3, 2, 5, 4)).astype(np.float64)
    e = rng.integers(-3, 3, o.shape).astype(np.float64) / 256.0
    do = rng.integers(-8, 8, o.shape).astype(np.float64)
    ref = np.einsum("...d,...d->...", do, o + e)               # exact: small dyadic values
    assert np.array_equal(oracle.compensated_delta(o, e, do), ref)
    assert np.array_equal(oracle.compensated_delta(o, None, do), np.einsum("...d,...d->...", do, o))


def test_sum_partials_closed_form():
    J, shape = 7, (3, 4)
    base = np.arange(12, dtype=np.float64).reshape(shape)
    parts = np.stack([base + i for i in range(J)])
    assert np.array_equal(oracle.sum_partials(parts), J * base + J * (J - 1) / 2)


def test_bf16_round_against_torch_edge_values():
    vals = [0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -(1 + 3 * 2 ** -8),
            3.14159, 1e-3, 65504.0, 2.0 ** -126, 2.0 ** -130, 2.0 ** -133, 3 * 2.0 ** -134,
            3.3895313892515355e38, 3.39e38, -3.39e38, 1e-40, 7.0e-45]
    rng = np.random.default_rng(3)
    vals += list(rng.standard_normal(2000).astype(np.float32).astype(np.float64))
    vals += list((rng.standard_normal(500) * 1e30).astype(np.float32).astype(np.float64))
    x = np.array(vals, dtype=np.float64)
    ref = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    got = oracle.bf16_round(x)
    assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.isinf(oracle.bf16_round(np.array([3.4e38]))[0])


def test_rmse_metrics():
    ref = np.array([3.0, 4.0])
    assert oracle.rel_rmse(ref, ref) == 0.0
    assert abs(oracle.rel_rmse(np.array([3.0, 4.0 + 5.0]), ref) - 1.0) < 1e-15
    assert abs(oracle.abs_rmse(np.array([4.0, 5.0]), ref) - 1.0) < 1e-15


def test_sampled_forms_equal_full_oracle():
    """The row/slice-restricted forms used at full size agree with the pinned full oracle."""
    w, x = _inputs(6, 9, 2, 4, seed=51, mask_p=0.2)
    g = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    rows = [(0, 0, 3), (0, 1, 8), (0, 1, 0)]
    r = oracle.dbias_rows(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"], rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(r[n] - g["dbias"][b, h, i])) < 1e-13
    sl = [(0, 5), (0, 2)]
    s = oracle.backward_slices(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"], sl)
    for n in ("o", "lse", "delta", "dq", "dk", "dv"):
        for j, (b, o) in enumerate(sl):
            assert np.max(np.abs(s[n][j] - g[n][b, o])) < 1e-13, n
