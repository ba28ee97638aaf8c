"""Plain float64 triangle-attention block (starting and ending node) on the CPU.

TEST INFRASTRUCTURE ONLY: the oracle that the GPU block path is checked against.

What the block computes, from "TurboPairFormer: Fast and Stable Protein Folding
Model Training with an Optimized Triangle Attention Kernel":

* Table 1: pair features Z are ``[B, N, N, C_z]``; fixing an outer token o takes
  row o of Z as one slice; Q, K, V, O are ``[B, N_o, H, N, D]`` with N_o = N.
* Figure 6, steps 1-4: within slice o the pair (o, q) is projected to query q,
  the pair (o, k) to key k and value k; the score of (q, k) adds a bias taken
  from the pair (q, k), the same for every slice; the softmax-weighted values
  update the pair (o, q).  The caption notes that a normalisation precedes the
  projections.

The pages leave the rest of the block open; the plainest reading, used here
and by the GPU path:

* LayerNorm over C_z (biased variance, eps added inside the square root) with
  a per-feature scale ``gamma`` and shift ``beta``;
* Q, K, V and a gate g are linear maps C_z -> H*D of the normalised pair, the
  pair bias a linear map C_z -> H; no additive terms in any projection; the
  feature index within H*D is ``h*D + d``;
* the attention is the plain triangular attention (``tri_attn_fp64``) with
  scale 1/sqrt(D) and no mask;
* the gated output ``sigmoid(g) * O`` (per pair, per h*D feature) goes through
  a linear map H*D -> C_z; the block returns that update (no residual add);
* weights are stored ``[out, in]`` (``y = x @ W.T``): ``w_qkvg`` stacks the
  Q, K, V and gate maps as ``[4*H*D, C_z]``, ``w_b`` is ``[H, C_z]``,
  ``w_o`` is ``[C_z, H*D]``;
* the ending-node form applies the same block to Z with its two token axes
  swapped and swaps the axes of the result back.

The backward is the chain rule written out (no autograd); it is pinned in the
tests by central finite differences, by torch float64 autograd of a separate
forward, and by the dependency pattern of the worked example.  All arithmetic
is float64.
"""
from __future__ import annotations

import math

import numpy as np

from .tri_attn_fp64 import _f64, backward as attn_backward, forward as attn_forward


def layer_norm(z, gamma, beta, eps=1e-5):
    """LayerNorm over the last axis: returns ``(zln, xhat, rstd)``.

    ``xhat = (z - mean) / sqrt(var + eps)`` with the biased variance;
    ``zln = xhat * gamma + beta``.
    """
    z, gamma, beta = _f64(z), _f64(gamma), _f64(beta)
    mean = np.mean(z, axis=-1, keepdims=True)
    var = np.mean((z - mean) ** 2, axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (z - mean) * rstd
    return xhat * gamma + beta, xhat, rstd


def layer_norm_backward(dzln, xhat, rstd, gamma):
    """Gradients of LayerNorm: ``(dz, dgamma, dbeta)`` (dgamma, dbeta summed over all rows)."""
    dxhat = dzln * gamma
    C = dzln.shape[-1]
    m1 = np.sum(dxhat, axis=-1, keepdims=True) / C
    m2 = np.sum(dxhat * xhat, axis=-1, keepdims=True) / C
    dz = rstd * (dxhat - m1 - xhat * m2)
    lead = tuple(range(dzln.ndim - 1))
    return dz, np.sum(dzln * xhat, axis=lead), np.sum(dzln, axis=lead)


def _head_major(t, H, D):
    """``[B, N, N, H*D]`` (pair-major features) -> ``[B, N_o, H, N, D]``."""
    B, N, _, _ = t.shape
    return t.reshape(B, N, N, H, D).transpose(0, 1, 3, 2, 4)


def _pair_major(t):
    """``[B, N_o, H, N, D]`` -> ``[B, N, N, H*D]``."""
    B, N_o, H, N, D = t.shape
    return t.transpose(0, 1, 3, 2, 4).reshape(B, N_o, N, H * D)


def _orient(z, ending):
    """The pair tensor as the starting-node block sees it."""
    return np.swapaxes(z, 1, 2) if ending else z


def block_forward(z, gamma, beta, w_qkvg, w_b, w_o, H, D, ending=False, eps=1e-5):
    """Forward of the block.  Returns a dict with ``y [B,N,N,C_z]`` and every intermediate
    (in the starting-node orientation): ``zln, xhat, rstd, q, k, v, g, bias, o, lse``."""
    z = _orient(_f64(z), ending)
    w_qkvg, w_b, w_o = _f64(w_qkvg), _f64(w_b), _f64(w_o)
    HD = H * D
    zln, xhat, rstd = layer_norm(z, gamma, beta, eps)
    proj = zln @ w_qkvg.T                                   # [B,N,N,4HD]
    q, k, v, g = (_head_major(proj[..., i * HD:(i + 1) * HD], H, D) for i in range(4))
    bias = (zln @ w_b.T).transpose(0, 3, 1, 2)              # [B,H,N,N]: pair (q,k) -> bias[q,k]
    o, lse = attn_forward(q, k, v, bias, None, 1.0 / math.sqrt(D))
    gate = 1.0 / (1.0 + np.exp(-g))
    go = _pair_major(gate * o)                              # [B,N,N,HD]
    y = go @ w_o.T                                          # [B,N,N,C_z]
    return {"y": _orient(y, ending), "zln": zln, "xhat": xhat, "rstd": rstd, "q": q, "k": k,
            "v": v, "g": g, "bias": bias, "o": o, "lse": lse, "go": go}


def block_backward(z, gamma, beta, w_qkvg, w_b, w_o, dy, H, D, ending=False, eps=1e-5):
    """Gradients of ``L = sum(y * dy)``.

    Returns a dict: ``dz`` (same orientation as z), ``dw_qkvg, dw_b, dw_o, dgamma, dbeta``,
    and the intermediate gradients of the attention call ``do, dg, dq, dk, dv, dbias``
    (starting-node orientation, head-major like q).
    """
    f = block_forward(z, gamma, beta, w_qkvg, w_b, w_o, H, D, ending, eps)
    w_qkvg, w_b, w_o, gamma = _f64(w_qkvg), _f64(w_b), _f64(w_o), _f64(gamma)
    dy = _orient(_f64(dy), ending)
    HD = H * D
    B, N = dy.shape[0], dy.shape[1]
    # output projection: y = go @ w_o.T
    rows = B * N * N
    dw_o = dy.reshape(rows, -1).T @ f["go"].reshape(rows, -1)          # [C_z, HD]
    dgo = _head_major(dy @ w_o, H, D)                                  # [B,N_o,H,N,D]
    # gate: go = sigmoid(g) * o
    s = 1.0 / (1.0 + np.exp(-f["g"]))
    do = dgo * s
    dg = dgo * f["o"] * s * (1.0 - s)
    # the attention itself
    a = attn_backward(f["q"], f["k"], f["v"], f["bias"], None, 1.0 / math.sqrt(D), do)
    # projections: proj = zln @ w_qkvg.T, bias = zln @ w_b.T
    dproj = np.concatenate([_pair_major(a["dq"]), _pair_major(a["dk"]), _pair_major(a["dv"]),
                            _pair_major(dg)], axis=-1)                 # [B,N,N,4HD]
    dbias_pm = a["dbias"].transpose(0, 2, 3, 1)                        # [B,N,N,H]
    zln = f["zln"]
    dw_qkvg = dproj.reshape(rows, -1).T @ zln.reshape(rows, -1)
    dw_b = dbias_pm.reshape(rows, -1).T @ zln.reshape(rows, -1)
    dzln = dproj @ w_qkvg + dbias_pm @ w_b
    dz, dgamma, dbeta = layer_norm_backward(dzln, f["xhat"], f["rstd"], gamma)
    return {"dz": _orient(dz, ending), "dw_qkvg": dw_qkvg, "dw_b": dw_b, "dw_o": dw_o,
            "dgamma": dgamma, "dbeta": dbeta, "do": do, "dg": dg, "dq": a["dq"],
            "dk": a["dk"], "dv": a["dv"], "dbias": a["dbias"], "y": f["y"]}


def block_rows(z, gamma, beta, w_qkvg, w_b, w_o, dy, H, D, rows, ending=False, eps=1e-5):
    """``y`` and ``dz`` of whole pair rows without the full backward (for full-size sampling).

    ``rows = [(b, a), ...]`` name rows of the block's own orientation (for the ending node,
    row a of the swapped tensors, i.e. column a of ``y`` and ``dz``).  Row a needs slice a
    (its queries, keys, values and gate) and, for the bias gradient of pairs (a, .), query a
    of every slice: ``dbias[h, a, :] = sum_o dS_o[h, a, :]`` (Figure 6, step 5).  Same
    definitions and arithmetic as ``block_backward``; returns ``{"y": [R,N,C], "dz": [R,N,C]}``.
    """
    z = _orient(_f64(z), ending)
    dy = _orient(_f64(dy), ending)
    w_qkvg, w_b, w_o, gamma = _f64(w_qkvg), _f64(w_b), _f64(w_o), _f64(gamma)
    HD = H * D
    scale = 1.0 / math.sqrt(D)
    zln, xhat, rstd = layer_norm(z, gamma, beta, eps)
    wq, wk, wv, wg = (w_qkvg[i * HD:(i + 1) * HD] for i in range(4))
    N = z.shape[1]
    ys, dzs = [], []
    cache = {}
    for (b, a) in rows:
        if b not in cache:
            kb = (zln[b] @ wk.T).reshape(N, N, H, D).transpose(0, 2, 1, 3)     # [o,H,k,D]
            vb = (zln[b] @ wv.T).reshape(N, N, H, D).transpose(0, 2, 1, 3)
            biasb = (zln[b] @ w_b.T).transpose(2, 0, 1)                          # [H,q,k]
            cache = {b: (kb, vb, biasb)}
        kb, vb, biasb = cache[b]
        # slice a: forward and backward of the attention
        qa = (zln[b, a] @ wq.T).reshape(N, H, D).transpose(1, 0, 2)[None, None]  # [1,1,H,N,D]
        ga = (zln[b, a] @ wg.T).reshape(N, H, D).transpose(1, 0, 2)[None, None]
        ka, va = kb[a][None, None], vb[a][None, None]
        oa, _ = attn_forward(qa, ka, va, biasb[None], None, scale)
        sa = 1.0 / (1.0 + np.exp(-ga))
        go = _pair_major(sa * oa)[0, 0]                                          # [N,HD]
        ys.append(go @ w_o.T)
        dgo = (dy[b, a] @ w_o).reshape(N, H, D).transpose(1, 0, 2)[None, None]    # [1,1,H,N,D]
        do_a = dgo * sa
        dg_a = dgo * oa * sa * (1.0 - sa)
        g = attn_backward(qa, ka, va, biasb[None], None, scale, do_a)
        # query a of every slice o: the bias-gradient row a
        qc = (zln[b, :, a] @ wq.T).reshape(N, H, D)                               # [o,H,D]
        gc = (zln[b, :, a] @ wg.T).reshape(N, H, D)
        s = scale * np.einsum("ohd,ohkd->ohk", qc, kb) + biasb[None, :, a, :]
        m = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - m)
        p = e / np.sum(e, axis=-1, keepdims=True)                                # [o,H,k]
        oc = np.einsum("ohk,ohkd->ohd", p, vb)
        sc = 1.0 / (1.0 + np.exp(-gc))
        doc = (dy[b, :, a] @ w_o).reshape(N, H, D) * sc
        dp = np.einsum("ohd,ohkd->ohk", doc, vb)
        ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
        drow = np.zeros((H, N))
        for o in range(N):                                                        # ascending o
            drow = drow + ds[o]
        dproj = np.concatenate([_pair_major(g["dq"])[0, 0], _pair_major(g["dk"])[0, 0],
                                _pair_major(g["dv"])[0, 0], _pair_major(dg_a)[0, 0]], axis=-1)
        dzln = dproj @ w_qkvg + drow.T @ w_b
        dz, _, _ = layer_norm_backward(dzln, xhat[b, a], rstd[b, a], gamma)
        dzs.append(dz)
        del oc
    return {"y": np.stack(ys), "dz": np.stack(dzs)}
