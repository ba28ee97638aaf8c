"""Plain float64 triangle multiplicative update (outgoing and incoming) on the CPU.

TEST INFRASTRUCTURE ONLY: the oracle that the GPU triangle-multiplication path is checked against.

What is computed, from "TurboPairFormer: Fast and Stable Protein Folding Model
Training with an Optimized Triangle Attention Kernel", Figure 12 and Table 10:
an input step normalises the pair features and forms five projections -- two
branch values, two branch gates and the output gate logits -- and gates the
branch values; a contraction of the two branch operands independently for each
channel; an output step that normalises the contraction, projects it back to
the pair features and multiplies by the sigmoid of the saved output gate logits.

The plainest reading of the steps the figure names, used here and by the GPU path:

* ``zln = LayerNorm(z)`` over C_z (biased variance, eps inside the root, scale and shift);
* ``a = sigmoid(zln @ w_ag.T) * (zln @ w_ap.T)``, ``b`` likewise (C_z -> c channels),
  ``g = zln @ w_g.T`` (C_z -> C_z, the output gate logits); no additive terms;
* outgoing: ``x[i, j, ch] = sum_k a[i, k, ch] * b[j, k, ch]``;
  incoming: ``x[i, j, ch] = sum_k a[k, i, ch] * b[k, j, ch]``;
* ``out = sigmoid(g) * (LayerNorm_c(x) @ w_o.T)`` (c -> C_z), no residual add;
* weights ``[out, in]``; ``w_in`` stacks ``w_ap, w_ag, w_bp, w_bg`` (each ``[c, C_z]``) and
  ``w_g`` (``[C_z, C_z]``) as ``[4c + C_z, C_z]``; no pair mask.

The backward is the chain rule written out; it is pinned in the tests by finite
differences, by torch float64 autograd of a separately written forward, and by
a brute-force loop form of the channel contraction.
"""
from __future__ import annotations

import numpy as np

from .block_fp64 import layer_norm, layer_norm_backward
from .tri_attn_fp64 import _f64


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _split(w_in, c):
    return w_in[:c], w_in[c:2 * c], w_in[2 * c:3 * c], w_in[3 * c:4 * c], w_in[4 * c:]


def _cm(t):
    """``[B, N, N, c]`` -> per-channel matrices ``[B, c, N, N]``."""
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2))


def _pm(t):
    """``[B, c, N, N]`` -> ``[B, N, N, c]``."""
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1))


def contract(a, b, incoming):
    """The per-channel triangle contraction of ``[B, N, N, c]`` operands (one matrix product per
    channel): outgoing ``x[i,j] = sum_k a[i,k] b[j,k]``, incoming ``x[i,j] = sum_k a[k,i] b[k,j]``."""
    A, Bm = _cm(a), _cm(b)
    if incoming:
        return _pm(np.swapaxes(A, -1, -2) @ Bm)
    return _pm(A @ np.swapaxes(Bm, -1, -2))


def trimul_forward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, c, incoming=False, eps=1e-5):
    """Forward.  Returns ``out [B,N,N,C_z]`` and the intermediates in a dict."""
    z, w_in, w_o = _f64(z), _f64(w_in), _f64(w_o)
    zln, xhat, rstd = layer_norm(z, gamma, beta, eps)
    wap, wag, wbp, wbg, wg = _split(w_in, c)
    ap, ag, bp, bg = zln @ wap.T, zln @ wag.T, zln @ wbp.T, zln @ wbg.T
    g = zln @ wg.T
    a = _sig(ag) * ap
    b = _sig(bg) * bp
    x = contract(a, b, incoming)
    xln, xhat_o, rstd_o = layer_norm(x, gamma_o, beta_o, eps)
    p = xln @ w_o.T
    out = _sig(g) * p
    return {"out": out, "zln": zln, "xhat": xhat, "rstd": rstd, "ap": ap, "ag": ag, "bp": bp, "bg": bg,
            "g": g, "a": a, "b": b, "x": x, "xln": xln, "xhat_o": xhat_o, "rstd_o": rstd_o, "p": p}


def trimul_backward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, dout, c, incoming=False, eps=1e-5):
    """Gradients of ``L = sum(out * dout)``: ``dz, dw_in, dgamma, dbeta, dw_o, dgamma_o, dbeta_o``
    plus the intermediate gradients ``dx, da, db, dg`` and the forward's ``out``."""
    f = trimul_forward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, c, incoming, eps)
    w_in, w_o, gamma, gamma_o = _f64(w_in), _f64(w_o), _f64(gamma), _f64(gamma_o)
    dout = _f64(dout)
    B, N = dout.shape[0], dout.shape[1]
    rows = B * N * N
    s = _sig(f["g"])
    dp = dout * s
    dg = dout * f["p"] * s * (1.0 - s)
    dw_o = dp.reshape(rows, -1).T @ f["xln"].reshape(rows, -1)
    dxln = dp @ w_o
    dx, dgamma_o, dbeta_o = layer_norm_backward(dxln, f["xhat_o"], f["rstd_o"], gamma_o)
    a, b = f["a"], f["b"]
    DX, A, Bm = _cm(dx), _cm(a), _cm(b)
    if incoming:     # x[i,j] = sum_k a[k,i] b[k,j]: da[k,i] = sum_j b[k,j] dx[i,j], db[k,j] = sum_i a[k,i] dx[i,j]
        da = _pm(Bm @ np.swapaxes(DX, -1, -2))
        db = _pm(A @ DX)
    else:            # x[i,j] = sum_k a[i,k] b[j,k]: da[i,k] = sum_j dx[i,j] b[j,k], db[j,k] = sum_i dx[i,j] a[i,k]
        da = _pm(DX @ Bm)
        db = _pm(np.swapaxes(DX, -1, -2) @ A)
    sa, sb = _sig(f["ag"]), _sig(f["bg"])
    dap, dag = da * sa, da * f["ap"] * sa * (1.0 - sa)
    dbp, dbg = db * sb, db * f["bp"] * sb * (1.0 - sb)
    dproj = np.concatenate([dap, dag, dbp, dbg, dg], axis=-1)          # [B,N,N,4c+C_z]
    dw_in = dproj.reshape(rows, -1).T @ f["zln"].reshape(rows, -1)
    dzln = dproj @ w_in
    dz, dgamma, dbeta = layer_norm_backward(dzln, f["xhat"], f["rstd"], gamma)
    return {"dz": dz, "dw_in": dw_in, "dgamma": dgamma, "dbeta": dbeta, "dw_o": dw_o,
            "dgamma_o": dgamma_o, "dbeta_o": dbeta_o, "dx": dx, "da": da, "db": db, "dg": dg,
            "out": f["out"], "x": f["x"], "a": a, "b": b, "g": f["g"]}
