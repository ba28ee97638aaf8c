"""Plain float64 triangular attention (forward and backward) on the CPU.

TEST INFRASTRUCTURE ONLY: the oracle that the GPU path is checked against.

Definitions (TurboPairFormer, Table 1, Figure 1(a), Figure 6):

* Q, K, V, O are ``[B, N_o, H, N, D]``; for one example b, outer slice o and
  head h each is an N x D matrix.  The pair bias ``[B, H, N, N]`` is indexed
  ``[query, key]`` and is the same for every outer slice o (Figure 6, step 3).
* Score: ``s[q,k] = scale * <Q[q], K[k]> + bias[q,k] + mask[o,k]``.  ``scale``
  multiplies the dot product only; bias and mask enter unscaled.  The mask is an
  additive per-slice key mask ``[B, N_o, N]`` (0 keeps, -1e9 removes a key).
* Softmax over keys k, then ``O[q] = sum_k P[q,k] V[k]`` (Figure 6, step 4).
* Backward (Figure 1(a), Figure 6 step 5): the three reduction axes are keys
  for dQ, queries for dK and dV, and outer slices for dbias::

      dV[k]  = sum_q P[q,k] dO[q]           dP[q,k] = <dO[q], V[k]>
      delta[q] = sum_k P[q,k] dP[q,k]       dS[q,k] = P[q,k] (dP[q,k] - delta[q])
      dQ[q]  = scale sum_k dS[q,k] K[k]     dK[k]   = scale sum_q dS[q,k] Q[q]
      dbias[h,q,k] = sum_o dS_(o,h)[q,k]

  The mask receives no gradient.

All arithmetic is float64 on the given (already bf16-rounded) values, which
float64 represents exactly.  Work is chunked over outer slices to bound memory;
no other blocking or reordering is applied.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _chunk(N_o: int, H: int, N: int, budget_bytes: float = 2.5e8) -> int:
    per_slice = H * N * N * 8.0
    return max(1, min(N_o, int(budget_bytes // per_slice)))


def _scores(q, k, bias_b, mask_bo, scale):
    """s[o,h,q,k] = scale * q.k + bias[h,q,k] + mask[o,k] for one chunk of slices."""
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))       # [oc,H,N,N]
    s = s + bias_b[None, :, :, :]                            # shared over o
    if mask_bo is not None:
        s = s + mask_bo[:, None, None, :]                    # per slice, per key
    return s


def _softmax_rows(s):
    """Row-wise softmax over the last (key) axis with the log-sum-exp (natural log)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=-1, keepdims=True)
    p = e / l
    lse = (m + np.log(l))[..., 0]
    return p, lse


def probabilities(q, k, bias, mask, scale) -> np.ndarray:
    """Materialised P ``[B,N_o,H,N,N]`` (small inputs only)."""
    q, k, bias, mask = _f64(q), _f64(k), _f64(bias), _f64(mask)
    B, N_o, H, N, D = q.shape
    P = np.empty((B, N_o, H, N, N))
    for b in range(B):
        s = _scores(q[b], k[b], bias[b], None if mask is None else mask[b], scale)
        P[b], _ = _softmax_rows(s)
    return P


def forward(q, k, v, bias, mask, scale):
    """Returns ``(O [B,N_o,H,N,D], LSE [B,N_o,H,N])`` in float64; LSE in natural log."""
    q, k, v, bias, mask = _f64(q), _f64(k), _f64(v), _f64(bias), _f64(mask)
    B, N_o, H, N, D = q.shape
    O = np.empty((B, N_o, H, N, D))
    LSE = np.empty((B, N_o, H, N))
    c = _chunk(N_o, H, N)
    for b in range(B):
        for o0 in range(0, N_o, c):
            o1 = min(N_o, o0 + c)
            s = _scores(q[b, o0:o1], k[b, o0:o1], bias[b],
                        None if mask is None else mask[b, o0:o1], scale)
            p, lse = _softmax_rows(s)
            O[b, o0:o1] = np.matmul(p, v[b, o0:o1])
            LSE[b, o0:o1] = lse
    return O, LSE


def backward(q, k, v, bias, mask, scale, do):
    """Plain backward of ``L = sum(O * dO)``.

    Returns a dict with float64 arrays ``o, lse, delta, dq, dk, dv, dbias``;
    ``delta[b,o,h,q] = sum_k P dP`` is the exact softmax correction.
    """
    q, k, v, bias, mask, do = _f64(q), _f64(k), _f64(v), _f64(bias), _f64(mask), _f64(do)
    B, N_o, H, N, D = q.shape
    out = {n: np.empty((B, N_o, H, N, D)) for n in ("o", "dq", "dk", "dv")}
    out["lse"] = np.empty((B, N_o, H, N))
    out["delta"] = np.empty((B, N_o, H, N))
    dbias = np.zeros((B, H, N, N))
    c = _chunk(N_o, H, N, budget_bytes=1.2e8)
    for b in range(B):
        for o0 in range(0, N_o, c):
            o1 = min(N_o, o0 + c)
            qs, ks, vs, dos = q[b, o0:o1], k[b, o0:o1], v[b, o0:o1], do[b, o0:o1]
            s = _scores(qs, ks, bias[b], None if mask is None else mask[b, o0:o1], scale)
            p, lse = _softmax_rows(s)
            del s
            out["o"][b, o0:o1] = np.matmul(p, vs)
            out["lse"][b, o0:o1] = lse
            out["dv"][b, o0:o1] = np.matmul(np.swapaxes(p, -1, -2), dos)
            dp = np.matmul(dos, np.swapaxes(vs, -1, -2))
            delta = np.sum(p * dp, axis=-1)
            out["delta"][b, o0:o1] = delta
            ds = p * (dp - delta[..., None])
            del dp, p
            out["dq"][b, o0:o1] = scale * np.matmul(ds, ks)
            out["dk"][b, o0:o1] = scale * np.matmul(np.swapaxes(ds, -1, -2), qs)
            for i in range(o1 - o0):            # sum over outer slices, ascending o
                dbias[b] += ds[i]
            del ds
    out["dbias"] = dbias
    return out


def compensated_delta(o, e, do) -> np.ndarray:
    """Softmax correction from a stored output and its residual (Figure 7(b)).

    ``delta_hat[...,q] = sum_d dO[q,d] * (O[q,d] + E[q,d])``; with ``e=None`` it is
    the uncompensated ``sum_d dO * O``.
    """
    o, do = _f64(o), _f64(do)
    x = o if e is None else o + _f64(e)
    return np.sum(do * x, axis=-1)


def sum_partials(partials) -> np.ndarray:
    """Sum of single-writer partial buffers over their leading index (Figure 7(d), Figure 11(a))."""
    p = _f64(partials)
    acc = np.zeros(p.shape[1:])
    for i in range(p.shape[0]):
        acc = acc + p[i]
    return acc


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Written from the IEEE-754 definition: bfloat16 has 8 significand bits
    (7 stored), 8 exponent bits and the float32 exponent range.  A value is
    rounded once, directly from float64.
    """
    x = _f64(x)
    out = np.empty_like(x)
    flat, res = x.reshape(-1), out.reshape(-1)
    for i, v in enumerate(flat):
        res[i] = _bf16_round_scalar(float(v))
    return out


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_NORMAL_EXP = -126
_BF16_MANT_BITS = 7


def _bf16_round_scalar(v: float) -> float:
    if math.isnan(v) or math.isinf(v) or v == 0.0:
        return v
    sign = -1.0 if v < 0 else 1.0
    a = abs(v)
    e = math.floor(math.log2(a))
    # guard against log2 rounding at exact powers of two
    if 2.0 ** e > a:
        e -= 1
    elif 2.0 ** (e + 1) <= a:
        e += 1
    e = max(e, _BF16_MIN_NORMAL_EXP)          # subnormals share the minimum exponent
    ulp = 2.0 ** (e - _BF16_MANT_BITS)
    n = a / ulp                               # exact in float64 (power-of-two scaling)
    lo = math.floor(n)
    frac = n - lo
    if frac > 0.5 or (frac == 0.5 and (lo % 2 == 1)):
        lo += 1
    r = lo * ulp
    # rounding past the largest finite value overflows to infinity
    if r > _BF16_MAX:
        halfway = _BF16_MAX + 2.0 ** (127 - _BF16_MANT_BITS - 1)
        return sign * (math.inf if a >= halfway else _BF16_MAX)
    return sign * r


def rel_rmse(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over all elements."""
    x, ref = _f64(x), _f64(ref)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((x - ref) ** 2)))
    return num / den if den > 0 else num


def abs_rmse(x, ref) -> float:
    x, ref = _f64(x), _f64(ref)
    return float(np.sqrt(np.mean((x - ref) ** 2)))


def dbias_rows(q, k, v, bias, mask, scale, do, rows):
    """dbias[b,h,i,:] for selected ``rows = [(b, h, i), ...]`` without materialising every slice.

    Row i of dS in slice o needs only query i of that slice and all of its keys,
    so one row of dbias costs O(N_o * N * D): this lets full-size results be
    sampled.  Same definition as ``backward``.
    """
    q, k, v, bias, mask, do = _f64(q), _f64(k), _f64(v), _f64(bias), _f64(mask), _f64(do)
    out = []
    for (b, h, i) in rows:
        s = scale * np.einsum("od,okd->ok", q[b, :, h, i], k[b, :, h]) + bias[b, h, i][None, :]
        if mask is not None:
            s = s + mask[b]
        p, _ = _softmax_rows(s)                                  # [N_o, N]
        dp = np.einsum("od,okd->ok", do[b, :, h, i], v[b, :, h])
        delta = np.sum(p * dp, axis=-1, keepdims=True)
        ds = p * (dp - delta)
        acc = np.zeros(ds.shape[1])
        for o in range(ds.shape[0]):                             # ascending o
            acc = acc + ds[o]
        out.append(acc)
    return np.stack(out)


def backward_slices(q, k, v, bias, mask, scale, do, slices):
    """``backward`` restricted to outer slices ``[(b, o), ...]`` (every output but dbias).

    Slices are independent for O, LSE, delta, dQ, dK and dV (Figure 1(a)); only
    dbias couples them.
    """
    q, k, v, bias, mask, do = _f64(q), _f64(k), _f64(v), _f64(bias), _f64(mask), _f64(do)
    res = {n: [] for n in ("o", "lse", "delta", "dq", "dk", "dv")}
    for (b, o) in slices:
        sub = lambda t: t[b:b + 1, o:o + 1]
        g = backward(sub(q), sub(k), sub(v), bias[b:b + 1],
                     None if mask is None else mask[b:b + 1, o:o + 1], scale, sub(do))
        for n in res:
            res[n].append(g[n][0, 0])
    return {n: np.stack(t) for n, t in res.items()}
