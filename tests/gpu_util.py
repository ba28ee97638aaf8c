"""Helpers shared by the GPU tests: run the HIP path on seeded inputs, compare with the oracle."""
import math

import numpy as np
import pytest
import torch

import synth


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import triangular_attention_amd as ta
    ta.load()          # fails loudly when the HIP library is missing
    return ta


def workload(N_o, N, H, D, mask_p=0.0, bias_std=1.0, scale=None, B=1):
    return synth.Workload("case", B, N_o, N, H, D, scale if scale is not None else 1.0 / math.sqrt(D),
                          bias_std=bias_std, mask_p=0.0, bf16=True), mask_p


def inputs(w, seed, mask_p=0.0):
    """CPU float32 tensors holding bf16 values (+ optional additive mask)."""
    x = synth.make_inputs(w, seed, bf16=True)
    if mask_p > 0:
        x["mask"] = synth.random_mask(w.B, w.N_o, w.N, mask_p, seed + 1000)
    elif w.mask_p > 0:
        pass
    return x


def to_dev(x):
    dev = {}
    for n in ("q", "k", "v", "do", "bias"):
        dev[n] = x[n].to(torch.bfloat16).cuda()
    dev["mask"] = None if x["mask"] is None else x["mask"].cuda()
    return dev


def run_gpu(ta, dev, scale, compensate=True):
    """Forward + backward through the five C-ABI calls.  Returns CPU float64 numpy arrays."""
    o, o_res, lse = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], scale, compensate)
    dq, dk, dv, dbias = ta.backward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], scale,
                                    o, o_res, lse, dev["do"])
    torch.cuda.synchronize()
    out = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "dbias": dbias}
    if o_res is not None:
        out["o_res"] = o_res
    return out


def np64(t):
    return t.detach().float().cpu().double().numpy()


def row_ratio(got, ref, tol, floor=0.25):
    """Largest per-row error of ``got`` against ``ref`` (rows = the last axis), in units of ``tol``.

    Each row's error ||g - r|| is divided by the larger of the row's own norm and ``floor``
    times the RMS row norm of the whole tensor (rows that are nearly zero in the reference,
    e.g. the key gradients of a masked key, are measured against the typical row), then by
    ``tol``.  A tensor-level relative RMSE can hide one wrong tile; this cannot: a wrong
    16 x 16 block gives rows whose error is comparable to their norm.
    """
    g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    rn = np.sqrt(np.sum(r * r, axis=1))
    rms = float(np.sqrt(np.mean(rn * rn)))
    if rms == 0.0:
        return float(np.max(np.abs(g))) / tol
    en = np.sqrt(np.sum((g - r) ** 2, axis=1))
    return float(np.max(en / np.maximum(rn, floor * rms))) / tol
