"""Python entry points of the triangle multiplicative update (C ABI: include/tri_mul.h).

The ``tri_mul_*`` functions check dtype/shape/contiguity and pass raw pointers and the
current HIP stream to the library; ``trimul_forward`` / ``trimul_backward`` chain them and
``triangle_multiplication`` wraps the update as a ``torch.autograd.Function``.  Every step runs
in the library's HIP kernels; PyTorch supplies memory and the stream.

The update (TurboPairFormer, Figure 12): LayerNorm of the pair features, five projections
(gated branch values a and b, output gate logits), one contraction per channel (outgoing
``x[i,j] = sum_k a[i,k] b[j,k]``, incoming ``x[i,j] = sum_k a[k,i] b[k,j]``), LayerNorm over the
channels, output projection, sigmoid gate.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from .api import _need, _ptr, _stream

C_Z = 128


def mul_dims(B, N, c, incoming=False, eps=1e-5) -> _lib.MulDims:
    return _lib.MulDims(int(B), int(N), C_Z, int(c), int(bool(incoming)), float(eps))


def mul_workspace(d: _lib.MulDims) -> dict:
    """Partial-buffer counts (``tri_mul_workspace``); host only."""
    lib = _lib.load()
    vals = [ctypes.c_int64() for _ in range(4)]
    _lib.check("tri_mul_workspace", lib.tri_mul_workspace(ctypes.byref(d), *[ctypes.byref(v) for v in vals]))
    return dict(zip(("n_w", "n_out", "n_ln", "n_lno"), (v.value for v in vals)))


def _shapes(d):
    B, N, c = d.B, d.N, d.c
    return (B, N, N, C_Z), (B, c, N, N), (B * N * N, 2)


def _f32(t, name, elems):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda \
            or not t.is_contiguous() or t.numel() < elems:
        raise ValueError(f"{name} must be a contiguous float32 device tensor with >= {elems} elements")


def tri_mul_in_fwd(d, z, gamma, beta, w_in, a, b, g, stats, stream=None):
    ps, cs, ss = _shapes(d)
    _need(z, "z", torch.bfloat16, ps)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(beta, "beta", torch.float32, (C_Z,))
    _need(w_in, "w_in", torch.bfloat16, (4 * d.c + C_Z, C_Z))
    _need(a, "a", torch.bfloat16, cs)
    _need(b, "b", torch.bfloat16, cs)
    _need(g, "g", torch.bfloat16, ps)
    _need(stats, "stats", torch.float32, ss)
    _lib.check("tri_mul_in_fwd", _lib.load().tri_mul_in_fwd(
        ctypes.byref(d), _ptr(z), _ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(a), _ptr(b), _ptr(g), _ptr(stats),
        _stream(stream)))


def tri_mul_contract(d, a, b, x, stream=None):
    _, cs, _ = _shapes(d)
    for n, t in (("a", a), ("b", b), ("x", x)):
        _need(t, n, torch.bfloat16, cs)
    _lib.check("tri_mul_contract", _lib.load().tri_mul_contract(
        ctypes.byref(d), _ptr(a), _ptr(b), _ptr(x), _stream(stream)))


def tri_mul_out_fwd(d, x, g, gamma_o, beta_o, w_o, out, stats_o, stream=None):
    ps, cs, ss = _shapes(d)
    _need(x, "x", torch.bfloat16, cs)
    _need(g, "g", torch.bfloat16, ps)
    _need(gamma_o, "gamma_o", torch.float32, (d.c,))
    _need(beta_o, "beta_o", torch.float32, (d.c,))
    _need(w_o, "w_o", torch.bfloat16, (C_Z, d.c))
    _need(out, "out", torch.bfloat16, ps)
    _need(stats_o, "stats_o", torch.float32, ss)
    _lib.check("tri_mul_out_fwd", _lib.load().tri_mul_out_fwd(
        ctypes.byref(d), _ptr(x), _ptr(g), _ptr(gamma_o), _ptr(beta_o), _ptr(w_o), _ptr(out), _ptr(stats_o),
        _stream(stream)))


def tri_mul_out_bwd(d, dout, x, g, stats_o, gamma_o, beta_o, w_o, dx, dg, wo_partial, lno_partial, stream=None):
    ps, cs, ss = _shapes(d)
    ws = mul_workspace(d)
    _need(dout, "dout", torch.bfloat16, ps)
    _need(x, "x", torch.bfloat16, cs)
    _need(g, "g", torch.bfloat16, ps)
    _need(stats_o, "stats_o", torch.float32, ss)
    _need(gamma_o, "gamma_o", torch.float32, (d.c,))
    _need(beta_o, "beta_o", torch.float32, (d.c,))
    _need(w_o, "w_o", torch.bfloat16, (C_Z, d.c))
    _need(dx, "dx", torch.bfloat16, cs)
    _need(dg, "dg", torch.bfloat16, ps)
    _f32(wo_partial, "wo_partial", ws["n_out"] * C_Z * d.c)
    _f32(lno_partial, "lno_partial", ws["n_lno"] * 2 * d.c)
    _lib.check("tri_mul_out_bwd", _lib.load().tri_mul_out_bwd(
        ctypes.byref(d), _ptr(dout), _ptr(x), _ptr(g), _ptr(stats_o), _ptr(gamma_o), _ptr(beta_o), _ptr(w_o),
        _ptr(dx), _ptr(dg), _ptr(wo_partial), _ptr(lno_partial), _stream(stream)))


def tri_mul_contract_bwd(d, dx, a, b, da, db, stream=None):
    _, cs, _ = _shapes(d)
    for n, t in (("dx", dx), ("a", a), ("b", b), ("da", da), ("db", db)):
        _need(t, n, torch.bfloat16, cs)
    _lib.check("tri_mul_contract_bwd", _lib.load().tri_mul_contract_bwd(
        ctypes.byref(d), _ptr(dx), _ptr(a), _ptr(b), _ptr(da), _ptr(db), _stream(stream)))


def tri_mul_in_bwd(d, z, stats, gamma, beta, w_in, da, db, dproj, stream=None):
    ps, cs, ss = _shapes(d)
    _need(z, "z", torch.bfloat16, ps)
    _need(stats, "stats", torch.float32, ss)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(beta, "beta", torch.float32, (C_Z,))
    _need(w_in, "w_in", torch.bfloat16, (4 * d.c + C_Z, C_Z))
    _need(da, "da", torch.bfloat16, cs)
    _need(db, "db", torch.bfloat16, cs)
    _need(dproj, "dproj", torch.bfloat16, (d.B * d.N * d.N, 4 * d.c))
    _lib.check("tri_mul_in_bwd", _lib.load().tri_mul_in_bwd(
        ctypes.byref(d), _ptr(z), _ptr(stats), _ptr(gamma), _ptr(beta), _ptr(w_in), _ptr(da), _ptr(db),
        _ptr(dproj), _stream(stream)))


def tri_mul_in_bwd_dz(d, z, stats, gamma, w_in, dproj, dg, dz, ln_partial, stream=None):
    ps, cs, ss = _shapes(d)
    _need(z, "z", torch.bfloat16, ps)
    _need(stats, "stats", torch.float32, ss)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(w_in, "w_in", torch.bfloat16, (4 * d.c + C_Z, C_Z))
    _need(dproj, "dproj", torch.bfloat16, (d.B * d.N * d.N, 4 * d.c))
    _need(dg, "dg", torch.bfloat16, ps)
    _need(dz, "dz", torch.bfloat16, ps)
    _f32(ln_partial, "ln_partial", mul_workspace(d)["n_ln"] * 2 * C_Z)
    _lib.check("tri_mul_in_bwd_dz", _lib.load().tri_mul_in_bwd_dz(
        ctypes.byref(d), _ptr(z), _ptr(stats), _ptr(gamma), _ptr(w_in), _ptr(dproj), _ptr(dg), _ptr(dz),
        _ptr(ln_partial), _stream(stream)))


def tri_mul_in_bwd_dw(d, z, stats, gamma, beta, dproj, dg, w_partial, stream=None):
    ps, cs, ss = _shapes(d)
    _need(z, "z", torch.bfloat16, ps)
    _need(stats, "stats", torch.float32, ss)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(beta, "beta", torch.float32, (C_Z,))
    _need(dproj, "dproj", torch.bfloat16, (d.B * d.N * d.N, 4 * d.c))
    _need(dg, "dg", torch.bfloat16, ps)
    _f32(w_partial, "w_partial", mul_workspace(d)["n_w"] * (4 * d.c + C_Z) * C_Z)
    _lib.check("tri_mul_in_bwd_dw", _lib.load().tri_mul_in_bwd_dw(
        ctypes.byref(d), _ptr(z), _ptr(stats), _ptr(gamma), _ptr(beta), _ptr(dproj), _ptr(dg), _ptr(w_partial),
        _stream(stream)))


def tri_mul_reduce_wgrad(d, w_partial, wo_partial, ln_partial, lno_partial, dw_in, dw_o, dgamma, dbeta,
                         dgamma_o, dbeta_o, stream=None):
    ws = mul_workspace(d)
    c = d.c
    _f32(w_partial, "w_partial", ws["n_w"] * (4 * c + C_Z) * C_Z)
    _f32(wo_partial, "wo_partial", ws["n_out"] * C_Z * c)
    _f32(ln_partial, "ln_partial", ws["n_ln"] * 2 * C_Z)
    _f32(lno_partial, "lno_partial", ws["n_lno"] * 2 * c)
    _need(dw_in, "dw_in", torch.float32, (4 * c + C_Z, C_Z))
    _need(dw_o, "dw_o", torch.float32, (C_Z, c))
    _need(dgamma, "dgamma", torch.float32, (C_Z,))
    _need(dbeta, "dbeta", torch.float32, (C_Z,))
    _need(dgamma_o, "dgamma_o", torch.float32, (c,))
    _need(dbeta_o, "dbeta_o", torch.float32, (c,))
    _lib.check("tri_mul_reduce_wgrad", _lib.load().tri_mul_reduce_wgrad(
        ctypes.byref(d), _ptr(w_partial), _ptr(wo_partial), _ptr(ln_partial), _ptr(lno_partial), _ptr(dw_in),
        _ptr(dw_o), _ptr(dgamma), _ptr(dbeta), _ptr(dgamma_o), _ptr(dbeta_o), _stream(stream)))


# --------------------------------------------------------------------------- composite calls


def trimul_forward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, c, incoming=False, eps=1e-5):
    """Forward: returns ``(out, saved)``."""
    B, N = z.shape[0], z.shape[1]
    d = mul_dims(B, N, c, incoming, eps)
    dev = z.device
    cs = (B, c, N, N)
    a = torch.empty(cs, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    x = torch.empty_like(a)
    g = torch.empty_like(z)
    stats = torch.empty((B * N * N, 2), dtype=torch.float32, device=dev)
    stats_o = torch.empty_like(stats)
    out = torch.empty_like(z)
    tri_mul_in_fwd(d, z, gamma, beta, w_in, a, b, g, stats)
    tri_mul_contract(d, a, b, x)
    tri_mul_out_fwd(d, x, g, gamma_o, beta_o, w_o, out, stats_o)
    return out, dict(d=d, a=a, b=b, x=x, g=g, stats=stats, stats_o=stats_o)


def trimul_backward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, saved, dout):
    """Backward: ``dict(dz, dw_in, dw_o, dgamma, dbeta, dgamma_o, dbeta_o)`` plus the intermediate
    gradients ``dx, dg, da, db, dproj`` for inspection."""
    d = saved["d"]
    c = d.c
    dev = z.device
    ws = mul_workspace(d)
    f32 = lambda n: torch.empty(n, dtype=torch.float32, device=dev)
    dx = torch.empty_like(saved["x"])
    dg = torch.empty_like(z)
    wo_part, lno_part = f32(ws["n_out"] * C_Z * c), f32(ws["n_lno"] * 2 * c)
    tri_mul_out_bwd(d, dout, saved["x"], saved["g"], saved["stats_o"], gamma_o, beta_o, w_o, dx, dg, wo_part, lno_part)
    da, db = torch.empty_like(saved["a"]), torch.empty_like(saved["b"])
    tri_mul_contract_bwd(d, dx, saved["a"], saved["b"], da, db)
    dproj = torch.empty((d.B * d.N * d.N, 4 * c), dtype=torch.bfloat16, device=dev)
    tri_mul_in_bwd(d, z, saved["stats"], gamma, beta, w_in, da, db, dproj)
    dz = torch.empty_like(z)
    ln_part = f32(ws["n_ln"] * 2 * C_Z)
    tri_mul_in_bwd_dz(d, z, saved["stats"], gamma, w_in, dproj, dg, dz, ln_part)
    w_part = f32(ws["n_w"] * (4 * c + C_Z) * C_Z)
    tri_mul_in_bwd_dw(d, z, saved["stats"], gamma, beta, dproj, dg, w_part)
    out = dict(dz=dz, dw_in=f32((4 * c + C_Z, C_Z)), dw_o=f32((C_Z, c)), dgamma=f32(C_Z), dbeta=f32(C_Z),
               dgamma_o=f32(c), dbeta_o=f32(c))
    tri_mul_reduce_wgrad(d, w_part, wo_part, ln_part, lno_part, out["dw_in"], out["dw_o"], out["dgamma"],
                         out["dbeta"], out["dgamma_o"], out["dbeta_o"])
    out.update(dx=dx, dg=dg, da=da, db=db, dproj=dproj)
    return out


class _TriMul(torch.autograd.Function):
    @staticmethod
    def forward(ctx, z, gamma, beta, w_in, gamma_o, beta_o, w_o, c, incoming, eps):
        out, saved = trimul_forward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, c, incoming, eps)
        ctx.saved = saved
        ctx.save_for_backward(z, gamma, beta, w_in, gamma_o, beta_o, w_o)
        return out

    @staticmethod
    def backward(ctx, dout):
        z, gamma, beta, w_in, gamma_o, beta_o, w_o = ctx.saved_tensors
        g = trimul_backward(z, gamma, beta, w_in, gamma_o, beta_o, w_o, ctx.saved, dout.contiguous())
        ctx.saved = None
        return (g["dz"], g["dgamma"], g["dbeta"], g["dw_in"].to(w_in.dtype), g["dgamma_o"], g["dbeta_o"],
                g["dw_o"].to(w_o.dtype), None, None, None)


def triangle_multiplication(z, gamma, beta, w_in, gamma_o, beta_o, w_o, incoming=False, eps=1e-5):
    """Triangle multiplicative update (outgoing, or incoming with ``incoming=True``).

    z ``[B, N, N, 128]`` bf16 (N % 8 == 0); gamma, beta ``[128]`` and gamma_o, beta_o ``[c]`` float32;
    w_in ``[4c + 128, 128]`` and w_o ``[128, c]`` bf16 (``[out, in]``), c in {64, 128}.  Returns the update
    ``[B, N, N, 128]`` bf16; differentiable in z and every parameter.
    """
    c = w_o.shape[1]
    return _TriMul.apply(z.contiguous(), gamma.contiguous(), beta.contiguous(), w_in.contiguous(),
                         gamma_o.contiguous(), beta_o.contiguous(), w_o.contiguous(), int(c), bool(incoming),
                         float(eps))
