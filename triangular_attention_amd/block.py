"""Python entry points of the triangle-attention block (C ABI: include/tri_attn_block.h).

The ``tri_block_*`` functions check dtype/shape/contiguity and pass raw pointers
and the current HIP stream to the library; ``block_forward`` / ``block_backward``
chain them with the attention calls, and ``triangle_attention_block`` wraps the
whole block as a ``torch.autograd.Function``.  Every step runs in the library's
HIP kernels; PyTorch supplies memory and the stream.

The block (TurboPairFormer, Table 1 and Figure 6, completed in the plain
Pairformer form): LayerNorm of the pair features, projections to Q, K, V, a
gate and the pair bias, triangular attention, sigmoid gate, output projection.
``ending=True`` runs the ending-node form (Z with its token axes swapped).
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from .api import _need, _ptr, _stream
from . import api

C_Z = 128


def block_dims(B, N, H, D, ending=False, eps=1e-5) -> _lib.BlockDims:
    return _lib.BlockDims(int(B), int(N), C_Z, int(H), int(D), int(bool(ending)), float(eps))


def block_workspace(d: _lib.BlockDims) -> dict:
    """Partial-buffer counts (``tri_block_workspace``); host only."""
    lib = _lib.load()
    vals = [ctypes.c_int64() for _ in range(3)]
    _lib.check("tri_block_workspace",
               lib.tri_block_workspace(ctypes.byref(d), *[ctypes.byref(v) for v in vals]))
    return dict(zip(("n_out", "n_w", "n_ln"), (v.value for v in vals)))


def _shapes(d):
    B, N, H, D = d.B, d.N, d.H, d.D
    return (B, N, N, C_Z), (B, N, H, N, D), (B, H, N, N), (B, N, N, 2)


def tri_block_ln_proj(d, z, gamma, beta, w_qkvg, w_b, q, k, v, g, bias, ln_stats, stream=None):
    zs, hs, bs, ss = _shapes(d)
    F = d.H * d.D
    _need(z, "z", torch.bfloat16, zs)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(beta, "beta", torch.float32, (C_Z,))
    _need(w_qkvg, "w_qkvg", torch.bfloat16, (4 * F, C_Z))
    _need(w_b, "w_b", torch.bfloat16, (d.H, C_Z))
    for n, t in (("q", q), ("k", k), ("v", v), ("g", g)):
        _need(t, n, torch.bfloat16, hs)
    _need(bias, "bias", torch.bfloat16, bs)
    _need(ln_stats, "ln_stats", torch.float32, ss)
    lib = _lib.load()
    _lib.check("tri_block_ln_proj", lib.tri_block_ln_proj(
        ctypes.byref(d), _ptr(z), _ptr(gamma), _ptr(beta), _ptr(w_qkvg), _ptr(w_b), _ptr(q), _ptr(k),
        _ptr(v), _ptr(g), _ptr(bias), _ptr(ln_stats), _stream(stream)))


def tri_block_gate_out(d, o, g, w_o, y, stream=None):
    zs, hs, _, _ = _shapes(d)
    _need(o, "o", torch.bfloat16, hs)
    _need(g, "g", torch.bfloat16, hs)
    _need(w_o, "w_o", torch.bfloat16, (C_Z, d.H * d.D))
    _need(y, "y", torch.bfloat16, zs)
    lib = _lib.load()
    _lib.check("tri_block_gate_out", lib.tri_block_gate_out(
        ctypes.byref(d), _ptr(o), _ptr(g), _ptr(w_o), _ptr(y), _stream(stream)))


def _need_f32(t, name, elems):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda \
            or not t.is_contiguous() or t.numel() < elems:
        raise ValueError(f"{name} must be a contiguous float32 device tensor with >= {elems} elements")


def tri_block_gate_out_bwd(d, dy, o, g, w_o, d_o, d_g, wo_partial, stream=None):
    zs, hs, _, _ = _shapes(d)
    F = d.H * d.D
    _need(dy, "dy", torch.bfloat16, zs)
    for n, t in (("o", o), ("g", g), ("d_o", d_o), ("d_g", d_g)):
        _need(t, n, torch.bfloat16, hs)
    _need(w_o, "w_o", torch.bfloat16, (C_Z, F))
    _need_f32(wo_partial, "wo_partial", block_workspace(d)["n_out"] * C_Z * F)
    lib = _lib.load()
    _lib.check("tri_block_gate_out_bwd", lib.tri_block_gate_out_bwd(
        ctypes.byref(d), _ptr(dy), _ptr(o), _ptr(g), _ptr(w_o), _ptr(d_o), _ptr(d_g), _ptr(wo_partial),
        _stream(stream)))


def tri_block_proj_bwd_dz(d, z, ln_stats, gamma, w_qkvg, w_b, dq, dk, dv, dg, dbias, dz, ln_partial,
                          stream=None):
    zs, hs, bs, ss = _shapes(d)
    F = d.H * d.D
    _need(z, "z", torch.bfloat16, zs)
    _need(ln_stats, "ln_stats", torch.float32, ss)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(w_qkvg, "w_qkvg", torch.bfloat16, (4 * F, C_Z))
    _need(w_b, "w_b", torch.bfloat16, (d.H, C_Z))
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
        _need(t, n, torch.bfloat16, hs)
    _need(dbias, "dbias", torch.bfloat16, bs)
    _need(dz, "dz", torch.bfloat16, zs)
    _need_f32(ln_partial, "ln_partial", block_workspace(d)["n_ln"] * 2 * C_Z)
    lib = _lib.load()
    _lib.check("tri_block_proj_bwd_dz", lib.tri_block_proj_bwd_dz(
        ctypes.byref(d), _ptr(z), _ptr(ln_stats), _ptr(gamma), _ptr(w_qkvg), _ptr(w_b), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dg), _ptr(dbias), _ptr(dz), _ptr(ln_partial), _stream(stream)))


def tri_block_proj_bwd_dw(d, z, ln_stats, gamma, beta, dq, dk, dv, dg, dbias, w_partial, stream=None):
    zs, hs, bs, ss = _shapes(d)
    F = d.H * d.D
    _need(z, "z", torch.bfloat16, zs)
    _need(ln_stats, "ln_stats", torch.float32, ss)
    _need(gamma, "gamma", torch.float32, (C_Z,))
    _need(beta, "beta", torch.float32, (C_Z,))
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dg", dg)):
        _need(t, n, torch.bfloat16, hs)
    _need(dbias, "dbias", torch.bfloat16, bs)
    _need_f32(w_partial, "w_partial", block_workspace(d)["n_w"] * (4 * F + d.H) * C_Z)
    lib = _lib.load()
    _lib.check("tri_block_proj_bwd_dw", lib.tri_block_proj_bwd_dw(
        ctypes.byref(d), _ptr(z), _ptr(ln_stats), _ptr(gamma), _ptr(beta), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dg), _ptr(dbias), _ptr(w_partial), _stream(stream)))


def tri_block_reduce_wgrad(d, w_partial, wo_partial, ln_partial, dw_qkvg, dw_b, dw_o, dgamma, dbeta,
                           stream=None):
    F = d.H * d.D
    ws = block_workspace(d)
    _need_f32(w_partial, "w_partial", ws["n_w"] * (4 * F + d.H) * C_Z)
    _need_f32(wo_partial, "wo_partial", ws["n_out"] * C_Z * F)
    _need_f32(ln_partial, "ln_partial", ws["n_ln"] * 2 * C_Z)
    _need(dw_qkvg, "dw_qkvg", torch.float32, (4 * F, C_Z))
    _need(dw_b, "dw_b", torch.float32, (d.H, C_Z))
    _need(dw_o, "dw_o", torch.float32, (C_Z, F))
    _need(dgamma, "dgamma", torch.float32, (C_Z,))
    _need(dbeta, "dbeta", torch.float32, (C_Z,))
    lib = _lib.load()
    _lib.check("tri_block_reduce_wgrad", lib.tri_block_reduce_wgrad(
        ctypes.byref(d), _ptr(w_partial), _ptr(wo_partial), _ptr(ln_partial), _ptr(dw_qkvg), _ptr(dw_b),
        _ptr(dw_o), _ptr(dgamma), _ptr(dbeta), _stream(stream)))


# --------------------------------------------------------------------------- composite calls


def block_forward(z, gamma, beta, w_qkvg, w_b, w_o, H, D, ending=False, eps=1e-5):
    """The block's forward: returns ``(y, saved)`` with the tensors the backward needs."""
    B, N = z.shape[0], z.shape[1]
    d = block_dims(B, N, H, D, ending, eps)
    dev = z.device
    hs = (B, N, H, N, D)
    q, k, v, g = (torch.empty(hs, dtype=torch.bfloat16, device=dev) for _ in range(4))
    bias = torch.empty((B, H, N, N), dtype=torch.bfloat16, device=dev)
    stats = torch.empty((B, N, N, 2), dtype=torch.float32, device=dev)
    tri_block_ln_proj(d, z, gamma, beta, w_qkvg, w_b, q, k, v, g, bias, stats)
    o, o_res, lse = api.forward(q, k, v, bias, None, 1.0 / math.sqrt(D), True)
    y = torch.empty_like(z)
    tri_block_gate_out(d, o, g, w_o, y)
    saved = dict(d=d, q=q, k=k, v=v, g=g, bias=bias, stats=stats, o=o, o_res=o_res, lse=lse)
    return y, saved


def block_backward(z, gamma, beta, w_qkvg, w_b, w_o, saved, dy):
    """The block's backward.  Returns ``dict(dz, dw_qkvg, dw_b, dw_o, dgamma, dbeta)`` and, for
    inspection, the gradients of the attention call (``d_o, d_g, dq, dk, dv, dbias``)."""
    d = saved["d"]
    H, D = d.H, d.D
    F = H * D
    dev = z.device
    ws = block_workspace(d)
    d_o = torch.empty_like(saved["o"])
    d_g = torch.empty_like(saved["g"])
    wo_part = torch.empty(ws["n_out"] * C_Z * F, dtype=torch.float32, device=dev)
    tri_block_gate_out_bwd(d, dy, saved["o"], saved["g"], w_o, d_o, d_g, wo_part)
    dq, dk, dv, dbias = api.backward(saved["q"], saved["k"], saved["v"], saved["bias"], None,
                                     1.0 / math.sqrt(D), saved["o"], saved["o_res"], saved["lse"], d_o)
    dz = torch.empty_like(z)
    ln_part = torch.empty(ws["n_ln"] * 2 * C_Z, dtype=torch.float32, device=dev)
    tri_block_proj_bwd_dz(d, z, saved["stats"], gamma, w_qkvg, w_b, dq, dk, dv, d_g, dbias, dz, ln_part)
    w_part = torch.empty(ws["n_w"] * (4 * F + H) * C_Z, dtype=torch.float32, device=dev)
    tri_block_proj_bwd_dw(d, z, saved["stats"], gamma, beta, dq, dk, dv, d_g, dbias, w_part)
    out = dict(dz=dz, dw_qkvg=torch.empty((4 * F, C_Z), dtype=torch.float32, device=dev),
               dw_b=torch.empty((H, C_Z), dtype=torch.float32, device=dev),
               dw_o=torch.empty((C_Z, F), dtype=torch.float32, device=dev),
               dgamma=torch.empty(C_Z, dtype=torch.float32, device=dev),
               dbeta=torch.empty(C_Z, dtype=torch.float32, device=dev))
    tri_block_reduce_wgrad(d, w_part, wo_part, ln_part, out["dw_qkvg"], out["dw_b"], out["dw_o"],
                           out["dgamma"], out["dbeta"])
    out.update(d_o=d_o, d_g=d_g, dq=dq, dk=dk, dv=dv, dbias=dbias)
    return out


class _TriBlock(torch.autograd.Function):
    @staticmethod
    def forward(ctx, z, gamma, beta, w_qkvg, w_b, w_o, H, D, ending, eps):
        y, saved = block_forward(z, gamma, beta, w_qkvg, w_b, w_o, H, D, ending, eps)
        ctx.saved = saved
        ctx.save_for_backward(z, gamma, beta, w_qkvg, w_b, w_o)
        return y

    @staticmethod
    def backward(ctx, dy):
        z, gamma, beta, w_qkvg, w_b, w_o = ctx.saved_tensors
        g = block_backward(z, gamma, beta, w_qkvg, w_b, w_o, ctx.saved, dy.contiguous())
        ctx.saved = None
        return (g["dz"], g["dgamma"], g["dbeta"], g["dw_qkvg"].to(w_qkvg.dtype), g["dw_b"].to(w_b.dtype),
                g["dw_o"].to(w_o.dtype), None, None, None, None)


def triangle_attention_block(z, gamma, beta, w_qkvg, w_b, w_o, H=4, ending=False, eps=1e-5):
    """Triangle-attention block (starting node, or ending node with ``ending=True``).

    z ``[B, N, N, 128]`` bf16; gamma, beta ``[128]`` float32; w_qkvg ``[4*128, 128]``,
    w_b ``[H, 128]``, w_o ``[128, 128]`` bf16 (``[out, in]``); H * D = 128 with D in {16, 32}.
    Returns the update ``[B, N, N, 128]`` bf16; differentiable in z and every parameter
    (weight gradients are computed in FP32 and returned in the weights' dtype).
    """
    D = 128 // H
    return _TriBlock.apply(z.contiguous(), gamma.contiguous(), beta.contiguous(), w_qkvg.contiguous(),
                           w_b.contiguous(), w_o.contiguous(), int(H), int(D), bool(ending), float(eps))
