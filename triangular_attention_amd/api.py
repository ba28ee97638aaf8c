"""Python entry points with the names of the C ABI, plus an autograd function.

The five calls (``tri_attn_fwd``, ``tri_attn_bwd_delta``, ``tri_attn_bwd``,
``tri_attn_reduce_dq``, ``tri_attn_reduce_dbias``) take device tensors,
check dtype/shape/contiguity, and pass raw pointers and the current HIP
stream to the library.  PyTorch only supplies memory and the stream.

``triangular_attention`` chains them as a ``torch.autograd.Function``:
forward = ``tri_attn_fwd``; backward = delta -> main backward -> the two
fixed-order reductions (TurboPairFormer, Figure 7(b)-(d)).
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib

MASK_VALUE = -1.0e9


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def dims_of(q: torch.Tensor, scale: float) -> _lib.Dims:
    if q.dim() != 5:
        raise ValueError("q must be [B, N_o, H, N, D]")
    B, N_o, H, N, D = q.shape
    return _lib.dims(B, N_o, H, N, D, scale)


def workspace(d: _lib.Dims, single_pass: bool = False) -> dict:
    """Partial-buffer sizes of the default backward (``tri_attn_workspace``) or, with
    ``single_pass``, of the single-pass key-tile kernel behind the bf16-partial variant and the
    chunked backward (``tri_attn_workspace_single_pass``); host-only, no device access."""
    lib = _lib.load()
    vals = [ctypes.c_int64() for _ in range(6)]
    name = "tri_attn_workspace_single_pass" if single_pass else "tri_attn_workspace"
    _lib.check(name, getattr(lib, name)(ctypes.byref(d), *[ctypes.byref(v) for v in vals]))
    keys = ("dq_partial_elems", "dbias_partial_elems", "j_k", "l", "key_tile", "outer_group")
    return {k: v.value for k, v in zip(keys, vals)}


def tri_attn_fwd(d, q, k, v, bias, mask, o, o_res, lse, stream=None):
    B, N_o, H, N, D = d.B, d.N_o, d.H, d.N, d.D
    x = (B, N_o, H, N, D)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, n, torch.bfloat16, x)
    _need(bias, "bias", torch.bfloat16, (B, H, N, N))
    if mask is not None:
        _need(mask, "mask", torch.float32, (B, N_o, N))
    if o_res is not None:
        _need(o_res, "o_res", torch.bfloat16, x)
    _need(lse, "lse", torch.float32, (B, N_o, H, N))
    lib = _lib.load()
    _lib.check("tri_attn_fwd", lib.tri_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(bias),
                                                _ptr(mask), _ptr(o), _ptr(o_res), _ptr(lse), _stream(stream)))


def tri_attn_bwd_delta(d, o, o_res, d_o, delta, stream=None):
    x = (d.B, d.N_o, d.H, d.N, d.D)
    _need(o, "o", torch.bfloat16, x)
    _need(d_o, "d_o", torch.bfloat16, x)
    if o_res is not None:
        _need(o_res, "o_res", torch.bfloat16, x)
    _need(delta, "delta", torch.float32, (d.B, d.N_o, d.H, d.N))
    lib = _lib.load()
    _lib.check("tri_attn_bwd_delta", lib.tri_attn_bwd_delta(ctypes.byref(d), _ptr(o), _ptr(o_res), _ptr(d_o),
                                                            _ptr(delta), _stream(stream)))


def _partial_dtype(bf16_partials):
    return torch.bfloat16 if bf16_partials else torch.float32


def _need_partial(t, name, dtype, elems):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous() \
            or t.numel() < elems:
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor with >= {elems} elements")


def tri_attn_bwd(d, q, k, v, bias, mask, d_o, lse, delta, dk, dv, dq_partial, dbias_partial, stream=None,
                 bf16_partials=False):
    """Main backward; ``bf16_partials`` selects ``tri_attn_bwd_bf16p`` (bf16 partial buffers)."""
    B, N_o, H, N, D = d.B, d.N_o, d.H, d.N, d.D
    x = (B, N_o, H, N, D)
    for n, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o), ("dk", dk), ("dv", dv)):
        _need(t, n, torch.bfloat16, x)
    _need(bias, "bias", torch.bfloat16, (B, H, N, N))
    if mask is not None:
        _need(mask, "mask", torch.float32, (B, N_o, N))
    _need(lse, "lse", torch.float32, (B, N_o, H, N))
    _need(delta, "delta", torch.float32, (B, N_o, H, N))
    ws = workspace(d, single_pass=bf16_partials)
    pdt = _partial_dtype(bf16_partials)
    _need_partial(dq_partial, "dq_partial", pdt, ws["dq_partial_elems"])
    _need_partial(dbias_partial, "dbias_partial", pdt, ws["dbias_partial_elems"])
    lib = _lib.load()
    name = "tri_attn_bwd_bf16p" if bf16_partials else "tri_attn_bwd"
    _lib.check(name, getattr(lib, name)(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
                                        _ptr(d_o), _ptr(lse), _ptr(delta), _ptr(dk), _ptr(dv),
                                        _ptr(dq_partial), _ptr(dbias_partial), _stream(stream)))


def tri_attn_reduce_dq(d, dq_partial, dq, stream=None, bf16_partials=False):
    """dQ from its partials; ``bf16_partials`` selects ``tri_attn_reduce_dq_bf16p``."""
    _need(dq, "dq", torch.bfloat16, (d.B, d.N_o, d.H, d.N, d.D))
    _need_partial(dq_partial, "dq_partial", _partial_dtype(bf16_partials),
                  workspace(d, single_pass=bf16_partials)["dq_partial_elems"])
    lib = _lib.load()
    name = "tri_attn_reduce_dq_bf16p" if bf16_partials else "tri_attn_reduce_dq"
    _lib.check(name, getattr(lib, name)(ctypes.byref(d), _ptr(dq_partial), _ptr(dq), _stream(stream)))


def tri_attn_reduce_dbias(d, dbias_partial, dbias, stream=None, bf16_partials=False):
    """dbias from its partials; ``bf16_partials`` selects ``tri_attn_reduce_dbias_bf16p``."""
    _need(dbias, "dbias", torch.bfloat16, (d.B, d.H, d.N, d.N))
    _need_partial(dbias_partial, "dbias_partial", _partial_dtype(bf16_partials),
                  workspace(d, single_pass=bf16_partials)["dbias_partial_elems"])
    lib = _lib.load()
    name = "tri_attn_reduce_dbias_bf16p" if bf16_partials else "tri_attn_reduce_dbias"
    _lib.check(name, getattr(lib, name)(ctypes.byref(d), _ptr(dbias_partial), _ptr(dbias), _stream(stream)))


def chunked_workspace(d, groups_per_chunk: int) -> dict:
    """Bytes the chunked backward needs for chunks of ``groups_per_chunk`` outer groups
    (``tri_attn_bwd_chunked_workspace``); host-only."""
    lib = _lib.load()
    nbytes, used = ctypes.c_int64(), ctypes.c_int64()
    _lib.check("tri_attn_bwd_chunked_workspace",
               lib.tri_attn_bwd_chunked_workspace(ctypes.byref(d), int(groups_per_chunk), ctypes.byref(nbytes),
                                                  ctypes.byref(used)))
    return {"bytes": nbytes.value, "groups_per_chunk": used.value}


def tri_attn_bwd_chunked(d, q, k, v, bias, mask, d_o, lse, delta, dq, dk, dv, dbias, workspace, stream=None):
    """Chunked backward (main backward + both reductions over chunks of outer groups whose
    partials fit in ``workspace``, a uint8 device tensor)."""
    B, N_o, H, N, D = d.B, d.N_o, d.H, d.N, d.D
    x = (B, N_o, H, N, D)
    for n, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, n, torch.bfloat16, x)
    for n, t in (("bias", bias), ("dbias", dbias)):
        _need(t, n, torch.bfloat16, (B, H, N, N))
    if mask is not None:
        _need(mask, "mask", torch.float32, (B, N_o, N))
    _need(lse, "lse", torch.float32, (B, N_o, H, N))
    _need(delta, "delta", torch.float32, (B, N_o, H, N))
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or not workspace.is_cuda \
            or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    lib = _lib.load()
    _lib.check("tri_attn_bwd_chunked",
               lib.tri_attn_bwd_chunked(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
                                        _ptr(d_o), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                        _ptr(dbias), _ptr(workspace), workspace.numel(), _stream(stream)))


def tri_attn_bwd_chunked_noalloc(d, q, k, v, bias, mask, d_o, lse, delta, dq, dk, dv, dbias, stream=None):
    """The chunked backward with the library's static scratch array (no allocation by the call)."""
    B, N_o, H, N, D = d.B, d.N_o, d.H, d.N, d.D
    x = (B, N_o, H, N, D)
    for n, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, n, torch.bfloat16, x)
    for n, t in (("bias", bias), ("dbias", dbias)):
        _need(t, n, torch.bfloat16, (B, H, N, N))
    if mask is not None:
        _need(mask, "mask", torch.float32, (B, N_o, N))
    _need(lse, "lse", torch.float32, (B, N_o, H, N))
    _need(delta, "delta", torch.float32, (B, N_o, H, N))
    lib = _lib.load()
    _lib.check("tri_attn_bwd_chunked_noalloc",
               lib.tri_attn_bwd_chunked_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(mask),
                                                _ptr(d_o), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                                                _ptr(dbias), _stream(stream)))


# --------------------------------------------------------------------------- composite calls


def forward(q, k, v, bias, mask=None, scale=None, compensate=True):
    """Returns ``(o, o_res or None, lse)``."""
    d = dims_of(q, (1.0 / math.sqrt(q.shape[-1])) if scale is None else scale)
    o = torch.empty_like(q)
    o_res = torch.empty_like(q) if compensate else None
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    tri_attn_fwd(d, q, k, v, bias, mask, o, o_res, lse)
    return o, o_res, lse


def backward(q, k, v, bias, mask, scale, o, o_res, lse, d_o, workspace_buffers=None, bf16_partials=False):
    """Delta, key-tile backward and the two reductions.  Returns ``(dq, dk, dv, dbias)``.
    ``bf16_partials`` runs the bf16-partial variant (half the partial bytes)."""
    d = dims_of(q, scale)
    ws = workspace(d, single_pass=bf16_partials)
    delta = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    tri_attn_bwd_delta(d, o, o_res, d_o, delta)
    if workspace_buffers is None:
        pdt = _partial_dtype(bf16_partials)
        dq_part = torch.empty(ws["dq_partial_elems"], dtype=pdt, device=q.device)
        db_part = torch.empty(ws["dbias_partial_elems"], dtype=pdt, device=q.device)
    else:
        dq_part, db_part = workspace_buffers
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    tri_attn_bwd(d, q, k, v, bias, mask, d_o, lse, delta, dk, dv, dq_part, db_part, bf16_partials=bf16_partials)
    dq = torch.empty_like(q)
    dbias = torch.empty_like(bias)
    # independent reductions; this order measured faster (the dQ reduction streams
    # better after the dbias reduction than straight after the backward)
    tri_attn_reduce_dbias(d, db_part, dbias, bf16_partials=bf16_partials)
    tri_attn_reduce_dq(d, dq_part, dq, bf16_partials=bf16_partials)
    return dq, dk, dv, dbias


def backward_chunked(q, k, v, bias, mask, scale, o, o_res, lse, d_o, groups_per_chunk=None, buffer=None):
    """Delta, then the chunked backward (bounded partial memory).  The workspace ``buffer``
    (uint8 device tensor) is allocated for ``groups_per_chunk`` outer groups (all groups when
    None) unless one is given.  Returns ``(dq, dk, dv, dbias)``, bitwise those of ``backward``."""
    d = dims_of(q, scale)
    if buffer is None:
        n = workspace(d, single_pass=True)["l"] if groups_per_chunk is None else groups_per_chunk
        buffer = torch.empty(chunked_workspace(d, n)["bytes"], dtype=torch.uint8, device=q.device)
    delta = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    tri_attn_bwd_delta(d, o, o_res, d_o, delta)
    dq, dk, dv, dbias = (torch.empty_like(t) for t in (q, k, v, bias))
    tri_attn_bwd_chunked(d, q, k, v, bias, mask, d_o, lse, delta, dq, dk, dv, dbias, buffer)
    return dq, dk, dv, dbias


class _TriAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, bias, mask, scale, compensate):
        o, o_res, lse = forward(q, k, v, bias, mask, scale, compensate)
        ctx.save_for_backward(q, k, v, bias, mask, o, o_res, lse)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, bias, mask, o, o_res, lse = ctx.saved_tensors
        dq, dk, dv, dbias = backward(q, k, v, bias, mask, ctx.scale, o, o_res, lse, d_o.contiguous())
        return dq, dk, dv, dbias, None, None, None


def triangular_attention(q, k, v, bias, mask=None, scale=None, compensate=True):
    """Triangular attention with a pair bias shared by every outer slice.

    q, k, v: ``[B, N_o, H, N, D]`` bf16 (D in {16, 32, 64}); bias ``[B, H, N, N]`` bf16;
    mask: ``[B, N_o, N]`` additive float32, or a bool tensor (True = keep), or None.
    Returns O ``[B, N_o, H, N, D]`` bf16; differentiable in q, k, v and bias.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if mask is not None and mask.dtype == torch.bool:
        mask = torch.where(mask, torch.zeros((), device=mask.device),
                           torch.full((), MASK_VALUE, device=mask.device)).float()
    if mask is not None:
        mask = mask.contiguous()
    return _TriAttn.apply(q.contiguous(), k.contiguous(), v.contiguous(), bias.contiguous(), mask,
                          float(scale), bool(compensate))
