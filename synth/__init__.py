"""Seeded synthetic inputs for triangular attention.

This module is shared by the FP64 oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and rounds them to bf16; it holds none
of the attention arithmetic.

Shapes follow the TurboPairFormer notation table (Table 1): Q, K, V, O and the
incoming gradient dO are ``[B, N_o, H, N, D]`` (N_o outer slices of N x D per
head), the pair bias shared by every slice is ``[B, H, N, N]`` indexed
``[query, key]`` (Figure 6, step 3), and the optional per-slice key mask is an
additive ``[B, N_o, N]`` FP32 tensor (0 keeps a key, -1e9 masks it).

Draw order for one seed is fixed: Q, K, V, dO, bias, then the mask uniforms.
All draws happen in FP32 on the CPU with ``torch.Generator``; inputs whose
dtype is bf16 are rounded once with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

MASK_VALUE = -1.0e9


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N_o: int
    N: int
    H: int
    D: int
    scale: float
    bias_std: float = 1.0
    mask_p: float = 0.0          # Bernoulli probability that a key is masked
    v_mean: float = 0.0          # mean of the values (V ~ N(v_mean, 1))
    bf16: bool = True            # round Q/K/V/dO/bias to bf16
    description: str = ""

    @property
    def flops_fwd_bwd(self) -> float:
        """FlashAttention-style count: 4 (QK^T, PV) + 10 (S recompute, dV, dP, dQ, dK) x D per score."""
        return 14.0 * self.B * self.N_o * self.H * self.N * self.N * self.D

    @property
    def flops_fwd(self) -> float:
        return 4.0 * self.B * self.N_o * self.H * self.N * self.N * self.D

    @property
    def flops_bwd(self) -> float:
        return 10.0 * self.B * self.N_o * self.H * self.N * self.N * self.D

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(name, N, H, D, scale, **kw):
    return Workload(name=name, B=1, N_o=N, N=N, H=H, D=D, scale=scale, **kw)


#: The workloads the method is measured on (crop sizes 384/640/768, head dims 16/32, H=4).
WORKLOADS = {
    "tiny": _w("tiny", 32, 2, 16, 0.25, bf16=False,
               description="B=1 N_o=N=32 H=2 D=16, fp32 N(0,1) inputs and bias, scale 1/4, no mask"),
    "n384_d32": _w("n384_d32", 384, 4, 32, 1.0 / math.sqrt(32),
                   description="B=1 N_o=N=384 H=4 D=32 bf16 N(0,1), bias N(0,1), scale 1/sqrt(32), no mask"),
    "n640_d16": _w("n640_d16", 640, 4, 16, 0.25, bias_std=2.0,
                   description="B=1 N_o=N=640 H=4 D=16 bf16 N(0,1), bias N(0, std 2), scale 1/4, no mask"),
    "n768_d32_mask": _w("n768_d32_mask", 768, 4, 32, 1.0 / math.sqrt(32), mask_p=0.1,
                        description="B=1 N_o=N=768 H=4 D=32 bf16 N(0,1), bias N(0,1), "
                                    "per-slice key mask Bernoulli(0.1) additive -1e9, scale 1/sqrt(32)"),
    # the largest crop of the pages' memory table (Table 2), which they size but do not time
    "n1024_d32_mask": _w("n1024_d32_mask", 1024, 4, 32, 1.0 / math.sqrt(32), mask_p=0.1,
                         description="B=1 N_o=N=1024 H=4 D=32 bf16 N(0,1), bias N(0,1), "
                                     "per-slice key mask Bernoulli(0.1) additive -1e9, scale 1/sqrt(32)"),
    # a wider head than the pages measure: the crop-768 workload with D = 64
    "n768_d64_mask": _w("n768_d64_mask", 768, 4, 64, 1.0 / 8.0, mask_p=0.1,
                        description="B=1 N_o=N=768 H=4 D=64 bf16 N(0,1), bias N(0,1), "
                                    "per-slice key mask Bernoulli(0.1) additive -1e9, scale 1/sqrt(64)"),
}

#: Input regimes in which the softmax correction matters (the output-residual ablation): the
#: headline shape with strongly peaked attention (bias std 4), and with values of mean 2 (the
#: output is then far from zero while dP - delta, which does not depend on the values' mean,
#: stays of unit size).
REGIMES = {
    "n768_d32_mask_peaked": _w("n768_d32_mask_peaked", 768, 4, 32, 1.0 / math.sqrt(32), mask_p=0.1, bias_std=4.0,
                               description="as n768_d32_mask with bias N(0, std 4)"),
    "n768_d32_mask_vmean": _w("n768_d32_mask_vmean", 768, 4, 32, 1.0 / math.sqrt(32), mask_p=0.1, v_mean=2.0,
                              description="as n768_d32_mask with V ~ N(2, 1)"),
}

#: The six-shape sweep: crops {384, 640, 768} x head dims {16, 32}, H=4, no mask.
SWEEP = {f"sweep_n{n}_d{d}": _w(f"sweep_n{n}_d{d}", n, 4, d, 1.0 / math.sqrt(d),
                                description=f"B=1 N_o=N={n} H=4 D={d} bf16 N(0,1), bias N(0,1), "
                                            f"scale 1/sqrt({d}), no mask")
         for n in (384, 640, 768) for d in (16, 32)}


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in SWEEP:
        return SWEEP[name]
    if name in REGIMES:
        return REGIMES[name]
    raise KeyError(name)


def make_inputs(w: Workload, seed: int, bf16: Optional[bool] = None) -> dict:
    """Draw the inputs of one fwd+bwd call.

    Returns CPU tensors: ``q, k, v, do`` ``[B,N_o,H,N,D]`` and ``bias`` ``[B,H,N,N]``
    as float32 (holding bf16-representable values when rounding is on), plus
    ``mask`` ``[B,N_o,N]`` float32 or ``None``.
    """
    round_bf16 = w.bf16 if bf16 is None else bf16
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shp = (w.B, w.N_o, w.H, w.N, w.D)
    q = torch.randn(shp, generator=g, dtype=torch.float32)
    k = torch.randn(shp, generator=g, dtype=torch.float32)
    v = torch.randn(shp, generator=g, dtype=torch.float32)
    if w.v_mean:
        v = v + w.v_mean
    do = torch.randn(shp, generator=g, dtype=torch.float32)
    bias = torch.randn((w.B, w.H, w.N, w.N), generator=g, dtype=torch.float32) * w.bias_std
    mask = None
    if w.mask_p > 0.0:
        u = torch.rand((w.B, w.N_o, w.N), generator=g, dtype=torch.float32)
        keep = u >= w.mask_p
        # every slice keeps at least one key (a fully masked slice has no
        # well-defined softmax); at p=0.1 and N>=32 a failure has odds < 1e-32
        assert bool(keep.any(dim=-1).all()), "a slice has every key masked"
        mask = torch.where(keep, torch.zeros((), dtype=torch.float32),
                           torch.full((), MASK_VALUE, dtype=torch.float32))
    out = {"q": q, "k": k, "v": v, "do": do, "bias": bias}
    if round_bf16:
        out = {n: t.to(torch.bfloat16).to(torch.float32) for n, t in out.items()}
    out["mask"] = mask
    return out


def random_mask(B: int, N_o: int, N: int, p: float, seed: int) -> torch.Tensor:
    """Additive key mask [B,N_o,N] with P(masked)=p; every slice keeps key 0..N-1 at least once."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    u = torch.rand((B, N_o, N), generator=g, dtype=torch.float32)
    keep = u >= p
    none_kept = ~keep.any(dim=-1)
    keep[..., 0] |= none_kept
    return torch.where(keep, torch.zeros((), dtype=torch.float32),
                       torch.full((), MASK_VALUE, dtype=torch.float32))


def bf16_tensor(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    """A seeded N(0, std) tensor rounded to bf16 (returned as float32)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16).to(torch.float32)


def make_inputs_device(w: Workload, seed: int, device="cuda") -> dict:
    """Seeded inputs drawn on the device (for tests that need many large inputs and no
    oracle): same shapes, distributions and bf16 rounding as ``make_inputs``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    shp = (w.B, w.N_o, w.H, w.N, w.D)
    out = {}
    for n in ("q", "k", "v", "do"):
        x = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        out[n] = (x + w.v_mean if n == "v" and w.v_mean else x).to(torch.bfloat16)
    out["bias"] = (torch.randn((w.B, w.H, w.N, w.N), generator=g, device=device, dtype=torch.float32)
                   * w.bias_std).to(torch.bfloat16)
    out["mask"] = None
    if w.mask_p > 0.0:
        u = torch.rand((w.B, w.N_o, w.N), generator=g, device=device, dtype=torch.float32)
        keep = u >= w.mask_p
        keep[..., 0] |= ~keep.any(dim=-1)
        out["mask"] = torch.where(keep, torch.zeros((), device=device),
                                  torch.full((), MASK_VALUE, device=device)).float()
    return out


# --------------------------------------------------------------------------- triangle-attention block


@dataclasses.dataclass(frozen=True)
class BlockWorkload:
    """Inputs of the whole triangle-attention block: pair features Z [B, N, N, 128]."""
    name: str
    B: int
    N: int
    H: int
    D: int
    ending: bool = False
    w_std: float = 0.02          # weights ~ N(0, w_std), rounded to bf16
    ln_std: float = 0.0          # gamma = 1 + N(0, ln_std), beta = N(0, ln_std); 0: gamma 1, beta 0
    description: str = ""

    C_z = 128

    @property
    def pairs(self) -> int:
        return self.B * self.N * self.N

    @property
    def flops_fwd_bwd(self) -> float:
        """Attention (14 per score per head feature) + 3 x each projection's 2 * in * out per pair
        (forward, input gradient, weight gradient)."""
        F = self.H * self.D
        attn = 14.0 * self.B * self.N * self.H * self.N * self.N * self.D
        proj = 3 * 2.0 * self.pairs * self.C_z * (4 * F + self.H) + 3 * 2.0 * self.pairs * F * self.C_z
        return attn + proj


BLOCK_WORKLOADS = {
    "block_n768": BlockWorkload(
        "block_n768", 1, 768, 4, 32,
        description="triangle-attention block, starting node: B=1 N=768 C_z=128 H=4 D=32; "
                    "Z bf16 N(0,1), weights bf16 N(0,0.02), LayerNorm gamma 1 beta 0, dY bf16 N(0,1)"),
    "block_n768_end": BlockWorkload(
        "block_n768_end", 1, 768, 4, 32, ending=True,
        description="triangle-attention block, ending node: B=1 N=768 C_z=128 H=4 D=32; "
                    "Z bf16 N(0,1), weights bf16 N(0,0.02), LayerNorm gamma 1 beta 0, dY bf16 N(0,1)"),
}


def make_block_inputs(w: BlockWorkload, seed: int) -> dict:
    """Seeded block inputs as CPU float32 tensors (bf16-representable where the kernels take bf16).

    Draw order: Z, dY, w_qkvg, w_b, w_o, then gamma and beta (only when ``ln_std > 0``).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    C, F = w.C_z, w.H * w.D
    rb = lambda t: t.to(torch.bfloat16).to(torch.float32)
    out = {
        "z": rb(torch.randn((w.B, w.N, w.N, C), generator=g)),
        "dy": rb(torch.randn((w.B, w.N, w.N, C), generator=g)),
        "w_qkvg": rb(torch.randn((4 * F, C), generator=g) * w.w_std),
        "w_b": rb(torch.randn((w.H, C), generator=g) * w.w_std),
        "w_o": rb(torch.randn((C, F), generator=g) * w.w_std),
    }
    if w.ln_std > 0:
        out["gamma"] = 1.0 + torch.randn(C, generator=g) * w.ln_std
        out["beta"] = torch.randn(C, generator=g) * w.ln_std
    else:
        out["gamma"] = torch.ones(C)
        out["beta"] = torch.zeros(C)
    return out


# --------------------------------------------------------------------------- triangle multiplicative update


@dataclasses.dataclass(frozen=True)
class TrimulWorkload:
    """Inputs of the triangle multiplicative update: pair features Z [B, N, N, 128], c channels."""
    name: str
    B: int
    N: int
    c: int
    incoming: bool = False
    w_std: float = 0.02          # weights ~ N(0, w_std), rounded to bf16
    ln_std: float = 0.0          # gammas = 1 + N(0, ln_std), betas = N(0, ln_std); 0: 1 and 0
    description: str = ""

    C_z = 128

    @property
    def pairs(self) -> int:
        return self.B * self.N * self.N

    @property
    def flops_fwd_bwd(self) -> float:
        """3 x (input projections + per-channel contraction + output projection): forward, input
        gradient and weight (or second operand) gradient of each product."""
        P, C, c = self.pairs, self.C_z, self.c
        return 3 * (2.0 * P * C * (4 * c + C) + 2.0 * self.B * c * self.N ** 3 + 2.0 * P * c * C)


def _tm(name, N, c, inc):
    side = "incoming" if inc else "outgoing"
    return TrimulWorkload(name, 1, N, c, incoming=inc,
                          description=f"triangle multiplicative update, {side}: B=1 N={N} C_z=128 c={c}; "
                                      f"Z bf16 N(0,1), weights bf16 N(0,0.02), LayerNorm gammas 1 betas 0, "
                                      f"dout bf16 N(0,1)")


#: The pages' update sizes (Table 10): crops 384/640/768 with 128 channels, 384/640 with 64.
TRIMUL_WORKLOADS = {w.name: w for w in [
    _tm(f"trimul_n{n}_c{c}_{'in' if inc else 'out'}", n, c, inc)
    for (n, c) in ((384, 128), (640, 128), (768, 128), (384, 64), (640, 64)) for inc in (False, True)]}


def make_trimul_inputs(w: TrimulWorkload, seed: int) -> dict:
    """Seeded inputs as CPU float32 tensors (bf16-representable where the kernels take bf16).

    Draw order: Z, dout, w_in, w_o, then gamma, beta, gamma_o, beta_o (only when ``ln_std > 0``).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    C, c = w.C_z, w.c
    rb = lambda t: t.to(torch.bfloat16).to(torch.float32)
    out = {
        "z": rb(torch.randn((w.B, w.N, w.N, C), generator=g)),
        "dout": rb(torch.randn((w.B, w.N, w.N, C), generator=g)),
        "w_in": rb(torch.randn((4 * c + C, C), generator=g) * w.w_std),
        "w_o": rb(torch.randn((C, c), generator=g) * w.w_std),
    }
    if w.ln_std > 0:
        out["gamma"] = 1.0 + torch.randn(C, generator=g) * w.ln_std
        out["beta"] = torch.randn(C, generator=g) * w.ln_std
        out["gamma_o"] = 1.0 + torch.randn(c, generator=g) * w.ln_std
        out["beta_o"] = torch.randn(c, generator=g) * w.ln_std
    else:
        out["gamma"], out["beta"] = torch.ones(C), torch.zeros(C)
        out["gamma_o"], out["beta_o"] = torch.ones(c), torch.zeros(c)
    return out
