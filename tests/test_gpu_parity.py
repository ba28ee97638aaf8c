"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Tolerances (relative RMSE over all compared elements, on bf16-rounded inputs):
O <= 5e-3 and dQ, dK, dV, dbias <= 1.5e-2.  The bf16 rounding of the output
alone is ~1.7e-3 for Gaussian data, so these leave ~3x headroom on O and ~4x
on the gradients (whose bf16 floor is similar).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import inputs, np64, require_gpu, row_ratio, run_gpu, to_dev, workload

pytestmark = pytest.mark.gpu

TOL_O = 5e-3
TOL_G = 1.5e-2

# (N_o, N, H, D, mask_p, bias_std, B): several tiles, ragged tails, every D, masks,
# all three bias-load paths (16-byte direct loads for N % 8 == 0, 4-byte direct loads
# for other even N, registers for odd N) and incomplete last outer groups
CASES = [
    (32, 32, 2, 16, 0.0, 1.0, 1),      # the tiny workload's shape, bf16-rounded
    (8, 1, 2, 32, 0.0, 1.0, 1),        # a single key (odd N)
    (6, 33, 2, 16, 0.2, 1.0, 1),       # odd N (register path), last group of 2 slices
    (9, 72, 3, 32, 0.1, 1.0, 1),       # ragged tail inside a 64-key tile, N % 8 == 0
    (5, 100, 2, 32, 0.3, 2.0, 2),      # N % 8 == 4 (4-byte loads), B = 2, masked
    (12, 200, 2, 32, 0.0, 1.0, 1),     # 4 key tiles, 4 query tiles, 2 query tiles of the forward
    (10, 130, 2, 16, 0.1, 2.0, 1),     # D = 16, masked, N % 8 == 2 (4-byte loads)
    (7, 64, 2, 32, 0.0, 1.0, 1),       # no mask, N % 8 == 0, last group of 3 slices
    (6, 48, 2, 16, 0.0, 2.0, 1),       # D = 16, no mask, N % 8 == 0, one group of 6 slices
    (8, 96, 2, 16, 0.15, 1.0, 1),      # D = 16, masked, N % 8 == 0, groups of 6 and 2 slices
    (7, 134, 3, 32, 0.0, 1.0, 1),      # no mask, N % 8 == 6 (4-byte loads), two key tiles
    (9, 67, 2, 32, 0.2, 1.0, 1),       # odd N, masked, D = 32
    (3, 63, 1, 16, 0.1, 1.0, 3),       # odd N, D = 16, one head, B = 3
    (5, 50, 2, 16, 0.0, 1.0, 1),       # D = 16, no mask, N % 8 == 2 (4-byte loads)
    (6, 72, 2, 64, 0.1, 1.0, 1),       # D = 64, masked, N % 8 == 0, three groups of 2 slices
    (5, 100, 2, 64, 0.3, 2.0, 1),      # D = 64, N % 8 == 4 (4-byte loads), last group of 1 slice
    (4, 200, 1, 64, 0.0, 1.0, 1),      # D = 64, 2 key tiles, 7 query tiles of 32 (stage cycle wraps)
    (7, 33, 2, 64, 0.2, 1.0, 2),       # D = 64, odd N (register path), B = 2
    (3, 130, 2, 64, 0.0, 1.0, 1),      # D = 64, no mask, N % 8 == 2, ragged key tile
    # D = 32, the query-tile kernel's plans: one 384-key range (4 waves x 96 keys, the last
    # wave mostly empty), two 256-key ranges, two and three 384-key ranges, and more slices
    # than 64 groups
    (2, 300, 1, 32, 0.1, 1.0, 1),
    (2, 504, 1, 32, 0.2, 1.0, 1),
    (2, 700, 1, 32, 0.1, 2.0, 1),
    (1, 800, 1, 32, 0.1, 1.0, 1),
    (70, 40, 1, 32, 0.1, 1.0, 1),
    # D = 16 past N = 640 (two kernels): 16-byte loads (64-key dK/dV tiles), 4-byte loads and
    # odd N (128-key dK/dV tiles, direct and register-staged), two and three key ranges
    (2, 656, 1, 16, 0.1, 1.0, 1),
    (2, 650, 1, 16, 0.2, 2.0, 1),
    (3, 771, 1, 16, 0.1, 1.0, 1),
]


def _id(c):
    return "No{}_N{}_H{}_D{}_m{}_b{}_B{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_fwd_bwd_matches_oracle(case):
    ta = require_gpu()
    N_o, N, H, D, mask_p, bstd, B = case
    w, _ = workload(N_o, N, H, D, mask_p, bstd, B=B)
    x = inputs(w, seed=N * 7 + D, mask_p=mask_p)
    print(f"case {_id(case)}", flush=True)
    got = run_gpu(ta, to_dev(x), w.scale)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    e_o = oracle.rel_rmse(np64(got["o"]), ref["o"])
    assert e_o <= TOL_O, e_o
    # and no single row far off (one wrong tile would not move the tensor-level figure much)
    assert row_ratio(np64(got["o"]), ref["o"], TOL_O) <= 3.0
    lse_err = np.max(np.abs(np64(got["lse"]) - ref["lse"]))
    assert lse_err <= 1e-3 + 1e-4 * np.max(np.abs(ref["lse"])), lse_err
    # the residual brings the stored output closer to the exact one
    e_oe = oracle.rel_rmse(np64(got["o"]) + np64(got["o_res"]), ref["o"])
    assert e_oe < e_o or e_oe < 1e-6, (e_oe, e_o)
    for n in ("dq", "dk", "dv", "dbias"):
        if np.max(np.abs(ref[n])) == 0.0:
            # exact zero in FP64 (a single key); the kernel's p for the row maximum is 1 up to
            # one FP32 rounding of the exponent argument, so tiny residues remain
            assert np.max(np.abs(np64(got[n]))) <= 1e-5, n
            continue
        e = oracle.rel_rmse(np64(got[n]), ref[n])
        assert e <= TOL_G, (n, e)
        rr = row_ratio(np64(got[n]), ref[n], TOL_G)
        assert rr <= 3.0, (n, rr)
    if x["mask"] is not None:
        masked = (x["mask"] < -1e8).numpy()                    # [B, N_o, N]
        mk = np.broadcast_to(masked[:, :, None, :, None], ref["dk"].shape)
        assert np.all(np64(got["dk"])[mk] == 0.0) and np.all(np64(got["dv"])[mk] == 0.0)


def test_tiny_workload_fp32_inputs():
    """The tiny workload: fp32 N(0,1) inputs; the GPU sees their bf16 rounding and is
    compared with the oracle on those rounded values."""
    ta = require_gpu()
    w = synth.get("tiny")
    x = synth.make_inputs(w, 0, bf16=False)
    xr = {n: (None if t is None else t.to(torch.bfloat16).float()) for n, t in x.items()}
    got = run_gpu(ta, to_dev(xr), w.scale)
    ref = oracle.backward(xr["q"], xr["k"], xr["v"], xr["bias"], xr["mask"], w.scale, xr["do"])
    assert oracle.rel_rmse(np64(got["o"]), ref["o"]) <= TOL_O
    for n in ("dq", "dk", "dv", "dbias"):
        assert oracle.rel_rmse(np64(got[n]), ref[n]) <= TOL_G, n


def test_delta_kernel_matches_oracle():
    ta = require_gpu()
    w, _ = workload(7, 45, 3, 32)
    d = ta.dims_of(torch.empty(w.B, w.N_o, w.H, w.N, w.D, device="meta"), w.scale)
    o = synth.bf16_tensor((1, 7, 3, 45, 32), 1)
    e = synth.bf16_tensor((1, 7, 3, 45, 32), 2, std=2.0 ** -9)
    do = synth.bf16_tensor((1, 7, 3, 45, 32), 3)
    for use_e in (True, False):
        delta = torch.empty((1, 7, 3, 45), dtype=torch.float32, device="cuda")
        ta.tri_attn_bwd_delta(d, o.to(torch.bfloat16).cuda(), e.to(torch.bfloat16).cuda() if use_e else None,
                              do.to(torch.bfloat16).cuda(), delta)
        torch.cuda.synchronize()
        ref = oracle.compensated_delta(o, e if use_e else None, do)
        x = o.double().numpy() + (e.double().numpy() if use_e else 0.0)
        bound = 32 * 2.0 ** -24 * np.sum(np.abs(do.double().numpy() * x), axis=-1)   # FP32 summation bound
        assert np.all(np.abs(np64(delta) - ref) <= bound + 1e-12)


@pytest.mark.parametrize("which", ["dq", "dbias"])
def test_reduce_kernels_match_oracle(which):
    ta = require_gpu()
    w, _ = workload(9, 70, 2, 16)
    d = ta.dims_of(torch.empty(w.B, w.N_o, w.H, w.N, w.D, device="meta"), w.scale)
    ws = ta.workspace(d)
    n = ws["dq_partial_elems"] if which == "dq" else ws["dbias_partial_elems"]
    parts = synth.bf16_tensor((n,), 5) * 3.0
    shape = (1, 9, 2, 70, 16) if which == "dq" else (1, 2, 70, 70)
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    if which == "dq":
        ta.tri_attn_reduce_dq(d, parts.cuda(), out)
    else:
        ta.tri_attn_reduce_dbias(d, parts.cuda(), out)
    torch.cuda.synchronize()
    P = ws["j_k"] if which == "dq" else ws["l"]
    exact = oracle.sum_partials(parts.double().numpy().reshape(P, -1)).reshape(shape)
    ref = oracle.bf16_round(exact)
    got = np64(out)
    # FP32 accumulation can move a value across a bf16 rounding boundary: at most one bf16 ulp
    ulp = np.where(ref != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(ref != 0, ref, 1.0)))) - 7), 2.0 ** -133)
    assert np.all(np.abs(got - ref) <= ulp)
    assert np.mean(got == ref) > 0.99


def test_bwd_kernel_with_oracle_statistics():
    """The main backward fed with the oracle's own lse and delta (FP64 -> FP32): isolates
    the backward kernel and the reductions from the forward."""
    ta = require_gpu()
    w, _ = workload(8, 136, 2, 32)
    x = inputs(w, seed=77, mask_p=0.15)
    ref = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    dev = to_dev(x)
    d = ta.dims_of(dev["q"], w.scale)
    ws = ta.workspace(d)
    lse = torch.tensor(ref["lse"], dtype=torch.float32).cuda()
    delta = torch.tensor(ref["delta"], dtype=torch.float32).cuda()
    dk, dv = torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    dqp = torch.full((ws["dq_partial_elems"],), float("nan"), device="cuda")
    dbp = torch.full((ws["dbias_partial_elems"],), float("nan"), device="cuda")
    ta.tri_attn_bwd(d, dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], dev["do"], lse, delta,
                    dk, dv, dqp, dbp)
    dq, dbias = torch.empty_like(dev["q"]), torch.empty_like(dev["bias"])
    ta.tri_attn_reduce_dq(d, dqp, dq)
    ta.tri_attn_reduce_dbias(d, dbp, dbias)
    torch.cuda.synchronize()
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dbias", dbias)):
        e = oracle.rel_rmse(np64(t), ref[n])
        assert e <= 6e-3, (n, e)       # no output-rounding error in delta here: tighter than the gate


def test_autograd_function_matches_entry_points():
    ta = require_gpu()
    w, _ = workload(6, 48, 2, 32)
    x = inputs(w, seed=3, mask_p=0.1)
    dev = to_dev(x)
    leaves = {n: dev[n].clone().requires_grad_(True) for n in ("q", "k", "v", "bias")}
    o = ta.triangular_attention(leaves["q"], leaves["k"], leaves["v"], leaves["bias"], dev["mask"], w.scale)
    o.backward(dev["do"])
    got = run_gpu(ta, dev, w.scale)
    assert torch.equal(o.detach(), got["o"])
    for n in ("q", "k", "v", "bias"):
        assert torch.equal(leaves[n].grad, got["d" + n]), n
    # boolean mask (True keeps) is the same as the additive one
    keep = dev["mask"] > -1.0
    o2 = ta.triangular_attention(dev["q"], dev["k"], dev["v"], dev["bias"], keep, w.scale)
    assert torch.equal(o2, got["o"])


def test_python_validation_on_device():
    ta = require_gpu()
    q = torch.zeros(1, 2, 1, 8, 32, dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros(1, 1, 8, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):
        ta.forward(q.float(), q, q, bias)
    with pytest.raises(ValueError):
        ta.forward(q, q, q, bias[:, :, :4])
    with pytest.raises(ValueError):
        ta.forward(q.transpose(3, 4).contiguous().transpose(3, 4), q, q, bias)
    q48 = torch.zeros(1, 2, 1, 8, 48, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ta.TriAttnError):
        ta.forward(q48, q48, q48, bias)


@pytest.mark.parametrize("case", [(9, 72, 3, 32, 0.1, 1.0, 1), (5, 100, 2, 32, 0.3, 2.0, 2), (8, 96, 2, 16, 0.15, 1.0, 1),
                                  (9, 67, 2, 32, 0.2, 1.0, 1), (6, 72, 2, 64, 0.1, 1.0, 1)], ids=_id)
def test_bf16_partials_variant_matches_oracle(case):
    """The bf16-partial variant (tri_attn_bwd_bf16p and its reductions): every gradient within
    the tolerance of the oracle, dK and dV bitwise equal to the FP32-partial path (they never
    pass through a partial), and repeated calls bitwise identical."""
    ta = require_gpu()
    N_o, N, H, D, mask_p, bstd, B = case
    w, _ = workload(N_o, N, H, D, mask_p, bstd, B=B)
    x = inputs(w, seed=N * 7 + D + 1, mask_p=mask_p)
    print(f"bf16 partials {_id(case)}", flush=True)
    dev = to_dev(x)
    mask = dev["mask"]
    o, o_res, lse = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], mask, w.scale)
    args = (dev["q"], dev["k"], dev["v"], dev["bias"], mask, w.scale, o, o_res, lse, dev["do"])
    g32 = ta.backward(*args)
    g16 = ta.backward(*args, bf16_partials=True)
    g16b = ta.backward(*args, bf16_partials=True)
    torch.cuda.synchronize()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"])
    for i, n in enumerate(("dq", "dk", "dv", "dbias")):
        assert torch.equal(g16[i], g16b[i]), n
        e = oracle.rel_rmse(np64(g16[i]), ref[n])
        assert e <= TOL_G, (n, e)
    assert torch.equal(g16[1], g32[1]) and torch.equal(g16[2], g32[2])
