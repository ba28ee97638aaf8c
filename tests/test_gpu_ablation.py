"""Output-residual compensation on and off, following the pages' accuracy protocol
(TurboPairFormer, Figure 9): identical inputs and incoming gradients, ten seeds, the mean
absolute RMSE of the public bf16 gradients against the FP64 oracle with its sample standard
deviation, next to the floor of the FP64 result rounded once to bf16.

The residual enters only the softmax correction delta = sum_d dO (O + E), so O and dV are
bitwise the same in both runs and only dQ, dK and dbias move.  How much they move depends on
the inputs: delta's error without the residual is about one bf16 rounding of O, relative to
|dO| |O|, while the score gradient scales with dP - delta.  With N(0,1) values and a bias of
unit size the attention over hundreds of keys is nearly uniform, |O| is small and the
correction's error is negligible; with peaked attention or values of non-zero mean |O| is of
the size of |V| and the correction's error is a large share of the gradient error.  Both kinds
of workload are measured here; the reduction is asserted where the correction matters.

Each seed compares 4 sampled outer slices (dQ, dK) and 16 sampled dbias rows at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import np64, require_gpu

pytestmark = pytest.mark.gpu

SEEDS = range(10)
GRADS = ("dq", "dk", "dbias")
# (workload, least relative reduction of the mean absolute RMSE asserted for dQ, dK, dbias):
# None = reported only (the N(0,1) workloads, where the correction's error is negligible)
CASES = [("n384_d32", None), ("n640_d16", None), ("n768_d32_mask", None),
         ("n768_d32_mask_peaked", 0.15), ("n768_d32_mask_vmean", 0.15)]


def _bf16_once(x):
    """The FP64 values rounded to bf16 (through FP32: a double rounding that differs from a
    single one only within 2^-24 relative of a bf16 tie, immaterial for an RMSE)."""
    return torch.from_numpy(np.ascontiguousarray(x)).float().to(torch.bfloat16).double().numpy()


def _abs_rmse(a, b):
    return float(np.sqrt(np.mean((np.asarray(a) - np.asarray(b)) ** 2)))


def _one_seed(ta, w, seed):
    dev = synth.make_inputs_device(w, seed)
    res = {}
    o0 = dv0 = None
    for comp in (True, False):
        o, o_res, lse = ta.forward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], w.scale, comp)
        dq, dk, dv, dbias = ta.backward(dev["q"], dev["k"], dev["v"], dev["bias"], dev["mask"], w.scale,
                                        o, o_res, lse, dev["do"])
        torch.cuda.synchronize()
        if comp:
            o0, dv0 = o, dv
        else:
            assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
            assert torch.equal(dv.view(torch.int16), dv0.view(torch.int16))
        res[comp] = {"dq": dq, "dk": dk, "dbias": dbias}
    rng = np.random.default_rng(seed)
    slices = [int(o) for o in rng.choice(w.N_o, 4, replace=False)]
    rows = [(int(rng.integers(w.H)), int(q)) for q in rng.choice(w.N, 16, replace=False)]
    x = {n: dev[n].float().cpu().double().numpy() for n in ("q", "k", "v", "do", "bias")}
    x["mask"] = None if dev["mask"] is None else dev["mask"].cpu().double().numpy()
    ref = oracle.backward_slices(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"],
                                 [(0, o) for o in slices])
    ref["dbias"] = oracle.dbias_rows(x["q"], x["k"], x["v"], x["bias"], x["mask"], w.scale, x["do"],
                                     [(0, h, i) for h, i in rows])
    out = {}
    for n in GRADS:
        r = ref[n]
        pick = (lambda t: np.stack([np64(t[0, o]) for o in slices])) if n != "dbias" else \
               (lambda t: np.stack([np64(t[0, h, i]) for h, i in rows]))
        out[n] = {"on": _abs_rmse(pick(res[True][n]), r), "off": _abs_rmse(pick(res[False][n]), r),
                  "floor": _abs_rmse(_bf16_once(r), r)}
    return out


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_residual_compensation_ten_seeds(case):
    name, least = case
    ta = require_gpu()
    w = synth.get(name)
    per = []
    for seed in SEEDS:
        per.append(_one_seed(ta, w, seed))
        print(f"ablation {name} seed {seed}: " +
              " ".join(f"{n} {per[-1][n]['on']:.3e}/{per[-1][n]['off']:.3e}" for n in GRADS), flush=True)
    summary = {}
    for n in GRADS:
        on = np.array([p[n]["on"] for p in per])
        off = np.array([p[n]["off"] for p in per])
        fl = np.array([p[n]["floor"] for p in per])
        summary[n] = (on.mean(), on.std(ddof=1), off.mean(), off.std(ddof=1), fl.mean(), 1.0 - on.mean() / off.mean())
    print(f"ABLATION {name}: grad | with residual mean (sd) | without mean (sd) | bf16 floor | reduction")
    for n, (a, sa, b, sb, f, red) in summary.items():
        print(f"ABLATION {name}: {n} | {a:.4e} ({sa:.1e}) | {b:.4e} ({sb:.1e}) | {f:.4e} | {100 * red:.1f}%",
              flush=True)
    for n, (a, _, b, _, f, red) in summary.items():
        assert a <= b * 1.005, (n, a, b)          # never measurably worse with the residual
        if least is not None:
            assert red >= least, (n, red)
