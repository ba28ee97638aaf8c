"""Benchmark: triangular attention forward + backward on one MI355X.

One step = the whole hot path on one batch of synthetic input: tri_attn_fwd,
tri_attn_bwd_delta, tri_attn_bwd, tri_attn_reduce_dq, tri_attn_reduce_dbias.
Inputs, outputs and partial buffers are resident in HBM before timing starts.

Prints ONE JSON line (rank 0) with the throughput in TFLOP/s (FlashAttention
count 14*B*N_o*H*N^2*D per fwd+bwd), the per-kernel breakdown, the roofline
of the dominant kernel (HIP events on the launch stream), and the FP64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published 8 TB/s)
# the dbias reduction runs first: measured, the dQ reduction streams 10% faster after it
# than straight after the backward, and the dbias reduction loses less in that place
KERNELS = ("fwd", "delta", "bwd", "reduce_dbias", "reduce_dq")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="n768_d32_mask")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-compensate", action="store_true", help="run without the output residual")
    ap.add_argument("--partials", choices=("fp32", "bf16"), default="fp32",
                    help="partial precision: fp32 (the reference contract) or the bf16-partial variant")
    ap.add_argument("--chunk-groups", type=int, default=0,
                    help="run the backward as tri_attn_bwd_chunked with chunks of this many outer groups "
                         "(bounded partial memory); 0 = the unchunked calls")
    ap.add_argument("--sweep", action="store_true",
                    help="bench the pages' six timing shapes and the three configured workloads, each with the "
                         "oracle timed beside it (--cpu-seconds each), and print a table")
    ap.add_argument("--cpu-seconds", type=float, default=25.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after timing, also run a plain device copy of this many bytes (3 times): the "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write a markdown summary of a rocprofv3 --kernel-trace --stats output dir and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn FETCH_SIZE / WRITE_SIZE counter runs into per-launch bytes and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PASS_DIR",
                    help="summarise rocprofv3 --pmc passes (SQ_* / GRBM_* counters) into per-kernel "
                         "utilisation figures (--out: the markdown file; --counters: the JSON they go to)")
    ap.add_argument("--counters", default=os.path.join(ROOT, "profiles", "counters.json"),
                    help="per-kernel counter summary (MFMA busy fraction etc.), valid for the sources it was "
                         "measured on")
    ap.add_argument("--command", default="", help="the command line that produced the profile (recorded)")
    ap.add_argument("--out", default="", help="output file of the summarize modes")
    return ap.parse_args()


def algorithmic(w, jk, L, pb=4, two_kernel=False):
    """Algorithmic flops and minimum HBM bytes of one launch of each call (pb = bytes per
    partial element).  The backward call's flops are the method's (one recompute of S); its
    bytes are each tensor once per kernel: with two kernels (dK/dV key-tile kernel and dQ/dbias
    query-tile kernel) Q, K, V, dO, the bias, lse, delta and the mask are read by both."""
    X = w.B * w.N_o * w.H * w.N * w.D
    Y = w.B * w.H * w.N * w.N
    R = w.B * w.N_o * w.H * w.N
    M = w.B * w.N_o * w.N if w.mask_p > 0 else 0
    S = w.B * w.N_o * w.H * w.N * w.N
    return {
        "fwd": {"flops": 4.0 * S * w.D, "bytes": 2 * (3 * X + Y + 2 * X) + 4 * (M + R)},
        "delta": {"flops": 2.0 * X, "bytes": 2 * 3 * X + 4 * R},
        "bwd": {"flops": 10.0 * S * w.D,
                "bytes": (2 * (8 * X + 2 * Y + 2 * X) + 4 * (4 * R + 2 * M) if two_kernel else
                          2 * (4 * X + Y + 2 * X) + 4 * (2 * R + M)) + pb * (jk * X + L * Y)},
        "reduce_dq": {"flops": float(jk * X), "bytes": pb * jk * X + 2 * X},
        "reduce_dbias": {"flops": float(L * Y), "bytes": pb * L * Y + 2 * Y},
    }


def cpu_baseline(w, seconds):
    """The FP64 oracle (as it stands) on the first S outer slices of the same workload."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    x = synth.make_inputs(w, 0)
    sub = lambda t, s: None if t is None else t[:, :s].contiguous()

    def run(s):
        t0 = time.perf_counter()
        oracle.backward(sub(x["q"], s), sub(x["k"], s), sub(x["v"], s), x["bias"], sub(x["mask"], s),
                        w.scale, sub(x["do"], s))
        return time.perf_counter() - t0

    s0 = min(4, w.N_o)
    t0 = run(s0)
    s = int(max(s0, min(w.N_o, s0 * seconds / max(t0, 1e-3))))
    t = run(s) if s != s0 else t0
    flops = 14.0 * w.B * s * w.H * w.N * w.N * w.D
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fwd+bwd of outer slices 0..{s - 1} of {w.N_o} (all heads, all queries/keys) "
                      f"of workload {w.name}, seed 0, FP64 numpy; {t:.1f} s",
            "seconds": t, "slices": s, "threads_note": "BLAS threads (numpy elementwise ops run on one core)"}


def _short_kernel_name(name):
    name = name.replace("void ", "")
    if "copy" in name.lower() or "elementwise" in name.lower():
        return "copy:" + name.split("(")[0][-60:]
    if "tri::" in name:
        # keep template arguments: cut the parameter list at the first "(" after the last "::"
        base = name.replace("(anonymous namespace)::", "").replace("tri::", "")
        return base.split("(")[0]
    return name.split("(")[0][-60:]


def summarize_trace(d, command, out):
    """Markdown table from rocprofv3 --kernel-trace --stats (kernel_stats.csv)."""
    import csv
    import glob
    f = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not f:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(f[0])))
    lines = ["# rocprofv3 kernel-trace summary", "", f"Command: `{command}`", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| {} | {} | {:.1f} | {:.1f} | {:.1f} | {:.1f}% |".format(
            _short_kernel_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    txt = "\n".join(lines) + "\n"
    if out:
        open(out, "w").write(txt)
    print(txt)


N_XCD, N_SIMD = 8, 1024      # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_counters(dirs, workload, command, out, counters_json):
    """Per-kernel utilisation from rocprofv3 --pmc passes (each pass its own run).

    Per dispatch the counters are summed over the whole GPU: GRBM_GUI_ACTIVE over the 8 XCDs (so
    GRBM_GUI_ACTIVE / 8 is the kernel's duration in GPU cycles), SQ_VALU_MFMA_BUSY_CYCLES and
    SQ_VALU_MFMA_COEXEC_CYCLES over the 1024 SIMDs (cycles), SQ_ACTIVE_INST_VALU over waves (issue
    cycles of 4 clocks each for wave64).  Fractions are of the SIMD cycles of the dispatch:
    MFMA busy = MFMA_BUSY / (1024 * cycles); VALU busy = 4 * ACTIVE_INST_VALU / (1024 * cycles);
    co-exec = COEXEC / (1024 * cycles).  The median over dispatches is taken per counter."""
    import csv
    import glob
    vals = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                k = _short_kernel_name(r["Kernel_Name"])
                if k.startswith("copy:"):
                    continue
                dur = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3
                v = vals.setdefault(k, {})
                v.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                v.setdefault("_dur_us", []).append(dur)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    res = {"workload": workload, "kernel_hash": kernel_hash(_hash_files(workload)), "command": command,
           "kernels": {}}
    for k, v in vals.items():
        m = {c: med(x) for c, x in v.items()}
        g = m.get("GRBM_GUI_ACTIVE")
        if not g:
            continue
        cyc = g / N_XCD
        row = {"cycles": cyc, "us_under_counters": m["_dur_us"],
               "clock_ghz": cyc / (m["_dur_us"] * 1e3) if m["_dur_us"] > 0 else None}
        simd = N_SIMD * cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            row["mfma_busy"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / simd
        if "SQ_ACTIVE_INST_VALU" in m:
            row["valu_busy"] = 4.0 * m["SQ_ACTIVE_INST_VALU"] / simd
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
            row["mfma_valu_coexec"] = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd
        if "SQ_INSTS_MFMA" in m and m["SQ_INSTS_MFMA"] > 0 and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            row["mfma_cycles_per_inst"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / m["SQ_INSTS_MFMA"]
        waves = m.get("SQ_WAVES")
        for c, name in (("SQ_INSTS_VALU", "valu_insts_per_wave"), ("SQ_INSTS_MFMA", "mfma_insts_per_wave"),
                        ("SQ_INSTS_LDS", "lds_insts_per_wave"), ("SQ_INSTS_SALU", "salu_insts_per_wave"),
                        ("SQ_INSTS_VMEM_RD", "vmem_rd_insts_per_wave")):
            if waves and c in m:
                row[name] = m[c] / waves
        if "SQ_WAIT_INST_ANY" in m and "SQ_WAVE_CYCLES" in m and m["SQ_WAVE_CYCLES"] > 0:
            row["wave_wait_inst_frac"] = m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_ACTIVE_INST_LDS" in m and m["SQ_ACTIVE_INST_LDS"] > 0:
            row["lds_bank_conflict_per_lds_inst"] = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_ACTIVE_INST_LDS"]
        row["raw_median"] = {c: x for c, x in m.items() if not c.startswith("_")}
        res["kernels"][k] = row
    old = json.load(open(counters_json)) if os.path.exists(counters_json) else {}
    old[workload] = res
    open(counters_json, "w").write(json.dumps(old, indent=1) + "\n")
    f = lambda x, p=1: "-" if x is None else (f"{100 * x:.{p}f}%")
    lines = ["# rocprofv3 counter summary: " + workload, "",
             f"Command: `{command}`", "",
             "Fractions are of the SIMD cycles of each dispatch (1024 SIMDs x GRBM_GUI_ACTIVE / 8 cycles); "
             "median over dispatches.  Kernel sources hash: " + res["kernel_hash"] + ".", "",
             "| kernel | cycles | clock (GHz) | MFMA busy | VALU busy | MFMA+VALU co-exec | MFMA cycles/inst | "
             "VALU inst/wave | MFMA inst/wave | LDS inst/wave | wait-inst share | LDS conflicts/LDS inst |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k, r in res["kernels"].items():
        g = lambda n, fmt="{:.1f}": "-" if r.get(n) is None else fmt.format(r[n])
        lines.append(f"| {k} | {r['cycles']:.3g} | {g('clock_ghz', '{:.2f}')} | {f(r.get('mfma_busy'))} | "
                     f"{f(r.get('valu_busy'))} | {f(r.get('mfma_valu_coexec'))} | {g('mfma_cycles_per_inst')} | "
                     f"{g('valu_insts_per_wave', '{:.0f}')} | {g('mfma_insts_per_wave', '{:.0f}')} | "
                     f"{g('lds_insts_per_wave', '{:.0f}')} | {f(r.get('wave_wait_inst_frac'))} | "
                     f"{g('lds_bank_conflict_per_lds_inst', '{:.2f}')} |")
    txt = "\n".join(lines) + "\n"
    if out:
        open(out, "w").write(txt)
    print(txt)


def summarize_pmc(fetch_dir, write_dir, workload, copy_bytes, command, out):
    """Per-launch HBM bytes of every kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the plain copy of copy_bytes bytes."""
    import csv
    import glob

    def load(d, counter):
        f = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        vals = {}
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(_short_kernel_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_k = [k for k in fetch if k.startswith("copy:")]
    if not copy_k:
        raise SystemExit("no copy kernel in the counter runs (run bench.py with --copy-bytes)")
    ck = max(copy_k, key=lambda k: max(fetch[k]))
    # the copy reads copy_bytes and writes copy_bytes
    f_scale = copy_bytes / (max(fetch[ck]) * 1024.0)
    w_scale = copy_bytes / (max(write[ck]) * 1024.0)
    res = {"workload": workload, "copy_bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
           "kernel_hash": kernel_hash(_hash_files(workload)), "command": command, "kernels": {}}
    for k in fetch:
        if k.startswith("copy:"):
            continue
        fb = sorted(fetch[k])[len(fetch[k]) // 2] * 1024.0 * f_scale
        wb = sorted(write.get(k, [0.0]))[len(write.get(k, [0.0])) // 2] * 1024.0 * w_scale
        res["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    txt = json.dumps(res, indent=1)
    if out:
        old = {}
        if os.path.exists(out):
            old = json.load(open(out))
        old[workload] = res
        open(out, "w").write(json.dumps(old, indent=1) + "\n")
    print(txt)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command, args.out)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.command, args.out, args.counters)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.copy_bytes,
                      args.command, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described in DESIGN.md but not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import triangular_attention_amd as ta

    ta.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in synth.BLOCK_WORKLOADS:
        bench_block(args, synth.BLOCK_WORKLOADS[args.workload], dev)
        return
    if args.workload in synth.TRIMUL_WORKLOADS:
        bench_trimul(args, synth.TRIMUL_WORKLOADS[args.workload], dev)
        return
    if args.sweep:
        sweep(args, dev)
        return
    out = bench_attn(args, synth.get(args.workload), dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth.get(args.workload), args.cpu_seconds)
    print(json.dumps(out))


# the three configured workloads (n384_d32 is also the sweep's 384 x 32 shape) and the rest of the
# pages' six timing shapes
SWEEP_WORKLOADS = ("n384_d32", "n640_d16", "n768_d32_mask", "sweep_n384_d16", "sweep_n640_d16", "sweep_n640_d32",
                   "sweep_n768_d16", "sweep_n768_d32")


def sweep(args, dev):
    """The pages' six timing shapes (crops 384/640/768 x D 16/32) and the three configured workloads:
    one bench line each (ms, TFLOP/s, the dominant kernel's roofline fraction) with the FP64
    oracle timed on a short sample of the same workload beside it, then a markdown table."""
    import synth
    rows = []
    for name in SWEEP_WORKLOADS:
        w = synth.get(name)
        out = bench_attn(args, w, dev)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        print(json.dumps(out), flush=True)
        rows.append(out)
    print("| workload | ms / fwd+bwd | TFLOP/s | % bf16 peak | fwd ms | bwd ms (delta + main + reductions) | "
          "dominant kernel | its bound | its roofline fraction | oracle TFLOP/s (cores) | GPU / oracle |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        k = r["kernels"]
        bwd = sum(v["ms"] for n, v in k.items() if n != "fwd")
        cb = r.get("cpu_baseline")
        ro = r["roofline"]
        kname = ro["kernel"].split(" (")[0] + (" (2 kernels)" if "two kernels" in ro["kernel"] else "")
        print(f"| {r['config']['workload']} | {r['ms_per_step']:.3f} | {r['value']:.0f} | {r['pct_bf16_peak']:.1f} | "
              f"{k['fwd']['ms']:.3f} | {bwd:.3f} | {kname} | {ro['bound']} | {ro['frac']:.3f} | "
              + (f"{cb['value']:.3f} ({cb['cores']}) | {r['value'] / cb['value']:.0f}x |" if cb else "- | - |"))


def bench_attn(args, w, dev):
    """One bench line (dict) for an attention workload: the five calls (or the chunked
    backward) timed on resident inputs, per-kernel times and the dominant kernel's roofline."""
    import torch

    import synth
    import triangular_attention_amd as ta
    x = synth.make_inputs(w, args.seed)
    q, k, v, do, bias = (x[n].to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do", "bias"))
    mask = None if x["mask"] is None else x["mask"].to(dev)
    d = ta.dims_of(q, w.scale)
    bp = args.partials == "bf16"
    ws = ta.workspace(d, single_pass=bp)
    # the default FP32 backward call runs two kernels (dK/dV, then dQ/dbias) for D = 32 and
    # for D = 16 past N = 640
    two = (w.D == 32 or (w.D == 16 and w.N > 640)) and not bp
    comp = not args.no_compensate
    o = torch.empty_like(q)
    o_res = torch.empty_like(q) if comp else None
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dk, dv, dq = torch.empty_like(k), torch.empty_like(v), torch.empty_like(q)
    dbias = torch.empty_like(bias)
    pdt = torch.bfloat16 if bp else torch.float32
    dqp = torch.empty(ws["dq_partial_elems"], dtype=pdt, device=dev)
    dbp = torch.empty(ws["dbias_partial_elems"], dtype=pdt, device=dev)
    stream = torch.cuda.current_stream()

    calls = {
        "fwd": lambda: ta.tri_attn_fwd(d, q, k, v, bias, mask, o, o_res, lse, stream),
        "delta": lambda: ta.tri_attn_bwd_delta(d, o, o_res, do, delta, stream),
        "bwd": lambda: ta.tri_attn_bwd(d, q, k, v, bias, mask, do, lse, delta, dk, dv, dqp, dbp, stream,
                                       bf16_partials=bp),
        "reduce_dq": lambda: ta.tri_attn_reduce_dq(d, dqp, dq, stream, bf16_partials=bp),
        "reduce_dbias": lambda: ta.tri_attn_reduce_dbias(d, dbp, dbias, stream, bf16_partials=bp),
    }

    names = KERNELS
    if args.chunk_groups > 0:
        if bp:
            raise SystemExit("--chunk-groups runs FP32 partials only")
        del dqp, dbp
        cw = ta.chunked_workspace(d, args.chunk_groups)
        cbuf = torch.empty(cw["bytes"], dtype=torch.uint8, device=dev)
        calls["bwd_chunked"] = lambda: ta.tri_attn_bwd_chunked(d, q, k, v, bias, mask, do, lse, delta, dq, dk, dv,
                                                              dbias, cbuf, stream)
        names = ("fwd", "delta", "bwd_chunked")

    def step():
        for n in names:
            calls[n]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps

    # per-kernel durations: events on the launch stream around each kernel, K more steps
    per = {n: 0.0 for n in names}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for s in range(args.steps):
        evs[s][0].record(stream)
        for i, n in enumerate(names):
            calls[n]()
            evs[s][i + 1].record(stream)
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, n in enumerate(names):
            per[n] += evs[s][i].elapsed_time(evs[s][i + 1]) / args.steps

    alg = algorithmic(w, ws["j_k"], ws["l"], 2 if bp else 4, two_kernel=two)
    # the chunked call does the work of the main backward and both reductions
    alg["bwd_chunked"] = {k: alg["bwd"][k] + alg["reduce_dq"][k] + alg["reduce_dbias"][k] for k in ("flops", "bytes")}
    kernels = {}
    for n in names:
        ms = per[n]
        kernels[n] = {"ms": round(ms, 5),
                      "tflops": round(alg[n]["flops"] / (ms * 1e-3) / 1e12, 2) if ms > 0 else None,
                      "alg_gbs": round(alg[n]["bytes"] / (ms * 1e-3) / 1e9, 1) if ms > 0 else None}
    dom = max(names, key=lambda n: per[n])
    # kernels of the dominant call (the two-kernel backward call launches both)
    prefixes = (dom + "_kernel",) + (("bwdq_kernel",) if dom == "bwd" and two else ())
    traffic = None
    traffic_all = None
    if os.path.exists(args.traffic):
        try:
            tr = json.load(open(args.traffic)).get(w.name, {})
            if tr.get("kernel_hash") == kernel_hash():
                traffic_all = tr["kernels"]
                hits = [v["bytes_per_launch"] for kname, v in traffic_all.items() if kname.startswith(prefixes)]
                if len(hits) == len(prefixes):
                    traffic = round(sum(hits))
        except Exception:
            traffic = None
    # roofline of the dominant kernel: the bound is the resource whose peak gives the longer
    # minimum time for the kernel's algorithmic flops and bytes (arithmetic intensity against
    # the machine balance); the other fraction is reported beside it
    t_mfma = alg[dom]["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = alg[dom]["bytes"] / (PEAK_HBM_GBS * 1e9)
    ach_f = alg[dom]["flops"] / (per[dom] * 1e-3) / 1e12
    ach_b = alg[dom]["bytes"] / (per[dom] * 1e-3) / 1e9
    common = {"kernel": dom + (" (two kernels: dK/dV key-tile, dQ/dbias query-tile)" if dom == "bwd" and two else ""),
              "traffic": traffic, "avg_launch_ms": round(per[dom], 5),
              "intensity_flop_per_byte": round(alg[dom]["flops"] / alg[dom]["bytes"], 1),
              "mfma_frac": round(ach_f / PEAK_BF16_TFLOPS, 4), "hbm_frac": round(ach_b / PEAK_HBM_GBS, 4)}
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": round(ach_f, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach_f / PEAK_BF16_TFLOPS, 4), **common}
    else:
        roof = {"bound": "hbm", "achieved": round(ach_b, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach_b / PEAK_HBM_GBS, 4), **common}

    # measured utilisation of the dominant kernel (rocprofv3 counters taken on these sources)
    cnt = [c for c in (_counters_lookup(args.counters, w.name, p) for p in prefixes) if c is not None]
    if cnt:
        roof["counters"] = cnt[0] if len(cnt) == 1 else cnt
    value = w.flops_fwd_bwd / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "tri-attn fwd+bwd TFLOP/s & ms at N=768,H=4,D=32 bf16; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N_o": w.N_o, "N": w.N, "H": w.H, "D": w.D,
                   "scale": w.scale, "bias_std": w.bias_std, "mask_p": w.mask_p,
                   "compensate": comp, "partials": args.partials, "flops_per_step": w.flops_fwd_bwd,
                   **({"chunk_groups": cw["groups_per_chunk"], "chunk_workspace_bytes": cw["bytes"]}
                      if args.chunk_groups > 0 else {}),
                   "key_tile": ws["key_tile"], "outer_group": ws["outer_group"],
                   "description": w.description},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernels": kernels,
        "roofline": roof,
        "wall_s_timed": round(t_wall, 4),
        "gpu": torch.cuda.get_device_name(0),
    }
    if traffic_all is not None:
        out["traffic_bytes_per_launch"] = {k: round(v["bytes_per_launch"]) for k, v in traffic_all.items()}
    _copy_calibration(args, dev, out)
    return out


BLOCK_KERNELS = ("ln_proj", "fwd", "gate_out", "gate_out_bwd", "delta", "bwd", "reduce_dbias", "reduce_dq",
                 "proj_dz", "proj_dw", "reduce_wgrad")


def algorithmic_block(bw, ws_attn, ws_blk):
    """Algorithmic flops and minimum HBM bytes of one launch of each kernel of the block step."""
    import synth
    P, C, H = bw.pairs, bw.C_z, bw.H
    F = bw.H * bw.D
    wa = synth.Workload("attn", bw.B, bw.N, bw.N, bw.H, bw.D, 1.0 / (bw.D ** 0.5))
    alg = algorithmic(wa, ws_attn["j_k"], ws_attn["l"])
    Xb = 2 * P * F            # bytes of one [B,N,H,N,D] bf16 tensor
    Zb = 2 * P * C            # bytes of Z / Y / dZ / dY
    Yb = 2 * P * H            # bytes of bias / dbias
    Wb = 2 * (4 * F + H) * C  # projection weights
    nw, no, nl = ws_blk["n_w"], ws_blk["n_out"], ws_blk["n_ln"]
    alg.update({
        "ln_proj": {"flops": 2.0 * P * C * (4 * F + H), "bytes": Zb + 4 * Xb + Yb + 8 * P + Wb + 8 * C},
        "gate_out": {"flops": 2.0 * P * F * C, "bytes": 2 * Xb + Zb + 2 * C * F},
        "gate_out_bwd": {"flops": 4.0 * P * F * C, "bytes": Zb + 4 * Xb + 2 * C * F + 4 * no * C * F},
        "proj_dz": {"flops": 2.0 * P * C * (4 * F + H), "bytes": 2 * Zb + 4 * Xb + Yb + 8 * P + Wb + 4 * nl * 2 * C},
        "proj_dw": {"flops": 2.0 * P * C * (4 * F + H), "bytes": Zb + 4 * Xb + Yb + 8 * P + 4 * nw * (4 * F + H) * C},
        "reduce_wgrad": {"flops": float(nw * (4 * F + H) * C + no * C * F + nl * 2 * C),
                         "bytes": 4 * (nw * (4 * F + H) * C + no * C * F + nl * 2 * C)
                                  + 4 * ((4 * F + H) * C + C * F + 2 * C)},
    })
    return alg


def _roofline(alg, per, dom, traffic):
    t_mfma = alg[dom]["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = alg[dom]["bytes"] / (PEAK_HBM_GBS * 1e9)
    ach_f = alg[dom]["flops"] / (per[dom] * 1e-3) / 1e12
    ach_b = alg[dom]["bytes"] / (per[dom] * 1e-3) / 1e9
    common = {"kernel": dom, "traffic": traffic, "avg_launch_ms": round(per[dom], 5),
              "intensity_flop_per_byte": round(alg[dom]["flops"] / alg[dom]["bytes"], 1),
              "mfma_frac": round(ach_f / PEAK_BF16_TFLOPS, 4), "hbm_frac": round(ach_b / PEAK_HBM_GBS, 4)}
    if t_mfma >= t_hbm:
        return {"bound": "mfma", "achieved": round(ach_f, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach_f / PEAK_BF16_TFLOPS, 4), **common}
    return {"bound": "hbm", "achieved": round(ach_b, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach_b / PEAK_HBM_GBS, 4), **common}


# kernel-name prefix of each call of the triangle-multiplication step (for measured traffic)
TRIMUL_LAUNCH_KERNELS = {"in_fwd": "tm_in_fwd_kernel", "contract": "tm_gemm_kernel<false, false",
                         "out_fwd": "tm_out_fwd_kernel", "out_bwd": "tm_out_bwd_kernel",
                         "in_bwd": "tm_in_bwd_kernel", "in_dz": "tm_in_dz_kernel", "in_dw": "tm_in_dw_kernel"}


def _traffic_lookup(path, workload, dom, prefix):
    """Measured bytes per launch of the dominant call's kernel from the counter summary, if it was
    taken on the current sources."""
    if not os.path.exists(path):
        return None, None
    try:
        tr = json.load(open(path)).get(workload, {})
        if tr.get("kernel_hash") != kernel_hash(_hash_files(workload)):
            return None, None
        allk = tr["kernels"]
        for kname, val in allk.items():
            if kname.startswith(prefix):
                return round(val["bytes_per_launch"]), allk
        return None, allk
    except Exception:
        return None, None


def _counters_lookup(path, workload, prefix):
    """MFMA / VALU busy fractions of a kernel from the counter summary, if it was taken on the
    current sources."""
    if not os.path.exists(path):
        return None
    try:
        c = json.load(open(path)).get(workload, {})
        if c.get("kernel_hash") != kernel_hash(_hash_files(workload)):
            return None
        for k, v in c["kernels"].items():
            if k.startswith(prefix):
                return {"kernel": k, **{n: round(v[n], 4) for n in ("mfma_busy", "valu_busy", "mfma_valu_coexec",
                                                                     "clock_ghz") if v.get(n) is not None}}
    except Exception:
        return None
    return None


def _copy_calibration(args, dev, out):
    """A plain device copy of --copy-bytes (3 times): the reference for the byte counters."""
    import torch
    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_bytes


def _time_steps(calls, names, steps, warmup, stream):
    """Whole-step time (HIP events around K steps) and per-kernel averages (events around each
    launch, K more steps), all on the launch stream."""
    import torch

    def step():
        for n in names:
            calls[n]()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = ev0.elapsed_time(ev1) / steps
    per = {n: 0.0 for n in names}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for s_ in range(steps):
        evs[s_][0].record(stream)
        for i, n in enumerate(names):
            calls[n]()
            evs[s_][i + 1].record(stream)
    torch.cuda.synchronize()
    for s_ in range(steps):
        for i, n in enumerate(names):
            per[n] += evs[s_][i].elapsed_time(evs[s_][i + 1]) / steps
    return ms_step, per, t_wall


def cpu_baseline_block(bw, seconds):
    """The FP64 block oracle (as it stands) on a smaller crop of the same block (same C_z, H, D,
    weights and distributions), sized to take about ``seconds``; rate in the metric's unit."""
    import synth
    from oracle import block_fp64 as blk
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))

    def run(n):
        w = synth.BlockWorkload("cpu", bw.B, n, bw.H, bw.D, ending=bw.ending, w_std=bw.w_std)
        x = synth.make_block_inputs(w, 0)
        a = [x[k].double().numpy() for k in ("z", "gamma", "beta", "w_qkvg", "w_b", "w_o")]
        t0 = time.perf_counter()
        blk.block_backward(*a, x["dy"].double().numpy(), bw.H, bw.D, ending=bw.ending)
        return time.perf_counter() - t0, w.flops_fwd_bwd

    n = 48
    t, fl = run(n)
    while t < seconds / 3 and n < bw.N:
        n = min(bw.N, int(n * 1.5))
        t, fl = run(n)
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole block fwd+bwd (FP64 numpy oracle, forward inside backward) at crop N={n} "
                      f"(B={bw.B}, C_z=128, H={bw.H}, D={bw.D}, {'ending' if bw.ending else 'starting'} node), "
                      f"seed 0; {t:.1f} s", "seconds": t, "crop": n}


def bench_block(args, bw, dev):
    """One step = the whole triangle-attention block, forward and backward (11 launches)."""
    import torch

    import synth
    import triangular_attention_amd as ta
    from triangular_attention_amd import block as tb

    x = synth.make_block_inputs(bw, args.seed)
    z, dy, w_qkvg, w_b, w_o = (x[n].to(torch.bfloat16).to(dev) for n in ("z", "dy", "w_qkvg", "w_b", "w_o"))
    gamma, beta = x["gamma"].float().to(dev), x["beta"].float().to(dev)
    B, N, H, D = bw.B, bw.N, bw.H, bw.D
    F, C = H * D, bw.C_z
    bd = tb.block_dims(B, N, H, D, bw.ending)
    wsb = tb.block_workspace(bd)
    hs = (B, N, H, N, D)
    e = lambda shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
    q, k, v, g, o, o_res, d_o, d_g, dq, dk, dv = (e(hs) for _ in range(11))
    bias, dbias = e((B, H, N, N)), e((B, H, N, N))
    stats = e((B, N, N, 2), torch.float32)
    lse, delta = e((B, N, H, N), torch.float32), e((B, N, H, N), torch.float32)
    y, dz = torch.empty_like(z), torch.empty_like(z)
    ad = ta.dims_of(q, 1.0 / D ** 0.5)
    wsa = ta.workspace(ad)
    dqp, dbp = e(wsa["dq_partial_elems"], torch.float32), e(wsa["dbias_partial_elems"], torch.float32)
    wo_part = e(wsb["n_out"] * C * F, torch.float32)
    ln_part = e(wsb["n_ln"] * 2 * C, torch.float32)
    w_part = e(wsb["n_w"] * (4 * F + H) * C, torch.float32)
    dw_qkvg, dw_b, dw_o = e((4 * F, C), torch.float32), e((H, C), torch.float32), e((C, F), torch.float32)
    dgamma, dbeta = e(C, torch.float32), e(C, torch.float32)
    st = torch.cuda.current_stream()
    calls = {
        "ln_proj": lambda: tb.tri_block_ln_proj(bd, z, gamma, beta, w_qkvg, w_b, q, k, v, g, bias, stats, st),
        "fwd": lambda: ta.tri_attn_fwd(ad, q, k, v, bias, None, o, o_res, lse, st),
        "gate_out": lambda: tb.tri_block_gate_out(bd, o, g, w_o, y, st),
        "gate_out_bwd": lambda: tb.tri_block_gate_out_bwd(bd, dy, o, g, w_o, d_o, d_g, wo_part, st),
        "delta": lambda: ta.tri_attn_bwd_delta(ad, o, o_res, d_o, delta, st),
        "bwd": lambda: ta.tri_attn_bwd(ad, q, k, v, bias, None, d_o, lse, delta, dk, dv, dqp, dbp, st),
        "reduce_dbias": lambda: ta.tri_attn_reduce_dbias(ad, dbp, dbias, st),
        "reduce_dq": lambda: ta.tri_attn_reduce_dq(ad, dqp, dq, st),
        "proj_dz": lambda: tb.tri_block_proj_bwd_dz(bd, z, stats, gamma, w_qkvg, w_b, dq, dk, dv, d_g, dbias,
                                                    dz, ln_part, st),
        "proj_dw": lambda: tb.tri_block_proj_bwd_dw(bd, z, stats, gamma, beta, dq, dk, dv, d_g, dbias, w_part, st),
        "reduce_wgrad": lambda: tb.tri_block_reduce_wgrad(bd, w_part, wo_part, ln_part, dw_qkvg, dw_b, dw_o,
                                                          dgamma, dbeta, st),
    }
    ms_step, per, t_wall = _time_steps(calls, BLOCK_KERNELS, args.steps, args.warmup, st)
    alg = algorithmic_block(bw, wsa, wsb)
    kernels = {n: {"ms": round(per[n], 5),
                   "tflops": round(alg[n]["flops"] / (per[n] * 1e-3) / 1e12, 2),
                   "alg_gbs": round(alg[n]["bytes"] / (per[n] * 1e-3) / 1e9, 1)} for n in BLOCK_KERNELS}
    dom = max(BLOCK_KERNELS, key=lambda n: per[n])
    traffic, traffic_all = None, None
    if os.path.exists(args.traffic):
        try:
            tr = json.load(open(args.traffic)).get(bw.name, {})
            if tr.get("kernel_hash") == kernel_hash(_hash_files(bw.name)):
                traffic_all = tr["kernels"]
                for kname, val in traffic_all.items():
                    if kname.startswith(dom + "_kernel"):
                        traffic = round(val["bytes_per_launch"])
        except Exception:
            traffic = None
    value = bw.flops_fwd_bwd / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "tri-attn fwd+bwd TFLOP/s & ms at N=768,H=4,D=32 bf16; % bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": bw.name, "B": B, "N": N, "C_z": C, "H": H, "D": D, "ending": bw.ending,
                   "w_std": bw.w_std, "flops_per_step": bw.flops_fwd_bwd,
                   "attention_flops": 14.0 * B * N * H * N * N * D, "description": bw.description},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernels": kernels,
        "roofline": _roofline(alg, per, dom, traffic),
        "wall_s_timed": round(t_wall, 4),
        "gpu": torch.cuda.get_device_name(0),
    }
    if traffic_all is not None:
        out["traffic_bytes_per_launch"] = {kk: round(vv["bytes_per_launch"]) for kk, vv in traffic_all.items()}
    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = args.copy_bytes
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(bw, args.cpu_seconds)
    print(json.dumps(out))


TRIMUL_KERNELS = ("in_fwd", "contract", "out_fwd", "out_bwd", "contract_bwd", "in_bwd", "in_dz", "in_dw",
                  "reduce_wgrad")


def algorithmic_trimul(tw, ws):
    """Algorithmic flops and minimum HBM bytes of one launch of each call of the update step."""
    P, C, c, B, N = tw.pairs, tw.C_z, tw.c, tw.B, tw.N
    Zb, Cb = 2 * P * C, 2 * P * c          # one pair-major [.., 128] / channel-major [B, c, N, N] bf16 tensor
    Wb = 2 * (4 * c + C) * C
    gemm = 2.0 * B * c * N ** 3
    nw, no, nl, nlo = ws["n_w"], ws["n_out"], ws["n_ln"], ws["n_lno"]
    return {
        "in_fwd": {"flops": 2.0 * P * C * (4 * c + C), "bytes": Zb + 2 * Cb + Zb + 8 * P + Wb},
        "contract": {"flops": gemm, "bytes": 3 * Cb},
        "out_fwd": {"flops": 2.0 * P * c * C, "bytes": Cb + 2 * Zb + 8 * P + 2 * C * c},
        "out_bwd": {"flops": 6.0 * P * c * C, "bytes": 2 * Zb + Cb + 8 * P + Cb + Zb + 4 * (no * C * c + nlo * 2 * c)},
        "contract_bwd": {"flops": 2 * gemm, "bytes": 5 * Cb},
        "in_bwd": {"flops": 2.0 * P * C * 4 * c, "bytes": Zb + 8 * P + 2 * Cb + 2 * P * 4 * c + Wb},
        "in_dz": {"flops": 2.0 * P * (4 * c + C) * C, "bytes": 2 * P * 4 * c + Zb + Zb + 8 * P + Zb + Wb},
        "in_dw": {"flops": 2.0 * P * (4 * c + C) * C, "bytes": 2 * P * 4 * c + Zb + Zb + 8 * P + 4 * nw * (4 * c + C) * C},
        "reduce_wgrad": {"flops": float(nw * (4 * c + C) * C + no * C * c + nl * 2 * C + nlo * 2 * c),
                         "bytes": 4 * (nw * (4 * c + C) * C + no * C * c + nl * 2 * C + nlo * 2 * c)},
    }


def cpu_baseline_trimul(tw, seconds):
    """The FP64 oracle (as it stands) on a smaller crop of the same update, sized to take about
    ``seconds``; rate in the metric's unit."""
    import synth
    from oracle import trimul_fp64 as tmo
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))

    def run(n):
        w = synth.TrimulWorkload("cpu", tw.B, n, tw.c, incoming=tw.incoming, w_std=tw.w_std)
        x = synth.make_trimul_inputs(w, 0)
        a = [x[k].double().numpy() for k in ("z", "gamma", "beta", "w_in", "gamma_o", "beta_o", "w_o")]
        t0 = time.perf_counter()
        tmo.trimul_backward(*a, x["dout"].double().numpy(), tw.c, incoming=tw.incoming)
        return time.perf_counter() - t0, w.flops_fwd_bwd

    n = 64
    t, fl = run(n)
    while t < seconds / 3 and n < tw.N:
        n = min(tw.N, int(n * 1.5) // 8 * 8)
        t, fl = run(n)
    return {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole update fwd+bwd (FP64 numpy oracle, forward inside backward) at crop N={n} "
                      f"(B={tw.B}, C_z=128, c={tw.c}, {'incoming' if tw.incoming else 'outgoing'}), seed 0; "
                      f"{t:.1f} s", "seconds": t, "crop": n}


def bench_trimul(args, tw, dev):
    """One step = the triangle multiplicative update, forward and backward (9 calls, 10 launches
    plus the reductions)."""
    import torch

    import synth
    from triangular_attention_amd import trimul as tmb

    x = synth.make_trimul_inputs(tw, args.seed)
    z, dout, w_in, w_o = (x[n].to(torch.bfloat16).to(dev) for n in ("z", "dout", "w_in", "w_o"))
    gamma, beta, gamma_o, beta_o = (x[n].float().to(dev) for n in ("gamma", "beta", "gamma_o", "beta_o"))
    B, N, c, C = tw.B, tw.N, tw.c, tw.C_z
    d = tmb.mul_dims(B, N, c, tw.incoming)
    ws = tmb.mul_workspace(d)
    e = lambda shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=dev)
    cs = (B, c, N, N)
    a, b, xx, dx, da, db = (e(cs) for _ in range(6))
    g, out, dg, dz = (torch.empty_like(z) for _ in range(4))
    stats, stats_o = e((B * N * N, 2), torch.float32), e((B * N * N, 2), torch.float32)
    dproj = e((B * N * N, 4 * c))
    wo_part, lno_part = e(ws["n_out"] * C * c, torch.float32), e(ws["n_lno"] * 2 * c, torch.float32)
    ln_part, w_part = e(ws["n_ln"] * 2 * C, torch.float32), e(ws["n_w"] * (4 * c + C) * C, torch.float32)
    dw_in, dw_o = e((4 * c + C, C), torch.float32), e((C, c), torch.float32)
    dgm, dbt, dgo, dbo = e(C, torch.float32), e(C, torch.float32), e(c, torch.float32), e(c, torch.float32)
    st = torch.cuda.current_stream()
    calls = {
        "in_fwd": lambda: tmb.tri_mul_in_fwd(d, z, gamma, beta, w_in, a, b, g, stats, st),
        "contract": lambda: tmb.tri_mul_contract(d, a, b, xx, st),
        "out_fwd": lambda: tmb.tri_mul_out_fwd(d, xx, g, gamma_o, beta_o, w_o, out, stats_o, st),
        "out_bwd": lambda: tmb.tri_mul_out_bwd(d, dout, xx, g, stats_o, gamma_o, beta_o, w_o, dx, dg, wo_part,
                                               lno_part, st),
        "contract_bwd": lambda: tmb.tri_mul_contract_bwd(d, dx, a, b, da, db, st),
        "in_bwd": lambda: tmb.tri_mul_in_bwd(d, z, stats, gamma, beta, w_in, da, db, dproj, st),
        "in_dz": lambda: tmb.tri_mul_in_bwd_dz(d, z, stats, gamma, w_in, dproj, dg, dz, ln_part, st),
        "in_dw": lambda: tmb.tri_mul_in_bwd_dw(d, z, stats, gamma, beta, dproj, dg, w_part, st),
        "reduce_wgrad": lambda: tmb.tri_mul_reduce_wgrad(d, w_part, wo_part, ln_part, lno_part, dw_in, dw_o, dgm,
                                                         dbt, dgo, dbo, st),
    }
    ms_step, per, t_wall = _time_steps(calls, TRIMUL_KERNELS, args.steps, args.warmup, st)
    alg = algorithmic_trimul(tw, ws)
    kernels = {n: {"ms": round(per[n], 5),
                   "tflops": round(alg[n]["flops"] / (per[n] * 1e-3) / 1e12, 2),
                   "alg_gbs": round(alg[n]["bytes"] / (per[n] * 1e-3) / 1e9, 1)} for n in TRIMUL_KERNELS}
    dom = max(TRIMUL_KERNELS, key=lambda n: per[n])
    traffic, traffic_all = _traffic_lookup(args.traffic, tw.name, dom, TRIMUL_LAUNCH_KERNELS.get(dom, dom))
    value = tw.flops_fwd_bwd / (ms_step * 1e-3) / 1e12
    res = {
        "metric": "tri-attn fwd+bwd TFLOP/s & ms at N=768,H=4,D=32 bf16; % bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": tw.name, "B": B, "N": N, "C_z": C, "c": c, "incoming": tw.incoming,
                   "w_std": tw.w_std, "flops_per_step": tw.flops_fwd_bwd, "description": tw.description},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "kernels": kernels,
        "roofline": _roofline(alg, per, dom, traffic),
        "wall_s_timed": round(t_wall, 4),
        "gpu": torch.cuda.get_device_name(0),
    }
    if traffic_all is not None:
        res["traffic_bytes_per_launch"] = {kk: round(vv["bytes_per_launch"]) for kk, vv in traffic_all.items()}
    _copy_calibration(args, dev, res)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_trimul(tw, args.cpu_seconds)
    print(json.dumps(res))


def _hash_files(workload):
    """The sources of the kernels a workload runs: the block runs the attention kernels too;
    the triangle update's weight-gradient reductions are the block's reduce kernel."""
    if workload.startswith("block"):
        return ATTN_SOURCES + BLOCK_SOURCES
    if workload.startswith("trimul"):
        return TRIMUL_SOURCES
    return ATTN_SOURCES


ATTN_SOURCES = ("common.h", "kernels.h", "bwd_layout.h", "api.hip", "fwd.hip", "bwd.hip", "bwd_q.hip",
                "delta_reduce.hip")
BLOCK_SOURCES = ("block_kernels.h", "block_api.hip", "block.hip", "pair_common.h")
TRIMUL_SOURCES = ("common.h", "pair_common.h", "trimul_kernels.h", "trimul_api.hip", "trimul.hip",
                  "block_kernels.h", "block.hip")


def kernel_hash(files=ATTN_SOURCES):
    """Hash of the kernel sources without comments and whitespace: stored traffic counters
    are valid only for the same code (a comment edit keeps them).  ``files`` = the sources of
    the measured kernels (None: every source)."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "triangular_attention_amd", "csrc")
    for f in sorted(os.listdir(csrc)) if files is None else sorted(files):
        txt = open(os.path.join(csrc, f), encoding="utf-8").read()
        txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", " ", txt)
        h.update(f.encode() + b"\0" + " ".join(txt.split()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
