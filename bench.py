#!/usr/bin/env python3
"""Decode-step benchmark of one MoE FFN layer on one MI355X.

Default workload: the Qwen3-30B-A3B-shaped layer (d=2048, 128 experts,
I=768, top-8 softmax, bf16 weights and activations, fp32 accumulation) at
decode batches 1, 4 and 16; the headline value is the layer latency at
batch 16.  Inputs are seeded synthetic tensors already resident in HBM.  The
weights are replicated R times at distinct addresses and consecutive steps
walk the replicas (like consecutive layers of a model), so that the weights a
step streams (R x active bytes >= 1 GiB) cannot be served from the 256 MB
Infinity Cache.

Prints ONE JSON line (the driver contract) on stdout; --sweep also writes a
line per (layer shape, batch) to --sweep-out.
"""
from __future__ import annotations

import argparse
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode latency (us) + achieved HBM GB/s vs peak at batch 1/4/16"
HBM_PEAK_GBS = 8000.0
HEADLINE = "qwen3_30b_a3b_d2048_e128_i768_top8"
HEADLINE_T = 16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--batches", type=str, default="1,2,4,8,16,32")
    p.add_argument("--shape", type=str, default=HEADLINE)
    p.add_argument("--sweep", action="store_true", help="also time every other layer shape")
    p.add_argument("--sweep-out", type=str, default="gpurun_out/sweep.jsonl")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-steps", type=int, default=3,
                   help="oracle steps per thread setting of the CPU baseline (median)")
    p.add_argument("--no-dept", action="store_true",
                   help="skip the department-layer comparisons (DeaMoE-7B-shaped against its "
                        "expanded vanilla form; the department transform against the "
                        "DeepSeek-V3-shaped layer)")
    p.add_argument("--dept-steps", type=int, default=60)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--profile-pass", action="store_true",
                   help="headline batch only, 20 eager steps + a 1 GiB calibration copy "
                        "(for rocprofv3 --pmc runs)")
    p.add_argument("--summarize-trace", type=str, default=None,
                   help="print per-kernel, per-grid-size mean durations of a rocprofv3 "
                        "kernel_trace.csv and exit")
    p.add_argument("--summarize-pmc", type=str, default=None,
                   help="print per-kernel, per-grid-size mean counter values of a rocprofv3 "
                        "counter_collection.csv and exit")
    p.add_argument("--profile-meta", type=str, default="gpurun_out/profile_pass.json",
                   help="--profile-pass writes the algorithmic bytes and source hash here; "
                        "--pmc-report reads them")
    p.add_argument("--pmc-report", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                   help="write the calibrated HBM traffic summary of two --pmc runs "
                        "(FETCH_SIZE, WRITE_SIZE) of --profile-pass as markdown")
    p.add_argument("--trace-report", nargs=2, metavar=("TRACE_CSV", "BENCH_JSON"), default=None,
                   help="write the kernel-trace summary of a profiled default run, beside the "
                        "JSON line of an unprofiled one, as markdown")
    p.add_argument("--sweep-report", type=str, default=None, metavar="SWEEP_JSONL",
                   help="write the --sweep lines as a markdown summary")
    p.add_argument("--source-hash", action="store_true",
                   help="print the hash of the kernel sources the counter summary refers to")
    return p.parse_args()


def _short(name):
    import re
    m = re.search(r"moe::(\w+)", name)
    if m:
        return m.group(1)
    if "at::native" in name:
        return "torch"
    return name[:48]


def trace_means(path):
    """Kernel durations (us) of a rocprofv3 kernel trace, per kernel and grid
    size (the grid size tells the decode batches apart)."""
    import csv
    from collections import defaultdict
    acc = defaultdict(list)
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]))
        acc[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return acc


def summarize_trace(path):
    acc = trace_means(path)
    print("| kernel | grid x | grid y | calls | mean us | min us |")
    print("|---|---|---|---|---|---|")
    for (k, gx, gy), v in sorted(acc.items()):
        if k == "torch":
            continue
        print(f"| {k} | {gx} | {gy} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} |")


def shape_tag(name):
    """Short name of a layer shape for output paths: the part before its sizes."""
    return re.split(r"_d[0-9]", name)[0]


def trace_report(trace_csv, bench_json):
    """Markdown summary: the kernel trace of a profiled default run, the
    unprofiled run's per-batch stage times, and the roofline kernel's
    event-timed launch beside its trace mean."""
    b = json.loads(open(bench_json).read().strip().splitlines()[-1])
    acc = trace_means(trace_csv)
    head_T = b["config"]["batch"]
    shape = b["config"]["workload"].split(" MoE")[0]
    batches = "/".join(b["batches"])
    # the commands as run: the default run, or one shape at its batches
    if shape == HEADLINE:
        what, args, tag = "bench.py default run", "", "bench"
    else:
        tag = shape_tag(shape)
        what = "bench.py, one layer shape"
        args = f" --shape {shape} --batches {batches.replace('/', ',')} --no-cpu-baseline --no-dept"
    print(f"# Kernel trace: {what} ({shape}, batches {batches})\n")
    print("Command (repo root, one MI355X):\n\n```")
    print(f"rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_{tag} -o run -- "
          f"python -u bench.py{args}")
    print(f"python bench.py{args} > gpurun_out/{tag}.json")
    print(f"python bench.py --trace-report gpurun_out/prof_{tag}/run_kernel_trace.csv "
          f"gpurun_out/{tag}.json")
    print("```\n")
    print("Per-kernel durations, split by grid size (grid x = work-items; each decode batch gives "
          "its own grid per expert kernel). `__amd_rocclr_copyBuffer` rows are the weight-replica "
          "clones and torch-side copies of the harness.\n")
    summarize_trace(trace_csv)
    print("\nStage times of the unprofiled run (HIP events around each kernel; a combine "
          "of 0 means the down launch wrote y itself):\n")
    print("| batch | step us (graph) | weight GB/s | route us | top-k+plan us | gate/up us "
          "| down us | combine us |")
    print("|---|---|---|---|---|---|---|---|")
    for T, r in b["batches"].items():
        st = r["stage_us"]
        print(f"| {T} | {r['us']} | {r['GBps']} | {st['route']} | {st['dispatch']} | {st['gateup']} "
              f"| {st['down']} | {st['combine']} |")
    rf = b["roofline"]
    # the roofline launch's own grid (other shapes timed in the same run give
    # the kernel other grids)
    gx = rf.get("grid_workitems", 0)
    v = [d for (k, g, gy), vals in acc.items() if k == rf["kernel"] and g == gx for d in vals]
    mean = sum(v) / len(v) if v else float("nan")
    print(f"\nRoofline ({rf['kernel']}, batch {head_T}): {rf['achieved']} GB/s of {rf['peak']} GB/s "
          f"= {rf['frac']} ({rf['algorithmic_bytes_per_launch']} algorithmic bytes per launch / "
          f"{rf['launch_us']} us event-timed launch); the trace gives the same kernel at the "
          f"batch-{head_T} grid ({gx}) a mean of {mean:.2f} us.")


def summarize_pmc(path):
    """Mean per-dispatch counter values of a rocprofv3 --pmc run, per kernel
    and grid size."""
    import csv
    from collections import defaultdict
    acc = defaultdict(list)
    for r in csv.DictReader(open(path)):
        key = (_short(r["Kernel_Name"]), int(r.get("Grid_Size", r.get("Grid_Size_X", 0))),
               r["Counter_Name"])
        acc[key].append(float(r["Counter_Value"]))
    print("| kernel | grid | counter | dispatches | mean value |")
    print("|---|---|---|---|---|")
    for (k, g, c), v in sorted(acc.items()):
        print(f"| {k} | {g} | {c} | {len(v)} | {sum(v) / len(v):.1f} |")


def _pmc_rows(path):
    import csv
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def pmc_report(fetch_csv, write_csv, meta_path):
    """Calibrated HBM bytes per launch of the layer kernels from a FETCH_SIZE
    and a WRITE_SIZE run of --profile-pass.  The pass ends with a plain 1 GiB
    write (fill) and a plain 1 GiB read (sum) after the last layer kernel:
    the largest counter value among the dispatches after it calibrates each
    counter to bytes."""
    from collections import defaultdict
    meta = json.load(open(meta_path)) if os.path.exists(meta_path) else {}
    GiB_KiB = float(1 << 20)
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _pmc_rows(path) if r["Counter_Name"] == counter]
        last = max(i for i, r in enumerate(rows) if "moe::" in r["Kernel_Name"])
        calib = max(float(r["Counter_Value"]) for r in rows[last + 1:])
        acc = defaultdict(list)
        for r in rows[:last + 1]:
            if "moe::" in r["Kernel_Name"]:
                acc[(_short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        out[counter] = (calib, {k: sum(v) / len(v) for k, v in acc.items()},
                        {k: len(v) for k, v in acc.items()})
    rf, wf = GiB_KiB / out["FETCH_SIZE"][0], GiB_KiB / out["WRITE_SIZE"][0]
    fetch, write = out["FETCH_SIZE"][1], out["WRITE_SIZE"][1]
    shape = meta.get("shape", HEADLINE)
    T = meta.get("batch", HEADLINE_T)
    # the commands as run: the headline shape with the default paths, any
    # other shape with its own name, output folders and pass record
    if shape == HEADLINE:
        extra, fdir, wdir, meta_arg = "", "pmc_fetch", "pmc_write", ""
    else:
        tag = shape_tag(shape)
        extra = f" --shape {shape} --profile-meta gpurun_out/profile_pass_{tag}.json"
        fdir, wdir = f"pmc_{tag}_fetch", f"pmc_{tag}_write"
        meta_arg = f" --profile-meta gpurun_out/profile_pass_{tag}.json"
    print(f"# HBM traffic of the layer kernels, {shape}, batch {T}\n")
    print("Commands (repo root, one MI355X; one counter per pass):\n\n```")
    print(f"rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/{fdir} -o run -- python -u bench.py "
          f"--profile-pass{extra}")
    print(f"rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/{wdir} -o run -- python -u bench.py "
          f"--profile-pass{extra}")
    print(f"python bench.py --pmc-report gpurun_out/{fdir}/run_counter_collection.csv "
          f"gpurun_out/{wdir}/run_counter_collection.csv{meta_arg}")
    print("```\n")
    print(f"`--profile-pass` runs 20 eager batch-{T} steps, then a plain 1 GiB write (torch `fill_`) "
          "and a plain 1 GiB read (torch `sum`); the largest counter value after the last layer "
          "kernel calibrates each counter.\n")
    print(f"Calibration: 1 GiB read -> FETCH_SIZE {out['FETCH_SIZE'][0]:.1f} KiB (factor {rf:.5f}); "
          f"1 GiB write -> WRITE_SIZE {out['WRITE_SIZE'][0]:.1f} KiB (factor {wf:.5f}).\n")
    alg = {"gateup_kernel": meta.get("gateup_bytes"), "down_kernel": meta.get("down_bytes")}
    print("| kernel (grid) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) "
          "| algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|")
    traffic = {}
    for key in sorted(set(fetch) | set(write)):
        f_kib, w_kib = fetch.get(key, 0.0), write.get(key, 0.0)
        b = int(round((f_kib * rf + w_kib * wf) * 1024))
        traffic[key[0]] = b
        a = alg.get(key[0])
        ratio = f"{b / a:.4f}" if a else ""
        print(f"| {key[0]} ({key[1]}) | {out['FETCH_SIZE'][2].get(key, 0)} | {f_kib:.1f} | {w_kib:.1f} "
              f"| {b} | {a or ''} | {ratio} |")
    print()
    print(f"kernel_source_sha256: `{meta.get('kernel_source_sha256', kernel_source_hash())}`")
    print(f"traffic_bytes_per_launch: `{traffic.get('gateup_kernel', '')}`")


def desc_of(M, shape, max_tokens):
    return M.layer_desc(shape.d, shape.n_experts, shape.top_k, shape.d_ff, n_depts=shape.n_depts,
                        d_ff_dept=shape.d_ff_dept, d_ff_shared=shape.d_ff_shared,
                        score=shape.score, renormalize=shape.renormalize,
                        route_scale=shape.route_scale, dtype=shape.dtype, max_tokens=max_tokens,
                        dept_form=shape.dept_form, k_dept=shape.k_dept,
                        dept_strict=shape.dept_strict, expert_dtype=shape.expert_dtype)


def gateup_bytes(shape, T, n_active, n_active_depts, n_rows, n_dept_rows):
    """Algorithmic bytes of the gate/up stage: gate+up weights of every active
    matrix once (private transforms are S x S in the factorised form; FP8:
    one byte per weight plus a 4-byte scale per row), the T activation rows
    read, the h rows written (activation dtype)."""
    ab = 4 if shape.dtype == "f32" else 2
    fp8 = shape.expert_dtype == "fp8"
    wb = 1 if fp8 else ab
    d = shape.d
    k_priv = shape.d_ff if shape.dept_form == "factorised" else d
    b = n_active * 2 * shape.d_ff * (k_priv * wb + (4 if fp8 else 0))
    b += n_active_depts * 2 * shape.d_ff_dept * (d * wb + (4 if fp8 else 0))
    b += (2 * shape.d_ff_shared * (d * wb + (4 if fp8 else 0))) if shape.d_ff_shared else 0
    b += T * d * ab
    b += ab * (n_rows * shape.d_ff + n_dept_rows * shape.d_ff_dept + T * shape.d_ff_shared)
    return b


def down_bytes(shape, T, n_active, n_active_depts, n_rows, n_dept_rows):
    """Algorithmic bytes of the down stage: down weights of every active matrix
    once (FP8: one byte per weight plus a 4-byte scale per output row), the h
    rows read (activation dtype), the fp32 output rows written."""
    ab = 4 if shape.dtype == "f32" else 2
    fp8 = shape.expert_dtype == "fp8"
    wb = 1 if fp8 else ab
    d = shape.d
    n_priv = shape.d_ff if shape.dept_form == "factorised" else d
    sc = 4 if fp8 else 0
    b = n_active * n_priv * (shape.d_ff * wb + sc)
    b += n_active_depts * d * (shape.d_ff_dept * wb + sc)
    b += (d * (shape.d_ff_shared * wb + sc)) if shape.d_ff_shared else 0
    b += ab * (n_rows * shape.d_ff + n_dept_rows * shape.d_ff_dept + T * shape.d_ff_shared)
    b += 4 * (n_rows * n_priv + n_dept_rows * d + (T * d if shape.d_ff_shared else 0))
    return b


class Runner:
    """R replicas of one layer; step i runs replica i % R."""

    def __init__(self, M, moe_synth, shape, T, dev, replicas=None, base=None):
        import torch
        self.M, self.shape, self.T, self.dev = M, shape, T, dev
        self.desc = desc_of(M, shape, T)
        self.base = base if base is not None else moe_synth.make_layer(shape, 0, dev)
        self.x = moe_synth.make_tokens(shape, 0, T, dev)
        self.y = torch.empty_like(self.x)
        first = M.MoeLayer(self.desc, self.base, dev)
        first(self.x, self.y)
        torch.cuda.synchronize()
        plan = first.plan(T)
        self.plan = plan
        self.n_active = int(plan["active"].size)
        self.n_active_depts = int(plan.get("active_depts", []).__len__()) if shape.n_depts else 0
        self.n_rows = int(plan["n_rows"])
        self.n_dept_rows = int(plan.get("n_dept_rows", 0))
        self.step_bytes = M.moe_loaded_weight_bytes(self.desc, self.n_active, self.n_active_depts)
        self.step_bytes += 2 * T * shape.d * (4 if shape.dtype == "f32" else 2)
        if replicas is None:
            replicas = max(2, math.ceil((1 << 30) / max(1, self.step_bytes)))
        self.R = replicas
        self.layers = [first] + [M.MoeLayer(self.desc, moe_synth.clone_weights(self.base), dev)
                                 for _ in range(replicas - 1)]
        self.i = 0

    def step(self, events=None):
        self.layers[self.i % self.R](self.x, self.y, events)
        self.i += 1

    def time_eager(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            self.step()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3  # us

    def time_graph(self, steps, warmup):
        """Capture R consecutive steps (one per replica) into one HIP graph and
        replay it."""
        import torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(2):
                for r in range(self.R):
                    self.layers[r](self.x, self.y)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(self.R):
                self.layers[r](self.x, self.y)
        torch.cuda.synchronize()
        reps = max(1, math.ceil(steps / self.R))
        for _ in range(max(1, math.ceil(warmup / self.R))):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / (reps * self.R) * 1e3
        # spread: one event pair per replay (R steps each), in a pass of its own
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) / self.R * 1e3 for e0, e1 in evs)
        self.spread = {q: round(per[min(len(per) - 1, int(q / 100 * len(per)))], 2)
                       for q in (10, 50, 90)}
        # the graph must reproduce the eager result
        y_graph = self.y.clone()
        self.layers[0](self.x, self.y)
        torch.cuda.synchronize()
        same = bool(torch.equal(y_graph, self.y))
        return us, reps * self.R, same

    def stage_times(self, steps):
        """Mean kernel time per stage over `steps` eager steps: the library
        launches each stage's kernel with start/stop events the runtime writes
        at kernel begin/end (on the launch stream)."""
        import torch
        M = self.M
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * M.N_STAGES)]
               for _ in range(steps)]
        for e in evs:  # create the events before handing their handles over
            for ev in e:
                ev.record()
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        tot = [0.0] * M.N_STAGES
        for e in evs:
            for s in range(M.N_STAGES):
                tot[s] += e[2 * s].elapsed_time(e[2 * s + 1]) * 1e3
        out = {M.STAGE_NAMES[s]: tot[s] / steps for s in range(M.N_STAGES)}
        if M.moe_layer_kernel_count(self.desc, self.T) == 4:
            out["combine"] = 0.0  # done by the down launch: the interval is event overhead
        return out


def measured_peak_GBps(M, dev, gib=2, iters=10):
    """Achievable HBM read rate of the expert kernels' load pattern: the
    library's streaming-read helper over a `gib` GiB buffer (8x the 256 MB
    last-level cache), best of `iters`."""
    import torch
    n = (gib << 30) // 2
    a = torch.ones(n, dtype=torch.bfloat16, device=dev)
    sink = torch.empty((gib << 30) // 16384, dtype=torch.float32, device=dev)
    for _ in range(3):
        M.moe_stream_read(a, sink)
    torch.cuda.synchronize()
    best = None
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        M.moe_stream_read(a, sink)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    del a, sink
    torch.cuda.empty_cache()
    return round((gib << 30) / best * 1e-9, 1)


def sweep_report(path):
    """Markdown table of a --sweep run: one row per (shape, batch)."""
    rows, dv, fv = [], [], []
    for line in open(path):
        r = json.loads(line)
        if "dept_vs_vanilla" in r:
            dv.append(r["dept_vs_vanilla"])
        elif "fp8_vs_bf16" in r:
            fv.append(r["fp8_vs_bf16"])
        else:
            rows.append(r)
    print("# Every layer shape at its batches: graph-replayed decode step\n")
    print("Command (repo root, one MI355X):\n\n```")
    print("python bench.py --sweep --sweep-out gpurun_out/sweep.jsonl --no-cpu-baseline --no-dept")
    print("python bench.py --sweep-report gpurun_out/sweep.jsonl")
    print("```\n")
    print("Weights bytes are the distinct weights one step streams (router, active experts, "
          "active departments, shared expert) plus x in and y out; stage times come from HIP "
          "events around each kernel in eager steps (combine 0: the down launch wrote y).\n")
    print("| shape | batch | step us | weight MB | GB/s | active experts | active depts "
          "| route | top-k+plan | gate/up | down | combine |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        st = r["stage_us"]
        print(f"| {r['shape']} | {r['batch']} | {r['us']} | {r['weight_bytes'] / 1e6:.1f} | "
              f"{r['GBps']} | {r['active_experts']} | {r['active_depts']} | {st['route']} | "
              f"{st['dispatch']} | {st['gateup']} | {st['down']} | {st['combine']} |")
    if dv:
        print("\nDepartment forms against the vanilla DeepSeek-V3-shaped layer at the same batch "
              "(the slice-form transform shares its router and tokens; DeaMoE's own configuration "
              "is the budget-matched one of its Table 1):\n")
        print("| department shape | batch | vanilla us | department us | speedup "
              "| byte ratio (dept / vanilla) |")
        print("|---|---|---|---|---|---|")
        for r in dv:
            print(f"| {r.get('dept_shape', '')} | {r['batch']} | {r['vanilla_us']} | {r['dept_us']} "
                  f"| {r['speedup']} | {r['byte_ratio']} |")
    if fv:
        print("\nFP8 expert weights (E4M3 codes, per-row fp32 scales) against the bf16 layer of "
              "the same shape and draws at the same batch:\n")
        print("| FP8 shape | batch | bf16 us | FP8 us | speedup | byte ratio (FP8 / bf16) |")
        print("|---|---|---|---|---|---|")
        for r in fv:
            print(f"| {r['fp8_shape']} | {r['batch']} | {r['bf16_us']} | {r['fp8_us']} "
                  f"| {r['speedup']} | {r['byte_ratio']} |")


def dept_vs_vanilla(lines):
    """Department forms against the vanilla DeepSeek-V3-shaped layer at the
    same batch: the slice-form transform of it (same router, tokens and seed)
    and DeaMoE's own budget-matched configuration (its Table 1: same tokens
    and shared expert, 864 factorised experts); speedup beside the ratio of
    streamed bytes."""
    by = {(l["shape"], l["batch"]): l for l in lines}
    out = []
    van = "deepseek_v3_d7168_e256_i2048_s2048_top8"
    for dept in ("deamoe_dsv3_d7168_e256_m32_s1792_p256_top8",
                 "deamoe_paper_dsv3_d7168_e864_m8_h2048_top10"):
        for T in sorted({b for (s_, b) in by if s_ == dept}):
            if (van, T) in by:
                a, b = by[(van, T)], by[(dept, T)]
                out.append({"dept_shape": dept, "batch": T, "vanilla_us": a["us"], "dept_us": b["us"],
                            "speedup": round(a["us"] / b["us"], 3),
                            "vanilla_bytes": a["weight_bytes"], "dept_bytes": b["weight_bytes"],
                            "byte_ratio": round(b["weight_bytes"] / a["weight_bytes"], 3)})
    return out


def fp8_vs_bf16(lines):
    """Each FP8-expert layer against the bf16 layer of the same shape and
    draws at the same batch: speedup beside the ratio of streamed bytes."""
    by = {(l["shape"], l["batch"]): l for l in lines}
    out = []
    for (name, T), b in sorted(by.items()):
        if not name.endswith("_fp8") or (name[:-4], T) not in by:
            continue
        a = by[(name[:-4], T)]
        out.append({"fp8_shape": name, "batch": T, "bf16_us": a["us"], "fp8_us": b["us"],
                    "speedup": round(a["us"] / b["us"], 3),
                    "byte_ratio": round(b["weight_bytes"] / a["weight_bytes"], 3)})
    return out


KERNEL_SOURCES = ("moe_layer_decode_amd/csrc/moe_kernels.hip",
                  "moe_layer_decode_amd/csrc/moe_device.h",
                  "moe_layer_decode_amd/csrc/moe_internal.h")
PMC_SUMMARY = "profiles/pmc_layer_kernels_qwen3_30b_a3b_batch16.md"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, only
    if it was taken on the kernel sources as they are now (else None)."""
    path = os.path.join(ROOT, PMC_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("kernel_source_sha256",
                                                            "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(shape, T, base, steps):
    """The oracle, as is, on the host: full decode steps of the same layer at
    batch T on the same inputs.  Timed single-threaded and with every host
    core the process may use (numpy's BLAS thread pool), `steps` steps each;
    the median step of each.  The reported value is the faster of the two,
    with the thread count it used."""
    import statistics
    import moe_synth
    import oracle as O
    from threadpoolctl import threadpool_limits
    host = {k: v.detach().cpu() for k, v in base.items()}
    if shape.expert_dtype == "fp8":  # the layer on its dequantized weights
        host = O.dequantize_layer(host)
    x = moe_synth.make_tokens(shape, 0, T, "cpu")
    token_output = (O.deamoe_token_output if shape.dept_form == "factorised"
                    else O.layer_token_output)

    def one_step():
        t0 = time.perf_counter()
        ids, w, _, _ = O.route(x, host["w_router"], shape.top_k, shape.score,
                               host.get("router_bias"), shape.renormalize, shape.route_scale,
                               shape.n_depts, shape.k_dept, shape.dept_strict)
        for t in range(T):
            token_output(x[t], ids[t], w[t], host, shape.n_experts, shape.n_depts)
        return time.perf_counter() - t0

    ncores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    res = {}
    for nt in (1, ncores):
        with threadpool_limits(nt):
            one_step()  # warm-up: first-touch of the host weights
            res[nt] = statistics.median(one_step() for _ in range(max(3, steps)))
    best = min(res, key=res.get)
    return {"value": round(res[best] * 1e6, 1), "unit": "us", "cores": int(best), "kind": "oracle",
            "sample": f"median of {max(3, steps)} full decode steps of {shape.name} at batch {T} "
                      f"(numpy fp64 oracle), single-threaded and with {ncores} BLAS threads",
            "single_thread_us": round(res[1] * 1e6, 1),
            "all_core_us": round(res[ncores] * 1e6, 1), "all_core_threads": int(ncores),
            "nproc": int(os.cpu_count() or 0), "cpu_model": _cpu_model()}


def measure(M, moe_synth, shape, T, dev, base, steps, warmup, graph=True, stage_steps=100):
    """One (layer, batch) point: graph-replayed and eager step time, stage
    kernel times, streamed bytes and rates."""
    import torch
    r = Runner(M, moe_synth, shape, T, dev, base=base)
    eager_us = r.time_eager(steps, warmup)
    graph_us, graph_same = None, None
    if graph:
        try:
            graph_us, _, graph_same = r.time_graph(steps, warmup)
        except Exception as ex:  # report, fall back to eager
            log(f"graph capture failed: {ex!r}")
    stages = r.stage_times(min(steps, stage_steps))
    us = graph_us if (graph_us is not None and graph_same) else eager_us
    gu = gateup_bytes(shape, T, r.n_active, r.n_active_depts, r.n_rows, r.n_dept_rows)
    dn = down_bytes(shape, T, r.n_active, r.n_active_depts, r.n_rows, r.n_dept_rows)
    rec = {"us": round(us, 2), "eager_us": round(eager_us, 2),
           "graph_us": None if graph_us is None else round(graph_us, 2),
           "graph_matches_eager": graph_same,
           "graph_replay_us_p10_p50_p90": [r.spread[q] for q in (10, 50, 90)]
           if graph_us is not None else None,
           "weight_bytes": r.step_bytes, "active_experts": r.n_active,
           "active_depts": r.n_active_depts,
           "GBps": round(r.step_bytes / us * 1e-3, 1),
           "frac_peak": round(r.step_bytes / us * 1e-3 / HBM_PEAK_GBS, 4),
           "stage_us": {k: round(v, 2) for k, v in stages.items()},
           "gateup_GBps": round(gu / stages["gateup"] * 1e-3, 1) if stages["gateup"] > 0 else None,
           "down_GBps": round(dn / stages["down"] * 1e-3, 1) if stages["down"] > 0 else None,
           "expert_stream_GBps": round((gu + dn) / (stages["gateup"] + stages["down"]) * 1e-3, 1),
           "expert_stream_frac_peak": round((gu + dn) / (stages["gateup"] + stages["down"]) * 1e-3
                                            / HBM_PEAK_GBS, 4),
           "replicas": r.R}
    del r
    torch.cuda.empty_cache()
    return rec, gu, stages


def expanded_vanilla(shape, base):
    """The department layer as a vanilla layer whose expert e carries the
    concatenated [department slice ; private slice] matrices (the same
    function; DeaMoE's loading comparison counts these bytes)."""
    import dataclasses
    import torch
    G = shape.n_experts // shape.n_depts
    dept = torch.arange(shape.n_experts, device=base["w_gate"].device) // G
    w = {"w_router": base["w_router"],
         "w_gate": torch.cat([base["wd_gate"][dept], base["w_gate"]], 1).contiguous(),
         "w_up": torch.cat([base["wd_up"][dept], base["w_up"]], 1).contiguous(),
         "w_down": torch.cat([base["wd_down"][dept], base["w_down"]], 2).contiguous()}
    if base.get("router_bias") is not None:
        w["router_bias"] = base["router_bias"]
    for k in ("ws_gate", "ws_up", "ws_down"):
        if base.get(k) is not None:
            w[k] = base[k]
    sh = dataclasses.replace(shape, name=shape.name + "_expanded_vanilla", n_depts=0,
                             d_ff_dept=0, d_ff=shape.d_ff_dept + shape.d_ff)
    return sh, w


def department_comparisons(M, moe_synth, dev, steps, warmup):
    """Timed department numbers: the DeaMoE-7B-shaped department
    layer against its expanded vanilla form at batches 1/4/16, and the
    department transform of the DeepSeek-V3-shaped layer against that layer
    (same tokens, router and bias) at 1/4/16; each speedup beside the ratio
    of streamed bytes (DeaMoE section 3.3, Figure 2; section 5.2)."""
    import torch
    out = {}
    dept = moe_synth.SHAPES["deamoe_7b_d2048_e64_m8_s1024_p128_top8"]
    base = moe_synth.make_layer(dept, 0, dev)
    vsh, vw = expanded_vanilla(dept, base)
    rows = {}
    for T in (1, 4, 16):
        a, _, _ = measure(M, moe_synth, dept, T, dev, base, steps, warmup, stage_steps=30)
        b, _, _ = measure(M, moe_synth, vsh, T, dev, vw, steps, warmup, stage_steps=30)
        rows[str(T)] = {"dept": a, "expanded_vanilla": b,
                        "speedup": round(b["us"] / a["us"], 3),
                        "byte_ratio": round(a["weight_bytes"] / b["weight_bytes"], 3)}
        log(f"{dept.name} T={T}: dept {a['us']} us, expanded {b['us']} us, "
            f"speedup {rows[str(T)]['speedup']} (byte ratio {rows[str(T)]['byte_ratio']})")
    out[dept.name] = rows
    del base, vw
    torch.cuda.empty_cache()
    van = moe_synth.SHAPES["deepseek_v3_d7168_e256_i2048_s2048_top8"]
    tr = moe_synth.SHAPES["deamoe_dsv3_d7168_e256_m32_s1792_p256_top8"]
    vrec = {}
    base = moe_synth.make_layer(van, 0, dev)
    for T in (1, 4, 16):
        vrec[T], _, _ = measure(M, moe_synth, van, T, dev, base, steps, warmup, stage_steps=30)
        log(f"{van.name} T={T}: {vrec[T]['us']} us")
    del base
    torch.cuda.empty_cache()
    base = moe_synth.make_layer(tr, 0, dev)
    rows = {}
    for T in (1, 4, 16):
        a, _, _ = measure(M, moe_synth, tr, T, dev, base, steps, warmup, stage_steps=30)
        b = vrec[T]
        rows[str(T)] = {"dept": a, "vanilla": b, "speedup": round(b["us"] / a["us"], 3),
                        "byte_ratio": round(a["weight_bytes"] / b["weight_bytes"], 3)}
        log(f"{tr.name} T={T}: {a['us']} us vs {b['us']} us, speedup {rows[str(T)]['speedup']} "
            f"(byte ratio {rows[str(T)]['byte_ratio']})")
    out[tr.name + "_vs_" + van.name] = rows
    del base
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.source_hash:
        print(kernel_source_hash())
        return
    if args.sweep_report:
        sweep_report(args.sweep_report)
        return
    if args.trace_report:
        trace_report(*args.trace_report)
        return
    if args.pmc_report:
        pmc_report(args.pmc_report[0], args.pmc_report[1], args.profile_meta)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this layer's hot path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_layer_decode_amd as M
    import moe_synth

    M.lib()
    dev = torch.device("cuda:0")
    shape = moe_synth.SHAPES[args.shape]
    batches = [int(b) for b in args.batches.split(",")]
    head_T = HEADLINE_T if HEADLINE_T in batches else batches[-1]
    log(f"bench: {shape.name} batches {batches}, steps {args.steps}, warmup {args.warmup}")
    base = moe_synth.make_layer(shape, 0, dev)

    if args.profile_pass:
        r = Runner(M, moe_synth, shape, head_T, dev, base=base)
        r.time_eager(20, 2)
        meta = {"shape": shape.name, "batch": head_T, "kernel_source_sha256": kernel_source_hash(),
                "gateup_bytes": gateup_bytes(shape, head_T, r.n_active, r.n_active_depts,
                                             r.n_rows, r.n_dept_rows),
                "down_bytes": down_bytes(shape, head_T, r.n_active, r.n_active_depts,
                                         r.n_rows, r.n_dept_rows)}
        os.makedirs(os.path.dirname(args.profile_meta) or ".", exist_ok=True)
        with open(args.profile_meta, "w") as f:
            json.dump(meta, f)
        # counter calibration: a plain 1 GiB read (sum) and a plain 1 GiB write (fill)
        n = 1 << 30
        a = torch.empty(n // 4, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        a.fill_(1.0)
        torch.cuda.synchronize()
        log(f"calibration sum {float(a.sum()):.0f}")
        torch.cuda.synchronize()
        log("profile pass done")
        return

    per_batch, head = {}, None
    for T in batches:
        rec, gu, stages = measure(M, moe_synth, shape, T, dev, base, args.steps, args.warmup,
                                  graph=not args.no_graph)
        per_batch[str(T)] = rec
        log(f"T={T}: {json.dumps(rec)}")
        if T == head_T:
            head = (rec, rec["us"], gu, stages)
        torch.cuda.empty_cache()

    rec, us, gu, stages = head
    head_R = rec["replicas"]
    achieved = gu / stages["gateup"] * 1e-3  # GB/s
    meas_peak = measured_peak_GBps(M, dev)
    out = {
        "metric": METRIC, "value": round(us, 2), "unit": "us", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": shape.dtype, "data": "synthetic",
        "config": {"workload": f"{shape.name} MoE FFN layer decode step, batch {head_T}",
                   "batch": head_T, "d": shape.d, "experts": shape.n_experts,
                   "top_k": shape.top_k, "d_ff": shape.d_ff, "replicas": head_R,
                   "timing": "hipgraph" if per_batch[str(head_T)]["graph_matches_eager"] else "eager"},
        "hbm_GBps": per_batch[str(head_T)]["GBps"],
        "batches": per_batch,
        "roofline": {"bound": "hbm",
                     "kernel": "gateup_fp8_kernel" if shape.expert_dtype == "fp8" else "gateup_kernel",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if shape.name == HEADLINE and head_T == 16 else None,
                     "algorithmic_bytes_per_launch": gu,
                     "launch_us": round(stages["gateup"], 2),
                     # the launch's grid as a kernel trace reports it (work-items)
                     "grid_workitems": M.moe_layer_launch_workitems(desc_of(M, shape, head_T),
                                                                    head_T, M.STAGE_GATEUP),
                     "measured_peak": meas_peak,
                     "frac_measured_peak": round(achieved / meas_peak, 4)},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(shape, head_T, base, args.cpu_steps)
        log(f"cpu baseline: {json.dumps(out['cpu_baseline'])}")
    if not args.no_dept and shape.name == HEADLINE:
        del base
        torch.cuda.empty_cache()
        base = None
        out["department_layers"] = department_comparisons(M, moe_synth, dev, args.dept_steps,
                                                          max(5, args.warmup // 2))
        base = moe_synth.make_layer(shape, 0, dev) if args.sweep else None
    if args.sweep:
        os.makedirs(os.path.dirname(args.sweep_out) or ".", exist_ok=True)
        sweep_lines = []
        with open(args.sweep_out, "w") as f:
            for name, sh in moe_synth.SHAPES.items():
                if name == shape.name:
                    continue
                del base
                torch.cuda.empty_cache()
                base = moe_synth.make_layer(sh, 0, dev)
                for T in sh.batches:
                    rr = Runner(M, moe_synth, sh, T, dev, base=base)
                    e_us = rr.time_eager(max(20, args.steps // 4), 5)
                    g_us = None
                    try:
                        g_us, _, same = rr.time_graph(max(20, args.steps // 4), 5)
                        g_us = g_us if same else None
                    except Exception as ex:
                        log(f"graph capture failed: {ex!r}")
                    st = rr.stage_times(20)
                    u = g_us or e_us
                    line = {"shape": name, "batch": T, "us": round(u, 2), "eager_us": round(e_us, 2),
                            "weight_bytes": rr.step_bytes, "active_experts": rr.n_active,
                            "active_depts": rr.n_active_depts,
                            "GBps": round(rr.step_bytes / u * 1e-3, 1),
                            "stage_us": {k: round(v, 2) for k, v in st.items()}}
                    sweep_lines.append(line)
                    f.write(json.dumps(line) + "\n")
                    f.flush()
                    log(json.dumps(line))
                    del rr
                    torch.cuda.empty_cache()
            dv = dept_vs_vanilla(sweep_lines)
            for line in dv:
                f.write(json.dumps({"dept_vs_vanilla": line}) + "\n")
            out["dept_vs_vanilla"] = dv
            # the headline shape's own line joins the FP8 comparison
            head_line = {"shape": shape.name, "batch": head_T, "us": round(us, 2),
                         "weight_bytes": per_batch[str(head_T)]["weight_bytes"]}
            extra = [dict(head_line, batch=int(b), us=r["us"], weight_bytes=r["weight_bytes"])
                     for b, r in per_batch.items()]
            fv = fp8_vs_bf16(sweep_lines + extra)
            for line in fv:
                f.write(json.dumps({"fp8_vs_bf16": line}) + "\n")
            out["fp8_vs_bf16"] = fv
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
