#!/usr/bin/env python3
"""Throughput of one speculative draft step of the shortlisted draft head.

A step is the whole hot path over one batch: for each of T draft positions
the router scores the clusters, the position's budget selects clusters, the
shortlist is built, the gathered LM head projects the hidden state onto it
and a draft token is sampled (router work of position t+1 on a second stream,
overlapped with the head of position t); then the drafts are verified by
rejection sampling against the softmax of the target logits (the softmax's
segment statistics, then the verification computing each target probability
it reads).  Default workload: Llama-3-8B-shaped head, V=128256, d=4096, bf16,
1024 Zipf-sized clusters, batch 1, depth 6, token budget 32768 -> 16384.

Inputs are seeded and synthetic.  Steps rotate over several input instances
(different hidden states, hence different shortlists), and every (instance,
position) head launch reads its own identical copy of W in HBM, so no launch
finds its rows in the 256 MB memory-side cache from an earlier one.

Printed: one JSON line (value = draft tokens/s of the whole step), with
`roofline` for the gathered head (algorithmic bytes per launch / its mean
duration; the duration comes from HIP events stamped at the head kernels'
own start and end, on eager replays of the timed steps, since events cannot
be timed inside graphs) and `cpu_baseline` (the CPU oracle, one core, on a
bounded sample of the same workload).  `roofline.traffic` (in the line and
in each workload of its `extra` block) is the head's measured HBM bytes per
launch when that workload's file under profiles/ (TRAFFIC_FILES) was made
from the current sources of its head kernel (see --pmc-probe).

HBM traffic of a workload's head (two profiler passes, then one parse):
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -- python3 bench.py --config C --pmc-probe
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -- python3 bench.py --config C --pmc-probe
    python3 bench.py --traffic-from OUT/fetch OUT/write
(all three with the same --probe-file; the parse writes the workload's file)
The probe runs eager steps of the workload, then a 1 GiB device-to-device
copy; each counter of the head is scaled by known bytes / the counter of
that copy.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# committed HBM traffic counters of each workload's head (--traffic-from)
TRAFFIC_FILES = {1: "head_gemv_traffic.json", 2: "head_union_traffic_llama3-8b-b32.json",
                 3: "head_gathered_traffic_qwen3-8b-8x64.json",
                 4: "head_union_traffic_gemma3-12b-b64.json"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", TRAFFIC_FILES[1])
# each head kernel's translation unit: its counters hold while it is unchanged
_CSRC = "dynamic_vocabulary_draft_amd/csrc/"
_MFMA_SOURCES = [_CSRC + f for f in ("head_mfma.hip", "mfma_tile.h", "common.h", "kernels.h")]
HEAD_SOURCES = {"head_gemv_kernel": [_CSRC + f for f in ("head.hip", "common.h", "kernels.h")],
                "head_union_kernel": _MFMA_SOURCES, "head_gathered_kernel": _MFMA_SOURCES}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def head_source_sha(kernel: str = "head_gemv_kernel") -> str:
    h = hashlib.sha256()
    for f in HEAD_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def cpu_baseline(wl, seconds: float, static_ids=None) -> dict:
    import oracle
    from oracle import pipeline as opipe
    oracle.build(force=False)
    cfg = wl.cfg
    # one core: this thread is pinned to the lowest core it may run on (in
    # this process, no re-exec), and the affinity is restored afterwards
    old_aff = os.sched_getaffinity(0)
    core = min(old_aff)
    os.sched_setaffinity(0, {core})
    try:
        n, t0 = 0, time.perf_counter()
        while True:
            if static_ids is None:
                opipe.run_step(wl)
            else:
                opipe.run_static_step(wl, static_ids)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
            log("oracle step %d done (%.1f s)" % (n, el))
    finally:
        os.sched_setaffinity(0, old_aff)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    per_step = cfg.B * (cfg.tree_nodes if cfg.is_tree else cfg.T)
    what = ("router, selection, shortlist, fp64 gathered head over all %d tree nodes, sampling, "
            "target softmax and tree verification" % cfg.tree_nodes if cfg.is_tree else
            "%s for all %d positions, target softmax and verification"
            % ("router, selection, shortlist, fp64 gathered head, sampling"
               if static_ids is None else "fp64 head over the static shortlist, sampling", cfg.T))
    return {"value": per_step * n / el, "unit": "draft tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d full step(s) of instance 0 (%s), %.1f s on 1 thread pinned to core "
                      "%d of %d (%s)" % (n, what, el, core, os.cpu_count() or 0,
                                         model or platform.machine())}


COPY_BYTES = 1 << 30


def head_kernel_name(cfg) -> str:
    from dynamic_vocabulary_draft_amd import synthetic as syn
    hrows = cfg.tree_nodes if cfg.is_tree else 1
    bf16 = cfg.dtype == syn.DT_BF16
    if bf16 and hrows == 1 and cfg.B >= 8:
        return "head_union_kernel"
    if bf16 and hrows >= 8:
        return "head_gathered_kernel"
    return "head_gemv_kernel"


def traffic_file(workload: str):
    """The committed traffic counters of this workload's head, or None."""
    from dynamic_vocabulary_draft_amd import synthetic as syn
    for i, name in TRAFFIC_FILES.items():
        if syn.CONFIGS[i].name == workload:
            return os.path.join(ROOT, "profiles", name)
    return None


def pmc_probe(args, cfg, steps, sizes, npos, stream, torch, np):
    """Eager steps over every (instance, position), then a plain copy of
    COPY_BYTES; writes the algorithmic bytes of each head launch, in launch
    order, to --probe-file."""
    e = cfg.elem_bytes
    hrows = cfg.tree_nodes if cfg.is_tree else 1
    n_steps = 2 * len(steps)
    launch_bytes = []
    with torch.cuda.stream(stream):
        for k in range(n_steps):
            i = k % len(steps)
            steps[i].step(stream)
            for t in range(npos):
                sz = sizes[i][t]
                launch_bytes.append(sz["union"] * cfg.d * e + sz["total"] * 4
                                    + cfg.B * hrows * cfg.d * e + sz["total"] * hrows * 4)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    with open(args.probe_file, "w") as f:
        json.dump({"workload": cfg.name, "head_kernel": head_kernel_name(cfg),
                   "launch_bytes": launch_bytes, "copy_bytes": COPY_BYTES,
                   "kernel_source_sha256": head_source_sha(head_kernel_name(cfg))}, f)
    log("pmc probe: %d head launches, copy of %d bytes" % (len(launch_bytes), COPY_BYTES))


def _counter_rows(d, counter):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv output."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    rows = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r.get("Dispatch_Id", 0)), r["Kernel_Name"],
                                 float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


def traffic_from(args):
    with open(args.probe_file) as f:
        probe = json.load(f)
    out = {"workload": probe["workload"], "kernel_source_sha256": probe["kernel_source_sha256"]}
    per = {}
    for name, d in (("FETCH_SIZE", args.traffic_from[0]), ("WRITE_SIZE", args.traffic_from[1])):
        rows = _counter_rows(d, name)
        copy = [v for k, v in rows if "copy" in k.lower()]
        head = [v for k, v in rows if probe["head_kernel"] in k]
        if not copy or not head:
            raise SystemExit("%s: copy or head dispatches missing" % name)
        copy_kib = copy[-1]  # the probe's copy is its last dispatch
        scale = probe["copy_bytes"] / (copy_kib * 1024.0)
        per[name] = {"head_kib_mean": sum(head) / len(head), "launches": len(head),
                     "copy_kib": copy_kib, "scale": scale,
                     "bytes_per_launch": sum(head) / len(head) * 1024.0 * scale}
    alg = sum(probe["launch_bytes"]) / len(probe["launch_bytes"])
    out.update({
        "head_kernel": probe["head_kernel"],
        "fetch_bytes_per_launch": round(per["FETCH_SIZE"]["bytes_per_launch"]),
        "write_bytes_per_launch": round(per["WRITE_SIZE"]["bytes_per_launch"]),
        "bytes_per_launch": round(per["FETCH_SIZE"]["bytes_per_launch"]
                                  + per["WRITE_SIZE"]["bytes_per_launch"]),
        "algorithmic_bytes_per_launch": round(alg),
        "fetch_scale": per["FETCH_SIZE"]["scale"], "write_scale": per["WRITE_SIZE"]["scale"],
        "launches": per["FETCH_SIZE"]["launches"],
        "copy_bytes": probe["copy_bytes"],
        "copy_fetch_kib": per["FETCH_SIZE"]["copy_kib"],
        "copy_write_kib": per["WRITE_SIZE"]["copy_kib"],
    })
    out["traffic_over_algorithmic"] = round(out["bytes_per_launch"] / alg, 4)
    dest = args.traffic_out or traffic_file(probe["workload"])
    if dest is None:
        raise SystemExit("no committed traffic file for %s: give --traffic-out" % probe["workload"])
    with open(dest, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def overlap_from(args):
    """Concurrency with the gathered head in a rocprofv3 kernel trace (the
    SQLite results file of `rocprofv3 --kernel-trace`): for every other
    kernel, its launches, mean duration, the share of its time during which
    a head kernel was running, and the share of its launches that
    overlapped a head at all.  Printed as a markdown table."""
    import re
    import sqlite3

    con = sqlite3.connect(args.overlap_from)
    rows = con.execute("select name, start, end from kernels order by start").fetchall()
    con.close()

    def short(n):
        n = n.replace("void ", "").replace("ds::(anonymous namespace)::", "")
        return re.split(r"[<(]", n)[0]

    heads = [(a, b) for n, a, b in rows if short(n).startswith("head_")]
    stats = {}
    for n, a, b in rows:
        k = short(n)
        if k.startswith("head_") or "rocclr" in n or "at::" in n:
            continue
        ov = 0
        for ha, hb in heads:  # sorted by start; heads do not overlap each other
            if hb <= a:
                continue
            if ha >= b:
                break
            ov += min(b, hb) - max(a, ha)
        d = stats.setdefault(k, [0, 0.0, 0.0, 0])
        d[0] += 1
        d[1] += (b - a) / 1e3
        d[2] += ov / 1e3
        d[3] += ov > 0
    hk = sorted({short(n) for n, _, _ in rows if short(n).startswith("head_")})
    print("| kernel | launches | mean us | time beside a head | launches beside a head |")
    print("|---|---:|---:|---:|---:|")
    for k, (cnt, tot, ov, anyc) in sorted(stats.items(), key=lambda x: -x[1][1]):
        print("| %s | %d | %.2f | %.0f%% | %.0f%% |" % (k, cnt, tot / cnt, 100 * ov / tot,
                                                       100 * anyc / cnt))
    hs = [(b - a) / 1e3 for a, b in heads]
    print("\nhead kernels (%s): %d launches, mean %.2f us" % (", ".join(hk), len(hs),
                                                            sum(hs) / max(1, len(hs))))


def stats_from(args):
    """Kernel statistics as a markdown table (kernel, calls, mean / min / max
    / total microseconds, share): from the kernel_stats.csv of `rocprofv3
    --stats`, or aggregated from the kernels of a results database (.db)."""
    import csv
    import re

    if args.stats_from.endswith(".db"):
        import sqlite3

        con = sqlite3.connect(args.stats_from)
        agg = con.execute("select name, count(*), avg(end - start), min(end - start), "
                          "max(end - start), sum(end - start) from kernels group by name"
                          ).fetchall()
        con.close()
        rows = [{"Name": n, "Calls": c, "AverageNs": a, "MinNs": lo, "MaxNs": hi,
                 "TotalDurationNs": t} for n, c, a, lo, hi, t in agg]
    else:
        with open(args.stats_from) as f:
            rows = list(csv.DictReader(f))
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    print("| kernel | calls | avg us | min us | max us | total us | % |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        n = re.sub(r"^void ", "", r["Name"])
        n = n.replace("ds::(anonymous namespace)::", "").replace("ds::", "")
        depth, cut = 0, len(n)  # drop the parameter list
        for i, ch in enumerate(n):
            if ch == "<":
                depth += 1
            elif ch == ">":
                depth -= 1
            elif ch == "(" and depth == 0:
                cut = i
                break
        n = n[:cut] if cut < 60 else n[:60] + "..."
        print("| %s | %s | %.2f | %.2f | %.2f | %.1f | %.2f |" % (
            n, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3,
            100 * float(r["TotalDurationNs"]) / tot))


PEAK_BF16_TFLOPS = 2500.0


def kmeans_bench(args):
    """Spherical k-means over the LM head's rows at the workload's shape:
    inverse norms once, then timed iterations of update (centroids from the
    labels) + assignment (labels from the centroids, on the matrix cores)."""
    import numpy as np
    import torch

    from dynamic_vocabulary_draft_amd import native as N
    from dynamic_vocabulary_draft_amd import synthetic as syn
    from dynamic_vocabulary_draft_amd.pipeline import to_dev

    torch.cuda.set_device(0)
    cfg = syn.CONFIGS[args.config]
    if cfg.dtype != syn.DT_BF16:
        raise SystemExit("--kmeans needs a bf16 head")
    V, d, M = cfg.V, cfg.d, cfg.M
    cluster_of, _ = syn.make_clusters(cfg)
    W_host = syn.make_lm_head(cfg, cluster_of, threads=min(16, os.cpu_count() or 8))
    W = to_dev(W_host)
    lab0 = syn.kmeans_init_assign(cfg, cluster_of, 0.5)
    lab = to_dev(lab0)
    inv = torch.empty(V, device="cuda")
    C32 = torch.zeros(M, d, device="cuda")
    C32b = torch.empty(M, d, device="cuda")
    Cb = torch.empty(M, d, dtype=torch.bfloat16, device="cuda")
    size = torch.empty(M, dtype=torch.int32, device="cuda")
    norm = torch.empty(M, dtype=torch.float64, device="cuda")
    score = torch.empty(V, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    uws = N.workspace(N.kmeans_update_workspace_bytes(V, d, M))
    aws = N.workspace(N.lib.ds_kmeans_assign_workspace_bytes(V))
    ev = N.HipEvents()
    N.kmeans_inv_norms(W, inv)
    bufs = [C32, C32b]

    def iteration(k, events=None):
        prev, out = bufs[k % 2], bufs[(k + 1) % 2]
        N.kmeans_update(W, inv, lab, prev, out, Cb, size, norm, uws, err_flag=flag)
        N.kmeans_assign(W, Cb, lab, score, aws, events=events)

    iteration(0)
    torch.cuda.synchronize()
    objs = [float(norm.sum().item())]
    n_it = args.kmeans_iters
    evs = ev.array(2 * n_it)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(n_it):
        iteration(k + 1, (evs[2 * k], evs[2 * k + 1]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    objs.append(float(norm.sum().item()))
    assert int(flag.item()) == 0
    durs = [ev.elapsed_ms(evs[2 * k], evs[2 * k + 1]) for k in range(n_it)]
    flops = 2.0 * V * M * d
    t_assign = float(np.mean(durs)) * 1e-3
    achieved = flops / t_assign / 1e12
    out = {
        "metric": "spherical k-means iterations/s over the LM-head rows (update + assignment), "
                  "V=%d d=%d M=%d bf16" % (V, d, M),
        "value": round(n_it / wall, 3), "unit": "iterations/s", "n_gpus": 1,
        "steps": n_it, "warmup": 1, "ms_per_step": round(wall * 1e3 / n_it, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic clustered-Gaussian LM head, labels started from the planted "
                "clusters with half of them random",
        "config": {"workload": "spherical k-means over the %s head" % cfg.name, "V": V, "d": d,
                   "clusters": M},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "assign": {"kernel": "kmeans_assign_kernel", "mean_us": round(t_assign * 1e6, 1),
                   "flops": flops, "timed_on": "HIP events stamped at the kernel's own start "
                                               "and end"},
        "update_plus_assign_ms": round(wall * 1e3 / n_it, 3),
        "objective": {"after_first_update": objs[0], "after_last_update": objs[1]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        rows = 256
        t1 = time.perf_counter()
        oracle.kmeans_assign(W_host[:rows], Cb.cpu().view(torch.int16).numpy().view(np.uint16))
        t_rows = time.perf_counter() - t1
        t1 = time.perf_counter()
        inv_h = oracle.kmeans_inv_norms(W_host)
        oracle.kmeans_update(W_host, inv_h, lab0, np.zeros((M, d), np.float32))
        t_upd = time.perf_counter() - t1
        t_it = t_rows * V / rows + t_upd
        out["cpu_baseline"] = {
            "value": round(1.0 / t_it, 6), "unit": "iterations/s", "cores": 1, "kind": "oracle",
            "sample": "assignment of %d of %d rows (%.1f s, extrapolated linearly to all rows) "
                      "+ inverse norms and one full update (%.1f s), 1 thread"
                      % (rows, V, t_rows, t_upd)}
    print(json.dumps(out), flush=True)


def router_train_bench(args):
    """Router training at the workload's shape: per step, the full drafter's
    logits for n training rows (the dense head on the matrix cores), their
    top-L cluster labels, and one SGD step of the router; input batches
    rotate over four instances."""
    import numpy as np
    import torch

    from dynamic_vocabulary_draft_amd import native as N
    from dynamic_vocabulary_draft_amd import synthetic as syn
    from dynamic_vocabulary_draft_amd.pipeline import to_dev

    torch.cuda.set_device(0)
    cfg = syn.CONFIGS[args.config]
    if cfg.dtype != syn.DT_BF16:
        raise SystemExit("--router-train needs a bf16 head")
    V, d, r, M = cfg.V, cfg.d, cfg.r, cfg.M
    n, L = args.train_rows, args.train_top
    cluster_of, _ = syn.make_clusters(cfg)
    W_host = syn.make_lm_head(cfg, cluster_of, threads=min(16, os.cpu_count() or 8))
    W = to_dev(W_host)
    R = syn.make_router(cfg)
    f32 = {k: syn.bf16_bits_to_f32(v) for k, v in R.items()}  # fp32 master weights
    P = {k: to_dev(v) for k, v in f32.items()}
    G = {k: torch.empty_like(v) for k, v in P.items()}
    hs = [to_dev(syn.make_train_hidden(cfg, n, instance=i)) for i in range(4)]
    co = to_dev(cluster_of)
    logits = torch.empty(n, V, device="cuda")
    labels = torch.empty(n, M, dtype=torch.uint8, device="cuda")
    loss = torch.empty(1, dtype=torch.float64, device="cuda")
    tws = N.workspace(N.router_train_workspace_bytes(n, r, M))
    ev = N.HipEvents()
    lr = 0.05

    def step(k, events=None):
        h = hs[k % len(hs)]
        N.dense_lm_head(W, h, logits, events=events)
        N.router_labels(logits, co, M, L, labels)
        N.router_train_step(h, labels, P["W1"], P["b1"], P["W2"], P["b2"], G, loss, cfg.act, lr,
                            tws)

    for k in range(max(args.warmup, 4)):
        step(k)
    torch.cuda.synchronize()
    losses = [float(loss.item())]
    steps = args.steps
    evs = ev.array(2 * steps)
    t_lab = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        h = hs[k % len(hs)]
        N.dense_lm_head(W, h, logits, events=(evs[2 * k], evs[2 * k + 1]))
        t_lab[3 * k].record()
        N.router_labels(logits, co, M, L, labels)
        t_lab[3 * k + 1].record()
        N.router_train_step(h, labels, P["W1"], P["b1"], P["W2"], P["b2"], G, loss, cfg.act, lr,
                            tws)
        t_lab[3 * k + 2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    losses.append(float(loss.item()))
    head_us = float(np.mean([ev.elapsed_ms(evs[2 * k], evs[2 * k + 1]) for k in range(steps)])) * 1e3
    lab_us = float(np.mean([t_lab[3 * k].elapsed_time(t_lab[3 * k + 1])
                            for k in range(steps)])) * 1e3
    trn_us = float(np.mean([t_lab[3 * k + 1].elapsed_time(t_lab[3 * k + 2])
                            for k in range(steps)])) * 1e3
    e = cfg.elem_bytes
    head_bytes = V * d * e + n * d * e + n * V * 4  # W once, the hidden rows, the logits
    head_flops = 2.0 * n * V * d
    achieved = head_bytes / (head_us * 1e-6) / 1e9
    train_flops = 2.0 * n * (2 * r * d + 3 * M * r)
    out = {
        "metric": "router training rows/s (full-drafter logits, top-%d cluster labels, one SGD "
                  "step of the %d->%d->%d router), V=%d d=%d bf16 head" % (L, d, r, M, V, d),
        "value": round(n * steps / wall, 1), "unit": "training rows/s", "n_gpus": 1,
        "steps": steps, "warmup": max(args.warmup, 4), "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: clustered-Gaussian head, N(0,1) training hidden states (4 batches "
                "rotated), router initialised as the drafting router",
        "config": {"workload": "router training on the %s head, %d rows per step" % (cfg.name, n),
                   "V": V, "d": d, "router": "%d->%d->%d" % (d, r, M), "rows": n, "top_L": L,
                   "lr": lr},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None},
        "dense_head": {"kernel": "kmeans_assign_kernel<true> (dense head: W x h^T on the "
                                 "matrix cores, store epilogue)",
                       "mean_us": round(head_us, 1), "algorithmic_bytes": head_bytes,
                       "algorithmic_flops": head_flops,
                       "flop_per_byte": round(head_flops / head_bytes, 1),
                       "tflops": round(head_flops / (head_us * 1e-6) / 1e12, 1),
                       "mfma_frac": round(head_flops / (head_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                                          4)},
        "labels_us": round(lab_us, 1),
        "train_step": {"mean_us": round(trn_us, 1), "flops": train_flops,
                       "tflops_fp32": round(train_flops / (trn_us * 1e-6) / 1e12, 2)},
        "loss": {"before": losses[0], "after": losses[1]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        rows = 2
        hh = syn.make_train_hidden(cfg, rows)
        t1 = time.perf_counter()
        lg = oracle.dense_lm_head(W_host, hh)
        lab = oracle.topl_labels(lg, cluster_of, M, L)
        t_lab_rows = time.perf_counter() - t1
        nt = 8
        ht = syn.bf16_bits_to_f32(syn.make_train_hidden(cfg, nt))
        yt = np.zeros((nt, M), np.uint8)
        yt[:rows] = lab
        t1 = time.perf_counter()
        oracle.router_train_step(ht, yt, f32["W1"], f32["b1"], f32["W2"], f32["b2"], cfg.act, lr)
        t_step = time.perf_counter() - t1
        per_row = t_lab_rows / rows + t_step / nt
        out["cpu_baseline"] = {
            "value": round(1.0 / per_row, 4), "unit": "training rows/s", "cores": 1,
            "kind": "oracle",
            "sample": "dense logits + labels of %d rows (%.1f s) and one step on %d rows "
                      "(%.1f s), 1 thread; per-row costs added" % (rows, t_lab_rows, nt, t_step)}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload index (1: Llama-shaped b1)")
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--no-replicas", action="store_true",
                    help="all head launches read one copy of W (cache-warm)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run eager steps and a 1 GiB copy under a counter profiler, then exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc outputs of --pmc-probe into "
                         "profiles/head_gemv_traffic.json and exit")
    ap.add_argument("--traffic-out", default=None,
                    help="where --traffic-from writes (default: the file the bench line "
                         "reads the probed workload's traffic from)")
    ap.add_argument("--stats-from", metavar="STATS_CSV_OR_DB",
                    help="print kernel statistics (a rocprofv3 --stats kernel_stats.csv, or a "
                         "--kernel-trace results database) as a markdown table, and exit")
    ap.add_argument("--overlap-from", metavar="RESULTS_DB",
                    help="print, from a rocprofv3 --kernel-trace results database, how much "
                         "of every kernel's time ran beside a head kernel, and exit")
    ap.add_argument("--probe-file", default=os.path.join(ROOT, "pmc_probe.json"),
                    help="where --pmc-probe writes (and --traffic-from reads) the launch list")
    ap.add_argument("--static", choices=["gathered", "packed"],
                    help="time the static baseline instead: one fixed frequency-ranked "
                         "shortlist at every position, gathered from W or from a packed slab")
    ap.add_argument("--static-size", type=int, default=32768,
                    help="tokens on the static list (the pages' static baselines keep ~32K)")
    ap.add_argument("--kmeans", action="store_true",
                    help="time spherical k-means iterations over the workload's LM head instead")
    ap.add_argument("--kmeans-iters", type=int, default=5)
    ap.add_argument("--router-train", action="store_true",
                    help="time router training steps (labels from the dense head + SGD)")
    ap.add_argument("--train-rows", type=int, default=256)
    ap.add_argument("--train-top", type=int, default=64)
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from the host instead of replaying step graphs")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the other full-size workloads after the default one")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--q-mode", choices=("stats", "dense"), default="stats",
                    help="draft sampler output: per-row statistics (verification recomputes "
                         "q; the default) or the q array")
    args = ap.parse_args()

    if args.traffic_from:
        return traffic_from(args)
    if args.overlap_from:
        return overlap_from(args)
    if args.stats_from:
        return stats_from(args)
    if args.kmeans:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        return kmeans_bench(args)
    if args.router_train:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        return router_train_bench(args)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    r = run_draft(args.config, n_steps=args.steps, warmup=args.warmup,
                  instances=args.instances, replicas=not args.no_replicas, eager=args.eager,
                  static=args.static, static_size=args.static_size,
                  pmc_probe_file=args.probe_file if args.pmc_probe else None,
                  q_mode=args.q_mode)
    if r is None:  # --pmc-probe
        return
    cfg, static_ids = r["cfg"], r["static_ids"]
    from dynamic_vocabulary_draft_amd import synthetic as syn
    out = {
        "metric": "gathered-LM-head draft tokens/sec + HBM GB/s (% peak), V=128256 d=4096 bf16",
        "value": r["value"], "unit": "draft tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": r["warmup"],
        "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == syn.DT_BF16 else "f32",
        "data": "synthetic (seeded clustered-Gaussian W, N(0,1) hidden states, N(0,3) target "
                "logits; %d instances rotated)" % args.instances,
        "config": r["config"],
        "step_ms": r["step_ms"],
        "roofline": r["roofline"],
        "head": r["head"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        wl0 = syn.make_workload(args.config, instance=0)
        out["cpu_baseline"] = cpu_baseline(wl0, args.cpu_seconds, static_ids)
        del wl0
    if args.extra and args.config == 1 and not args.static:
        # the other full-size workloads, head and step figures (fewer steps;
        # no W replicas: every head launch there streams >= 1 GB, four times
        # the 256 MB memory-side cache)
        extra = {}
        for k in (2, 3, 4):
            torch.cuda.empty_cache()
            x = run_draft(k, n_steps=args.extra_steps, warmup=4, instances=2, replicas=False,
                          eager=args.eager, q_mode=args.q_mode)
            extra[x["cfg"].name] = {
                "draft_tokens_per_s": x["value"], "ms_per_step": x["ms_per_step"],
                "step_ms": x["step_ms"], "steps": args.extra_steps, "instances": 2,
                "step": x["config"]["step"], "roofline": x["roofline"], "head": x["head"]}
        out["extra"] = extra
    print(json.dumps(out), flush=True)


def run_draft(index, *, n_steps, warmup, instances, replicas, eager, static=None,
              static_size=32768, pmc_probe_file=None, n_ev_max=120, q_mode="stats"):
    """Time n_steps whole draft steps (plus verification) of workload
    `index` and the head kernels inside them; returns the figures (or None
    after a --pmc-probe run)."""
    import numpy as np
    import torch

    from dynamic_vocabulary_draft_amd import native as N
    from dynamic_vocabulary_draft_amd import synthetic as syn
    from dynamic_vocabulary_draft_amd.pipeline import DraftStep, StaticStep, to_dev

    cfg = syn.CONFIGS[index]
    e = cfg.elem_bytes
    t_gen = time.perf_counter()
    cluster_of, _ = syn.make_clusters(cfg)
    W_host = syn.make_lm_head(cfg, cluster_of, threads=min(16, os.cpu_count() or 8))
    log("%s: W generated (%.1f s)" % (cfg.name, time.perf_counter() - t_gen))
    W = to_dev(W_host)
    wls = [syn.make_workload(index, instance=i, with_W=False) for i in range(instances)]
    for wl in wls:
        wl.W = W_host
    static_ids = None
    if static:
        if cfg.is_tree:
            raise SystemExit("--static drafts chains; pick a chain workload")
        static_ids = syn.static_shortlist(cfg, static_size)
        steps = [StaticStep(wl, static_ids, W=W, packed=static == "packed", q_mode=q_mode)
                 for wl in wls]
    else:
        steps = [DraftStep(wl, W=W, q_mode=q_mode) for wl in wls]
    del wls
    npos = 1 if cfg.is_tree else cfg.T
    if replicas and not cfg.is_tree:
        for i, st in enumerate(steps):
            base = st.head_matrix() if static else W
            reps = [base if t == 0 else base.clone() for t in range(npos)]
            st.set_W_positions(reps)
        log("head-matrix replicas: %d x %.2f GB" % (instances * npos,
                                                    reps[0].numel() * e / 1e9))
    del W_host
    torch.cuda.synchronize()

    ev = N.HipEvents()
    stream = torch.cuda.Stream()  # a capturable (non-default) head stream
    warmup = max(warmup, len(steps))  # every instance has run once
    with torch.cuda.stream(stream):
        for k in range(warmup):
            steps[k % len(steps)].step(stream)
    torch.cuda.synchronize()
    log("eager warmup done (%d steps)" % warmup)

    # shortlist sizes per (instance, position): deterministic per instance
    sizes = []
    for st in steps:
        off = st.sl_off.cpu().numpy()
        ids = st.sl_ids.cpu().numpy()
        per = []
        for t in range(npos):
            lo, hi = int(off[t * cfg.B]), int(off[(t + 1) * cfg.B])
            per.append({"total": hi - lo, "union": int(np.unique(ids[lo:hi]).size)})  # rows read
        sizes.append(per)
        assert int(st.err_flag.item()) == 0

    if pmc_probe_file:
        args = argparse.Namespace(probe_file=pmc_probe_file)
        return pmc_probe(args, cfg, steps, sizes, npos, stream, torch, np)
    graphs, mode = [], "eager"
    if not eager:
        # a few graphs per instance, replayed round-robin
        n_graphs = max(len(steps), min(n_steps, 16) // len(steps) * len(steps))
        try:
            for g in range(n_graphs):
                graphs.append(steps[g % len(steps)].capture(stream))
            mode = "hip-graph"
        except Exception as exc:  # noqa: BLE001 - fall back to eager launches
            log("graph capture unavailable (%s); timing eager steps" % exc)
            graphs = []
    if mode == "hip-graph":
        for g in graphs:
            g.launch(stream)
        torch.cuda.synchronize()
        log("captured %d step graphs" % len(graphs))

    def eager_steps(n, with_events):
        sets = [ev.array(2 * npos) if with_events else None for _ in range(n)]
        for k in range(n):
            st = steps[k % len(steps)]
            st.set_head_events(sets[k])
            st.step(stream)
        return sets

    # per-step boundaries on the head stream (torch events see this stream)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record(stream)
    if mode == "hip-graph":
        for k in range(n_steps):
            graphs[k % len(graphs)].launch(stream)
            marks[k + 1].record(stream)
    else:
        ev_sets = []
        for k in range(n_steps):
            st = steps[k % len(steps)]
            sset = ev.array(2 * npos)
            st.set_head_events(sset)
            st.step(stream)
            ev_sets.append(sset)
            marks[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [marks[k].elapsed_time(marks[k + 1]) for k in range(n_steps)]
    log("timed %d steps in %.3f s (%s)" % (n_steps, wall, mode))
    if mode == "hip-graph":
        # HIP cannot time events recorded inside graphs: the head launches
        # are timed on the same steps launched eagerly (same kernels, data)
        n_ev = min(n_steps, n_ev_max)
        torch.cuda.synchronize()
        ev_sets = eager_steps(n_ev, True)
        torch.cuda.synchronize()
        log("timed %d eager steps for the head roofline" % n_ev)
    for st in steps:
        st.set_head_events(None)
        assert int(st.err_flag.item()) == 0

    tokens_per_step = cfg.B * (cfg.tree_nodes if cfg.is_tree else cfg.T)
    hrows = cfg.tree_nodes if cfg.is_tree else 1  # head rows per shortlist
    value = tokens_per_step * n_steps / wall
    durs, nbytes, rows, flops = [], [], [], []
    for k in range(len(ev_sets)):
        i = k % len(steps)
        for t in range(npos):
            durs.append(ev.elapsed_ms(ev_sets[k][2 * t], ev_sets[k][2 * t + 1]))
            sz = sizes[i][t]
            # every needed W row once, the ids, the hidden rows, the logits
            nbytes.append(sz["union"] * cfg.d * e + sz["total"] * 4
                          + cfg.B * hrows * cfg.d * e + sz["total"] * hrows * 4)
            rows.append(sz["total"])
            flops.append(2.0 * hrows * sz["total"] * cfg.d)
    mean_ms = float(np.mean(durs))
    achieved = float(np.sum(nbytes)) / (float(np.sum(durs)) * 1e-3) / 1e9
    traffic = None
    tfile = traffic_file(cfg.name)
    if tfile is not None and os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256") == head_source_sha(head_kernel_name(cfg)) and \
                tr.get("workload") == cfg.name and tr.get("head_kernel") == head_kernel_name(cfg):
            traffic = tr.get("bytes_per_launch")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}
    mfma = cfg.dtype == syn.DT_BF16 and ((hrows == 1 and cfg.B >= 8) or hrows >= 8)
    kname = ("head_gemv_kernel" if not mfma else
             "head_union_kernel (tile index written by the build)" if hrows == 1 else
             "head_gathered_kernel")
    head = {"kernel": kname, "launches_timed": len(durs),
            "mean_us": round(mean_ms * 1e3, 2),
            "p10_us": round(float(np.percentile(durs, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(durs, 90)) * 1e3, 2),
            "mean_rows": round(float(np.mean(rows)), 1),
            "mean_union_rows": round(float(np.mean([s["union"] for p in sizes for s in p])), 1),
            "mean_algorithmic_bytes": round(float(np.mean(nbytes)), 0),
            "hbm_frac": round(achieved / PEAK_HBM_GBS, 4),
            "head_only_tokens_per_s": round(cfg.B * hrows / (mean_ms * 1e-3), 1),
            "w_replicas": bool(replicas and not cfg.is_tree),
            "timed_on": "eager steps (HIP events stamped at each head's own kernel start "
                        "and end)"}
    if hrows >= 8:
        # a real dense contraction: 64 head rows against each gathered row
        tf = float(np.sum(flops)) / (float(np.sum(durs)) * 1e-3) / 1e12
        ai = float(np.sum(flops)) / float(np.sum(nbytes))
        attain = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1e3)
        head.update({"algorithmic_flops": round(float(np.mean(flops)), 0),
                     "tflops": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "flop_per_byte": round(ai, 1),
                     "attainable_tflops": round(attain, 1),
                     "frac_of_attainable": round(tf / attain, 4)})
    for g in graphs:
        g.close()
    for st in steps:
        if hasattr(st, "close"):
            st.close()
    ev.close()
    config = {"workload": cfg.name if static_ids is None else
              "%s, static %s |S|=%d" % (cfg.name, static, static_ids.shape[0]),
              "V": cfg.V, "d": cfg.d, "clusters": cfg.M,
              "batch": cfg.B, "depth": cfg.T, "tree_nodes": cfg.tree_nodes,
              "budget": list(cfg.budget), "router": "%d->%d->%d" % (cfg.d, cfg.r, cfg.M),
              "step": ("router+select+build for the %d roots, gathered head over the "
                       "%d nodes of each tree + sample per node, target softmax over "
                       "the %d nodes + tree verify" % (cfg.B, cfg.tree_nodes,
                                                       cfg.tree_nodes + 1))
                      if cfg.is_tree else
                      ("router+select+build+gathered head+sample per position, "
                       "verify from target logits") if static_ids is None else
                      ("static baseline: %s head over one fixed %d-token frequency-ranked "
                       "shortlist + sample per position, verify from target logits"
                       % (static, static_ids.shape[0])),
              "launch": mode,
              "draft_q": ("row statistics (q recomputed where verification reads it)"
                          if q_mode == "stats" else "written")}
    return {"cfg": cfg, "static_ids": static_ids, "value": round(value, 1), "warmup": warmup,
            "ms_per_step": round(wall * 1e3 / n_steps, 4),
            "step_ms": {"median": round(float(np.median(step_ms)), 4),
                        "p10": round(float(np.percentile(step_ms, 10)), 4),
                        "p90": round(float(np.percentile(step_ms, 90)), 4),
                        "timed_on": "events between consecutive steps on the head stream"},
            "roofline": roof, "head": head, "config": config}


if __name__ == "__main__":
    main()
