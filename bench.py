"""Benchmark: verified tree nodes per second for one DDTree round on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one whole round on one batch of synthetic input: ddtree_build
(log-softmax + top-K + best-first tree + mask), ddtree_verify_attn (tree
attention over the prefix KV) and ddtree_accept (target argmax + walk; with
--target-temp T > 0, ddtree_accept_sample: a sample of the target's softmax at
temperature T per node, then the walk), all enqueued on the current HIP
stream. --commit-kv adds a fourth stage, ddtree_commit_kv (the accepted
path's K/V rows moved behind the prefix, in place); so that the walk
accepts a path, the target logits then carry, at every node, its first
child's token as their maximum. Inputs are resident in HBM before the
timed region; several copies rotate from step to step so that a step's
reads come from HBM rather than from the 256 MB last-level cache (the
default workload's inputs, 1.8 GB per step, exceed it with one copy).

Every timed step replays each stage's captured HIP graph with HIP events
between the stages on the stream the kernels run on, so every stage of
every timed step is event-timed (mean, median, p10, p90 in the JSON line).
With --graph-mode round (small workloads, whose stages are short enough for
host launch time to show between them), one graph holds the whole round and
every 20th timed step runs the stages eagerly with the events between them.

Prints one JSON line. value = sum over requests of (num_nodes - 1) per step
divided by the time per step. The CPU baseline is the oracle, timed on one
thread and on all host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time
import types

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from draft_tree_build_amd import api, synth  # noqa: E402

METRIC = "verified tree nodes/sec (build+tree-attn+accept) and % HBM roofline, 1 GPU"
DEFAULT_WORKLOAD = "B4_L32_V151936_K16_N512_P65536"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
KERNEL_SOURCES = {
    "build": ["draft_tree_build_amd/csrc/k_build.hip", "draft_tree_build_amd/csrc/k_tree.hip"],
    "verify": ["draft_tree_build_amd/csrc/k_attn.hip"],
    "accept": ["draft_tree_build_amd/csrc/k_accept.hip"],
    "accept_sample": ["draft_tree_build_amd/csrc/k_accept.hip"],
    "commit": ["draft_tree_build_amd/csrc/k_commit.hip"],
}
KERNEL_NAMES = {"build": "ddtree_build: k_rows (+ k_rows_sum for split rows), k_tree",
                "verify": "ddtree_verify_attn: k_attn_mfma (+ k_v_f16 before it when many row tiles "
                          "share each V tile, + k_attn_combine for split keys)",
                "accept": "ddtree_accept: k_argmax, k_walk",
                "accept_sample": "ddtree_accept_sample: k_sample, k_walk",
                "commit": "ddtree_commit_kv: k_commit"}
SAMPLE_SEED = 0x5EED
LLC_BYTES = 256 * 2**20        # MI355X last-level (Infinity) cache


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def algorithmic_work(w, prefix_lens, num_nodes, depths, esize, moved_rows=0):
    """Bytes (and flops) each stage must move per step, by its definition;
    moved_rows: accepted K/V rows not already in place (commit stage)."""
    B, L, V, K, T = w.batch, w.L, w.V, w.K, w.T
    W = (T + 63) // 64
    build_bytes = B * L * V * esize + B * L * K * 8 + B * T * (4 * 4 + W * 8)
    P = [int(p) for p in prefix_lens]
    kv_rows = sum(P) + B * T
    verify_bytes = kv_rows * w.Hkv * w.D * esize * 2 + B * T * w.Hq * w.D * esize * 2 + B * T * W * 8
    # QK^T and PV over the prefix, plus each node's ancestors (depth + 1 keys)
    anc = sum(int(depths[b][i]) + 1 for b in range(B) for i in range(int(num_nodes[b])))
    verify_flops = 4.0 * w.Hq * w.D * sum(T * p for p in P)
    verify_flops += 4.0 * w.Hq * w.D * anc
    accept_bytes = sum(int(n) for n in num_nodes) * V * esize
    commit_bytes = moved_rows * w.Hkv * w.D * esize * 2 * 2 + B * (8 + 4 * (4 + L) + 8)
    return dict(build_bytes=build_bytes, verify_bytes=verify_bytes, verify_flops=verify_flops,
                accept_bytes=accept_bytes, commit_bytes=commit_bytes)


def source_hash(rels):
    """Hash of the code of the given sources: comments and whitespace are
    removed first, so that an edit of the text alone keeps the counters."""
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel)) as f:
            code = f.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload, stage):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload, {}).get(stage)
    if not ent or ent.get("source_sha") != source_hash(KERNEL_SOURCES[stage]):
        return None
    return ent.get("bytes_per_launch")


def measured_peaks(dev):
    """Peaks measured on this device, outside the timed region, for the
    roofline fractions beside the published ones: HBM = bytes per second of
    one streaming read of 4 GiB (ddtree_probe_hbm_read; a 1 GiB device copy,
    read plus written bytes, is reported beside it); MFMA = bf16 flops per
    second of a dense v_mfma_f32_32x32x16_bf16 loop (ddtree_probe_mfma_bf16,
    two workgroups per compute unit)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    grid = 8 * cus
    fold = torch.empty(grid, dtype=torch.int32, device=dev)
    hbm_read = n / timed(lambda: api.ddtree_probe_hbm_read(src, fold, grid), 10) / 1e9
    a, b = src[: 1 << 30], src[1 << 30: 2 << 30]
    hbm_copy = 2.0 * (1 << 30) / timed(lambda: b.copy_(a), 10) / 1e9
    del src, fold, a, b
    grid, iters = 2 * cus, 4096
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    mfma = grid * 4 * 4 * iters * 32768.0 / timed(
        lambda: api.ddtree_probe_mfma_bf16(out, grid, iters), 5) / 1e12
    del out
    torch.cuda.empty_cache()
    return {"hbm_GBs": round(hbm_read, 1), "hbm_how": "streaming read of 4 GiB (ddtree_probe_hbm_read)",
            "hbm_copy_GBs": round(hbm_copy, 1),
            "bf16_mfma_TFs": round(mfma, 1),
            "bf16_mfma_how": "v_mfma_f32_32x32x16_bf16 loop, 4 chains per wave, 2 workgroups per CU "
                             "(ddtree_probe_mfma_bf16)"}


def stage_rooflines(work, stage_us, peaks):
    """Each stage's algorithmic work over its event time, against the
    published peak and the measured one, on its binding roofline."""
    out = {}
    for name, us in stage_us.items():
        t_s = us * 1e-6
        if name == "verify":
            t_mem = work["verify_bytes"] / (HBM_PEAK_GBS * 1e9)
            t_mma = work["verify_flops"] / (MFMA_BF16_PEAK_TFS * 1e12)
        else:
            t_mem, t_mma = 1.0, 0.0
        if t_mma > t_mem:
            ach = work["verify_flops"] / t_s / 1e12
            rec = dict(bound="mfma", unit="TFLOP/s", peak=MFMA_BF16_PEAK_TFS,
                       peak_measured=peaks["bf16_mfma_TFs"] if peaks else None)
        else:
            ach = work[name + "_bytes"] / t_s / 1e9
            rec = dict(bound="hbm", unit="GB/s", peak=HBM_PEAK_GBS,
                       peak_measured=peaks["hbm_GBs"] if peaks else None)
        rec["achieved"] = round(ach, 3)
        rec["frac"] = round(ach / rec["peak"], 5)
        rec["frac_measured"] = round(ach / rec["peak_measured"], 5) if rec["peak_measured"] else None
        rec["us"] = round(us, 3)
        out[name] = rec
    return out


def _pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    pos = (len(xs) - 1) * q
    lo, hi = int(math.floor(pos)), int(math.ceil(pos))
    return xs[lo] + (xs[hi] - xs[lo]) * (pos - lo)


def _summary(xs):
    return {"mean": round(sum(xs) / len(xs), 3), "median": round(_pct(xs, 0.5), 3),
            "p10": round(_pct(xs, 0.1), 3), "p90": round(_pct(xs, 0.9), 3), "n": len(xs)}


def cpu_baseline(w, inputs, nodes_per_step, target_temp, attn_seconds):
    """The oracle as it stands (plain C, not tuned), on the same host tensors:
    the whole build and the whole accept of one round, and the tree
    attention of a seeded sample of the round's valid query rows, scaled to
    all of them (a row's cost is its key count: the prefix plus the node's
    ancestors). Timed twice: on one thread, and on all the host cores this
    process may use (the oracle spreads independent drafter rows, requests,
    query rows and target rows over OpenMP threads; its arithmetic does not
    change). The sample is sized so that the one-thread attention takes
    about attn_seconds."""
    import numpy as np
    import oracle
    x, roots, q, k, v, P, offs, tl = inputs
    tau = w.taus[0]
    cores = oracle.host_cores()
    tree = oracle.build_tree(x, roots, w.K, w.N, tau)
    valid = [(b, i, h) for b in range(w.batch) for i in range(int(tree["num_nodes"][b]))
             for h in range(w.Hq)]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(valid))
    scale = 1.0 / math.sqrt(w.D)

    def attn(sel):
        t0 = time.perf_counter()
        oracle.attn_rows(q, k, v, offs, P, tree["num_nodes"], tree["mask"], w.T, w.Hq, w.Hkv,
                         w.D, scale, sel)
        return time.perf_counter() - t0

    # size the sample: the one-thread cost of a few rows
    probe = [valid[j] for j in order[:min(8, len(valid))]]
    per_row = attn(probe) / len(probe)
    nsamp = int(min(len(valid), max(16, attn_seconds / max(per_row, 1e-9))))
    sel = [valid[j] for j in order[:nsamp]]
    res = {}
    for nt in sorted({1, cores}):
        with oracle.threads(nt):
            t0 = time.perf_counter()
            tr = oracle.build_tree(x, roots, w.K, w.N, tau)
            t_build = time.perf_counter() - t0
            t_attn = attn(sel)
            t0 = time.perf_counter()
            if target_temp > 0:
                oracle.accept_sample(tl, tr["tokens"], tr["parents"], tr["num_nodes"], w.L,
                                     target_temp, SAMPLE_SEED, 0)
            else:
                oracle.accept(tl, None, tr["tokens"], tr["parents"], tr["num_nodes"], w.L)
            t_accept = time.perf_counter() - t0
        t_round = t_build + t_attn * len(valid) / len(sel) + t_accept
        res[nt] = dict(value=round(nodes_per_step / t_round, 3), round_s=round(t_round, 4),
                       build_s=round(t_build, 4), accept_s=round(t_accept, 4),
                       attn_sample_s=round(t_attn, 4))
    acc = "sampled accept at target temperature %g" % target_temp if target_temp > 0 else "greedy accept"
    return dict(
        value=res[cores]["value"], unit="nodes/s", cores=cores, kind="oracle",
        value_1thread=res[1]["value"],
        sample="one round of %s: the whole build and %s, and the tree attention of %d of the "
               "round's %d valid query rows (seeded sample), its time scaled by %d/%d; timed on "
               "%d thread(s) (value) and on 1 thread (value_1thread)"
               % (w.name, acc, len(sel), len(valid), len(valid), len(sel), cores),
        timings={("%d_threads" % nt): r for nt, r in res.items()})


def measure(w, args, dev):
    """Time whole rounds of workload w (the timed region of the contract);
    returns the measurement and what the report needs."""
    tau = w.taus[0]
    log("workload %s: generating inputs" % w.name)
    x_cpu, _ = synth.drafter_logits(w)
    roots_cpu = synth.root_tokens(w)
    P_cpu = synth.prefix_lengths(w)
    offs_cpu = synth.kv_offsets(P_cpu, w.T)
    q_cpu, k_cpu, v_cpu = synth.qkv(w, P_cpu)
    tl_cpu = synth.target_logits(w)
    esize = 2 if w.dtype == "bf16" else 4
    if args.commit_kv:
        # the drafted tree does not depend on the target: build it once, then
        # give every node's first child's token the largest target logit
        probe = api.Round(w.batch, w.L, w.V, w.K, w.N, dev)
        probe.build(x_cpu.to(dev), roots_cpu.to(dev), tau)
        torch.cuda.synchronize()
        toks, pars = probe.tokens.cpu(), probe.parents.cpu()
        nn_cpu = probe.num_nodes.cpu()
        del probe
        for b in range(w.batch):
            planted = set()
            for c in range(1, int(nn_cpu[b])):
                p = int(pars[b, c])
                if p not in planted:                    # first child only: one maximum per row
                    planted.add(p)
                    tl_cpu[b, p, int(toks[b, c])] = 100.0   # logits are ~N(0, sigma <= 3)
    step_bytes = sum(t.numel() * t.element_size() for t in (x_cpu, q_cpu, k_cpu, v_cpu, tl_cpu))
    R = 1
    if args.rotate_mb > 0:
        R = max(1, min(64, math.ceil(args.rotate_mb * 2**20 / step_bytes)))
        free = torch.cuda.mem_get_info(dev)[0]
        R = max(1, min(R, int(0.5 * free // step_bytes)))
    log("%d input cop%s of %.1f MB" % (R, "y" if R == 1 else "ies", step_bytes / 1e6))
    copies = []
    for _ in range(R):
        copies.append(tuple(t.to(dev) for t in (x_cpu, q_cpu, k_cpu, v_cpu, tl_cpu)))
    roots = roots_cpu.to(dev)
    P = P_cpu.to(dev)
    offs = offs_cpu.to(dev)
    rnd = api.Round(w.batch, w.L, w.V, w.K, w.N, dev, w.Hq, w.Hkv, w.D, int(w.prefix[1]),
                    dtype=w.torch_dtype)

    if args.commit_kv:
        rnd.prepare_commit()
    stages = (
        lambda c: rnd.build(c[0], roots, tau),
        lambda c: rnd.verify(c[1], c[2], c[3], offs, P),
        (lambda c: rnd.accept_sample(c[4], args.target_temp, SAMPLE_SEED, 0))
        if args.target_temp > 0 else (lambda c: rnd.accept(c[4])),
    ) + ((lambda c: rnd.commit(c[2], c[3], offs, P),) if args.commit_kv else ())
    stage_names = ("build", "verify", "accept", "commit")[:len(stages)]
    accept_kind = "accept_sample" if args.target_temp > 0 else "accept"

    log("warmup %d steps (eager)" % args.warmup)
    for i in range(args.warmup):
        for f in stages:
            f(copies[i % R])
    torch.cuda.synchronize()
    num_nodes = rnd.num_nodes.cpu()
    nodes_per_step = int((num_nodes - 1).sum())

    # Per input copy and stage, one captured HIP graph (the stage's kernels
    # with no host launch overhead between them). Every timed step replays
    # the stages' graphs in order on the current stream with an event before
    # the first and after each: the events time every stage of every timed
    # step on the stream the kernels run on. --no-graphs launches the ABI
    # calls directly instead, with the same events.
    # --graph-mode round (small workloads, where host launch time would
    # show between stages): one graph per copy holds the whole round; every
    # 20th timed step instead calls the ABI functions directly with the
    # events between them (the replays queued ahead keep the GPU busy).
    graphs = None
    per_stage = args.graphs and args.graph_mode == "stage"
    if args.graphs:
        log("capturing %d x %d graph(s)" % (R, len(stages) if per_stage else 1))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        with torch.cuda.stream(side):
            for c in range(R):
                row = []
                for f in (stages if per_stage else (lambda cc: [g(cc) for g in stages],)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        f(copies[c])
                    row.append(g)
                graphs.append(row)
        torch.cuda.current_stream().wait_stream(side)
        for i in range(min(R, max(1, args.warmup))):
            for g in graphs[i]:
                g.replay()
        torch.cuda.synchronize()

    every = 1 if (graphs is None or per_stage) else 20
    timed = [i for i in range(args.steps) if i % every == every - 1] or [args.steps - 1]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for i in timed}
    log("timing %d steps (stage events on %d)" % (args.steps, len(timed)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        c = i % R
        ev = evs.get(i)
        if ev is None:
            graphs[c][0].replay()
            continue
        ev[0].record()
        for k in range(len(stages)):
            if per_stage:
                graphs[c][k].replay()
            else:
                stages[k](copies[c])
            ev[k + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    stage_samples = {name: [evs[i][k].elapsed_time(evs[i][k + 1]) * 1e3 for i in timed]
                     for k, name in enumerate(stage_names)}
    step_samples = [evs[i][0].elapsed_time(evs[i][-1]) * 1e3 for i in timed]
    stage_us = {k: sum(v) / len(v) for k, v in stage_samples.items()}
    value = nodes_per_step / (ms_per_step * 1e-3)
    log("ms/step %.4f  stages(us, mean) %s" % (ms_per_step, {k: round(v, 2) for k, v in stage_us.items()}))
    return types.SimpleNamespace(
        w=w, tau=tau, x_cpu=x_cpu, roots_cpu=roots_cpu, P_cpu=P_cpu, offs_cpu=offs_cpu,
        q_cpu=q_cpu, k_cpu=k_cpu, v_cpu=v_cpu, tl_cpu=tl_cpu, esize=esize, R=R, rnd=rnd,
        stage_us=stage_us, stage_stats={k: _summary(v) for k, v in stage_samples.items()},
        step_stats=_summary(step_samples), value=value, ms_per_step=ms_per_step,
        nodes_per_step=nodes_per_step, num_nodes=num_nodes, accept_kind=accept_kind,
        step_bytes=step_bytes)


def budget_sweep(w, args, dev, budgets):
    """Whole rounds of workload w at each node budget N (the cost side of the
    budget trade-off): one JSON line with a record per budget."""
    recs = []
    for N in budgets:
        wn = dataclasses.replace(w, N=N, name="%s@N%d" % (w.name, N))
        m = measure(wn, args, dev)
        recs.append({"N": N, "ms_per_step": round(m.ms_per_step, 5),
                     "nodes_per_step": m.nodes_per_step, "value": round(m.value, 1),
                     "stages_us": {k: round(v, 3) for k, v in m.stage_us.items()}})
        del m
        torch.cuda.empty_cache()
    out = {"metric": "round time vs node budget (build+tree-attn+accept), 1 GPU", "unit": "ms",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
           "dtype": w.dtype, "data": "synthetic (seeded)",
           "config": {"workload": w.name, "batch": w.batch, "L": w.L, "V": w.V, "K": w.K,
                      "prefix": list(w.prefix), "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                      "target_temp": args.target_temp, "hip_graphs": bool(args.graphs),
                      "graph_mode": args.graph_mode},
           "sweep": recs}
    print(json.dumps(out), flush=True)


def summarize_traffic(fetch_csv, write_csv, workload, commands):
    """HBM bytes per launch of every stage from two rocprofv3 counter runs of
    this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled
    by what the same counter reads for the plain 256 MiB device copy that
    --copy-probe runs in the same process. Writes profiles/traffic.json
    (keyed by workload and stage, with a hash of the kernel sources) and
    profiles/traffic_<workload>.txt."""
    import collections
    import csv
    import statistics

    def load(path, counter):
        d = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                n = r["Kernel_Name"].replace("ddt::(anonymous namespace)::", "")
                n = n.split("(")[0].replace("void ", "")
                d[n].append(float(r["Counter_Value"]))
        return d

    F, Wr = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = [n for n in F if "copyBuffer" in n]
    if not copy:
        raise SystemExit("no device copy in the FETCH_SIZE run: profile with --copy-probe")
    cf, cw = max(F[copy[0]]), max(Wr[copy[0]])
    copy_kib = 256 * 1024
    ff, wf = copy_kib / cf, copy_kib / cw
    stages = {"build": ["k_rows", "k_rows_sum", "k_tree", "k_tree_level"],
              "verify": ["k_v_f16", "k_attn_mfma", "k_attn_combine", "k_attn_simple"],
              "accept": ["k_argmax", "k_walk"], "accept_sample": ["k_sample"],
              "commit": ["k_commit"]}
    res = {}
    for stage, prefixes in stages.items():
        ks, fsum, wsum = {}, 0.0, 0.0
        for n in F:
            if n.split("<")[0] in prefixes:
                fv, wv = statistics.mean(F[n]), statistics.mean(Wr.get(n, [0.0]))
                ks[n] = {"fetch_kib_raw": round(fv, 1), "write_kib_raw": round(wv, 1)}
                fsum += fv
                wsum += wv
        if not ks:
            continue
        res[stage] = {"bytes_per_launch": int(round((fsum * ff + wsum * wf) * 1024)),
                      "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                      "fetch_kib_raw": round(fsum, 1), "write_kib_raw": round(wsum, 1),
                      "kernels": ks, "source_sha": source_hash(KERNEL_SOURCES[stage])}
    if "accept_sample" in res and "accept" in res:       # k_walk serves both
        res["accept_sample"]["bytes_per_launch"] += int(round(
            sum(v["fetch_kib_raw"] * ff + v["write_kib_raw"] * wf
                for n, v in res["accept"]["kernels"].items() if n.startswith("k_walk")) * 1024))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            allres = json.load(f)
    except (OSError, ValueError):
        allres = {}
    allres[workload] = res
    with open(path, "w") as f:
        json.dump(allres, f, indent=1, sort_keys=True)
    with open(os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload), "w") as f:
        f.write("HBM traffic per launch, workload %s (rocprofv3 counters, KiB per dispatch "
                "averaged over dispatches)\n\n" % workload)
        f.write("commands (from /tmp, TMPDIR=/tmp, REPO = repository root):\n%s\n"
                "summary: python bench.py --workload %s --summarize-traffic FETCH_CSV WRITE_CSV\n\n"
                % ("".join("  %s\n" % c for c in commands.split(" ;; ") if c), workload))
        f.write("calibration: the 256 MiB device copy run by --copy-probe reads FETCH_SIZE %.0f KiB "
                "and WRITE_SIZE %.0f KiB;\nscale factors fetch %.4f, write %.4f (bytes moved / "
                "counter)\n\n" % (cf, cw, ff, wf))
        f.write("%-52s %12s %12s %14s\n" % ("kernel", "FETCH_KiB", "WRITE_KiB", "scaled_MB"))
        for stage in res:
            for n, v in sorted(res[stage]["kernels"].items()):
                f.write("%-52s %12.1f %12.1f %14.3f\n" % (
                    n[:52], v["fetch_kib_raw"], v["write_kib_raw"],
                    (v["fetch_kib_raw"] * ff + v["write_kib_raw"] * wf) * 1024 / 1e6))
        f.write("\n")
        for stage in res:
            f.write("stage %-13s scaled bytes per launch: %d\n" % (stage, res[stage]["bytes_per_launch"]))
    print(json.dumps({k: v["bytes_per_launch"] for k, v in res.items()}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(synth.WORKLOADS))
    ap.add_argument("--rotate-mb", type=int, default=768,
                    help="rotate input copies until their total exceeds this (0: one copy)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="one-thread seconds of the oracle's attention sample (CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graphs", dest="graphs", action="store_false",
                    help="launch the ABI calls eagerly instead of replaying captured HIP graphs")
    ap.add_argument("--graph-mode", choices=("stage", "round"), default="stage",
                    help="stage: one graph per stage, events between stages on every timed step; "
                         "round: one graph per round (no host time between stages; for small "
                         "workloads), every 20th timed step event-timed per stage")
    ap.add_argument("--target-temp", type=float, default=0.0,
                    help="target temperature of the acceptance (0: greedy arg-max; > 0: "
                         "ddtree_accept_sample)")
    ap.add_argument("--commit-kv", action="store_true",
                    help="add the KV compaction of the accepted path as a fourth stage (target "
                         "logits then lead the walk down first children)")
    ap.add_argument("--budgets", default="",
                    help="comma-separated node budgets N: time whole rounds at each (one JSON "
                         "line with a record per budget) instead of the single measurement")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--no-peak-probe", dest="peak_probe", action="store_false",
                    help="skip measuring the device's copy bandwidth and bf16 GEMM rate")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and "
                         "a WRITE_SIZE rocprofv3 run of this script (with --copy-probe) into "
                         "profiles/traffic.json and a text summary for --workload")
    ap.add_argument("--commands", default="",
                    help="with --summarize-traffic: the commands that made the runs (recorded)")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.workload,
                          args.commands)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)
    api.lib()  # fail loudly if the library is not built

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.budgets:
        budget_sweep(w, args, dev, [int(x) for x in args.budgets.split(",")])
        return
    m = measure(w, args, dev)
    (tau, x_cpu, roots_cpu, P_cpu, offs_cpu, q_cpu, k_cpu, v_cpu, tl_cpu, esize, R, rnd, stage_us,
     value, ms_per_step, nodes_per_step, num_nodes, accept_kind) = (
        m.tau, m.x_cpu, m.roots_cpu, m.P_cpu, m.offs_cpu, m.q_cpu, m.k_cpu, m.v_cpu, m.tl_cpu,
        m.esize, m.R, m.rnd, m.stage_us, m.value, m.ms_per_step, m.nodes_per_step, m.num_nodes,
        m.accept_kind)

    if args.copy_probe:
        a = torch.empty(256 * 2**20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    moved = 0
    if args.commit_kv:
        alen, anodes = rnd.accept_len.cpu().tolist(), rnd.accepted_nodes.cpu().tolist()
        moved = sum(1 for b in range(w.batch) for k in range(alen[b]) if anodes[b][k] != k + 1)
        log("accepted %s, %d rows moved per step" % (alen[:8], moved))
    work = algorithmic_work(w, P_cpu.tolist(), num_nodes.tolist(), rnd.depths.cpu().tolist(), esize,
                            moved)
    dom = max(stage_us, key=stage_us.get)
    t_s = stage_us[dom] * 1e-6
    if dom == "verify":
        t_mem = work["verify_bytes"] / (HBM_PEAK_GBS * 1e9)
        t_mma = work["verify_flops"] / (MFMA_BF16_PEAK_TFS * 1e12)
        if t_mma > t_mem:
            achieved, peak, unit, bound = work["verify_flops"] / t_s / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = work["verify_bytes"] / t_s / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    else:
        nbytes = work[dom + "_bytes"]
        achieved, peak, unit, bound = nbytes / t_s / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    kname = accept_kind if dom == "accept" else dom
    peaks = None
    if args.peak_probe:
        log("measuring device peaks (HBM read stream, bf16 MFMA loop)")
        try:
            peaks = measured_peaks(dev)
        except (RuntimeError, torch.cuda.OutOfMemoryError) as e:  # the benchmark line stands without them
            log("device peaks not measured: %s" % e)
            torch.cuda.empty_cache()
    stages_rl = stage_rooflines(work, stage_us, peaks)
    roofline = dict(bound=bound, achieved=round(achieved, 3), peak=peak, unit=unit,
                    frac=round(achieved / peak, 5), traffic=load_traffic(w.name, kname),
                    kernel=KERNEL_NAMES[kname], stage=kname,
                    avg_launch_us=round(stage_us[dom], 3),
                    peak_measured=stages_rl[dom]["peak_measured"],
                    frac_measured=stages_rl[dom]["frac_measured"])

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (one thread and all cores)")
        inputs = (x_cpu, roots_cpu, q_cpu, k_cpu, v_cpu, P_cpu.numpy(), offs_cpu.numpy(), tl_cpu)
        cpu = cpu_baseline(w, inputs, nodes_per_step, args.target_temp, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; drafter/target logits ~N(0,sigma) with planted peaks, "
                "Q/K/V ~N(0,1))",
        "config": {"workload": w.name, "batch": w.batch, "L": w.L, "V": w.V, "K": w.K, "N": w.N,
                   "prefix": list(w.prefix), "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "draft_temp": tau, "target_temp": args.target_temp,
                   "commit_kv": bool(args.commit_kv), "input_copies": R,
                   "hip_graphs": bool(args.graphs), "graph_mode": args.graph_mode,
                   "stage_event_steps": m.stage_stats["build"]["n"],
                   "cache": "cold" if R > 1 or m.step_bytes > LLC_BYTES else "warm",
                   "step_input_MB": round(m.step_bytes / 1e6, 1)},
        "stages_us": {k: round(v, 3) for k, v in stage_us.items()},
        "stages_us_stats": m.stage_stats,
        "step_us_stats": m.step_stats,
        "roofline": roofline,
        "stages_roofline": stages_rl,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
