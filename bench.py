#!/usr/bin/env python3
"""Draft-tree construction benchmark on one MI355X.

One step = the whole hot path over one batch of the batch-64 workload
(64 requests x 15 draft positions x V = 151936 bf16 logits, node budget 128):
  stage 1  ddtree_row_topk  per-row log-sum-exp + sorted top-128 (HBM-bound)
  stage 2+3 ddtree_select   top-128 prefix tree + bit-packed ancestor mask
  stage 4  ddtree_accept    greedy walk against per-node target tokens
Inputs are synthetic (draft_tree_construction_depth_amd.gen), already resident
in HBM; four copies of the batch rotate so that the 256 MB Infinity Cache
cannot serve repeated reads. Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft trees/sec at batch 64, V=151936, L=15, B=128; achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
KERNEL_SAMPLES = 100  # event-timed launches of stage 1 and of the read probe
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_stage1_batch64.json")
STAGE1_SOURCES = ["draft_tree_construction_depth_amd/csrc/stage1.hpp",
                  "draft_tree_construction_depth_amd/csrc/common.hpp"]


def stage1_source_hash() -> str:
    h = hashlib.sha256()
    for p in STAGE1_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per stage-1 launch from committed rocprofv3 counters, or None
    when the counters were taken on a different version of the kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != stage1_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, Y, B, L, sample_1core: int = 8):
    """The oracle as it stands, timed on this host: the whole batch at the
    host's CPU share (threads over requests), and a sample of requests on one
    core. Returns (report, oracle trees of the whole batch with tables)."""
    from draft_tree_construction_depth_amd import gen
    from oracle import oracle as O
    if not os.path.exists(O.LIB):
        O.build_oracle()
    visible = len(os.sched_getaffinity(0))
    # the host's CPU share for one GPU is 16 threads, whatever more it shows
    threads = max(1, min(visible, 16))

    def run(xs, T):
        t0 = time.perf_counter()
        o = O.build(xs, gen.DTYPE_BF16, B, threads=T, tables=True)
        O.mask(o["parents"], o["num_nodes"], B)
        t1 = time.perf_counter()
        tgt = gen.node_targets_from_depths(Y[:xs.shape[0]], o["depths"], o["num_nodes"], B)
        t2 = time.perf_counter()
        O.accept(o["tree_tokens"], o["parents"], o["num_nodes"], tgt, L)
        t3 = time.perf_counter()
        return (t1 - t0) + (t3 - t2), o

    secs, o = run(x, threads)
    n1 = min(sample_1core, x.shape[0])
    secs1, _ = run(x[:n1], 1)
    n = x.shape[0]
    rep = {"value": n / secs, "unit": "trees/s", "cores": threads, "kind": "oracle",
           "sample": f"all {n} requests of one batch (build + mask + accept), {secs:.2f} s",
           "value_1core": n1 / secs1,
           "sample_1core": f"the first {n1} requests on one thread, {secs1:.2f} s",
           "host_cpus_visible": visible, "cpu_model": cpu_model()}
    return rep, o


def parity_of_run(g: dict, o: dict, tgt, B: int, L: int) -> dict:
    """The benchmark's own trees against the oracle's: tree classes (oracle/
    parity.py), masks (of the device's parents) and walks (on the device's
    trees, same targets) bit for bit."""
    import numpy as np

    from oracle import oracle as O
    from oracle.parity import ddtree_batch_counts
    res = ddtree_batch_counts(g, o, B)
    counts = {k: res["counts"].get(k, 0) for k in ("exact", "E1", "E2", "F")}
    m_ok = np.array_equal(g["mask"], O.mask(g["parents"], g["num_nodes"], B))
    oa = O.accept(g["tree_tokens"], g["parents"], g["num_nodes"], tgt, L)
    w_ok = all(np.array_equal(a, b) for a, b in zip(
        (g["accepted_nodes"], g["accept_len"], g["next_token"]), oa))
    return {**counts, "masks_bit_exact": bool(m_ok), "walks_bit_exact": bool(w_ok),
            "requests": int(len(o["num_nodes"]))}


def read_ceiling(pkg, torch, bufs, rows, row_bytes, n):
    """Event-timed launches of the read probe over the same rotated buffers:
    GB/s of stage 1's load path with nothing computed."""
    sink = torch.empty((rows, 4), dtype=torch.int32, device=bufs[0].device)
    for i in range(3):
        pkg.ddtree_read_probe(bufs[i % len(bufs)], rows, row_bytes, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record()
        pkg.ddtree_read_probe(bufs[i % len(bufs)], rows, row_bytes, sink)
        b.record()
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
    return rows * row_bytes / (us * 1e-6) / 1e9, us


def treespark_bench(args) -> int:
    """TreeSpark parent-conditioned expansion: 32 requests x 7 depths over
    V = 151936 with a 2560-wide head; one step = one treespark_expand call."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.TREESPARK
    batch, D, V, H, k, F, N = (c[x] for x in ("batch", "D", "V", "H", "k", "F", "N"))
    bb, W, E, anc = gen.treespark_inputs(0)
    dev = torch.device("cuda:0")
    as_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    bbd, Wd, Ed = as_bf16(bb), as_bf16(W), as_bf16(E)
    ancd = torch.from_numpy(anc).to(dev)
    out = pkg.treespark_expand(bbd, Wd, Ed, ancd, k=k, F=F, N=N)
    for _ in range(args.warmup):
        pkg.treespark_expand(bbd, Wd, Ed, ancd, k=k, F=F, N=N, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        pkg.treespark_expand(bbd, Wd, Ed, ancd, k=k, F=F, N=N, out=out)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / args.steps
    # parents per depth: 1 per request at depth 1, then min(F, previous * k)
    fd, Ms = 1, []
    for _ in range(D):
        Ms.append(batch * fd)
        fd = min(F, fd * k)
    w_bytes = V * H * 2
    alg_bytes = D * w_bytes + batch * D * V * 2 + sum(Ms) * H * 2
    flops = sum(2.0 * V * H * m for m in Ms)
    res = {
        "metric": "TreeSpark trees/sec at batch 32, 7 depths, V=151936, H=2560, k=4, N=32",
        "value": round(batch / (ms / 1e3), 1), "unit": "trees/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/f32",
        "data": "synthetic",
        "config": {"workload": "treespark_batch32_D7_V151936_H2560_k4_F4_N32", "batch": batch,
                   "D": D, "V": V, "H": H, "k": k, "F": F, "N": N},
        "algorithmic_gbps": round(alg_bytes / (ms / 1e3) / 1e9, 1),
        "hbm_frac": round(alg_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
        "mfma_tflops": round(flops / (ms / 1e3) / 1e12, 1),
        "mfma_frac_bf16": round(flops / (ms / 1e3) / 2.5e15, 4),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(res), flush=True)
    return 0


def sparkling_bench(args) -> int:
    """SparklingTree conditioned tree: 64 requests x 15 drafter rows over
    V = 151936, top C = 128 per row, rank-256 Markov head, B = 64 nodes; one
    step = one sparkling_build call (top-C rows, Markov-delta table,
    selection + mask). Two copies of the logits rotate."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.SPARKLING
    batch, L, V, B, C, R = (c[x] for x in ("batch", "L", "V", "B", "C", "R"))
    x, W1, W2t = gen.sparkling_inputs(0)
    dev = torch.device("cuda:0")
    as_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    xs = [as_bf16(x), as_bf16(gen.sparkling_inputs(1)[0])]
    W1d, W2d = as_bf16(W1), as_bf16(W2t)
    out = pkg.sparkling_build(xs[0], W1d, W2d, B, C=C)
    for i in range(args.warmup):
        pkg.sparkling_build(xs[i % 2], W1d, W2d, B, C=C, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(args.steps):
        pkg.sparkling_build(xs[i % 2], W1d, W2d, B, C=C, out=out)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / args.steps
    # logits once; per conditioned row block: C rows of W1 and of W2t, the C x C
    # float log-probs written; the selection's reads of visited rows are not counted
    blocks = batch * (L - 1)
    alg_bytes = batch * L * V * 2 + blocks * (2 * C * R * 2 + C * C * 4 + C * 5)
    res = {
        "metric": "SparklingTree trees/sec at batch 64, L=15, V=151936, C=128, R=256, B=64",
        "value": round(batch / (ms / 1e3), 1), "unit": "trees/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/f32/f64", "data": "synthetic",
        "config": {"workload": "sparkling_batch64_L15_V151936_C128_R256_B64", "batch": batch,
                   "L": L, "V": V, "C": C, "R": R, "B": B, "input_buffers": 2},
        "algorithmic_gbps": round(alg_bytes / (ms / 1e3) / 1e9, 1),
        "hbm_frac": round(alg_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
        "wall_s": round(wall, 3),
    }
    print(json.dumps(res), flush=True)
    return 0


def beam_bench(args) -> int:
    """Beam tree on SparklingTree's rows: the --sparkling workload with the
    budget B = 64 spread evenly over the 15 depths; one step = one
    sparkling_beam call (top-C rows, Markov-delta table, beam + mask)."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.SPARKLING
    batch, L, V, B, C, R = (c[x] for x in ("batch", "L", "V", "B", "C", "R"))
    x, W1, W2t = gen.sparkling_inputs(0)
    dev = torch.device("cuda:0")
    as_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    xs = [as_bf16(x), as_bf16(gen.sparkling_inputs(1)[0])]
    W1d, W2d = as_bf16(W1), as_bf16(W2t)
    out = pkg.sparkling_beam(xs[0], W1d, W2d, B=B, C=C)
    for i in range(args.warmup):
        pkg.sparkling_beam(xs[i % 2], W1d, W2d, B=B, C=C, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(args.steps):
        pkg.sparkling_beam(xs[i % 2], W1d, W2d, B=B, C=C, out=out)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / args.steps
    res = {
        "metric": "beam trees/sec at batch 64, L=15, V=151936, C=128, R=256, B=64 spread evenly",
        "value": round(batch / (ms / 1e3), 1), "unit": "trees/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16/f32/f64", "data": "synthetic",
        "config": {"workload": "beam_batch64_L15_V151936_C128_R256_B64_even", "batch": batch,
                   "L": L, "V": V, "C": C, "R": R, "widths": "even (library default)",
                   "input_buffers": 2},
        "wall_s": round(wall, 3),
    }
    print(json.dumps(res), flush=True)
    return 0


def dspark_bench(args) -> int:
    """DSpark's verification budget over 256 active requests with blocks of
    16 guesses (4096 slots), cost 25 ms + 0.1 ms per verified token; one
    step = one dspark_budget call (survival, ranking, budget, lengths)."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.DSPARK
    batch, P = c["batch"], c["P"]
    conf, cost = gen.dspark_inputs(0)
    dev = torch.device("cuda:0")
    cd, kd = torch.from_numpy(conf).to(dev), torch.from_numpy(cost).to(dev)
    out = pkg.dspark_budget(cd, kd)
    for _ in range(args.warmup):
        pkg.dspark_budget(cd, kd, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        pkg.dspark_budget(cd, kd, out=out)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / args.steps
    res = {
        "metric": "DSpark budget decisions/sec at 256 requests x 16 guesses",
        "value": round(1e3 / ms, 1), "unit": "decisions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "dspark_budget_batch256_P16", "batch": batch, "P": P,
                   "cost": "25 ms + 0.1 ms per token"},
        "n_keep": int(out["n_keep"].item()), "wall_s": round(wall, 3),
    }
    print(json.dumps(res), flush=True)
    return 0


def latency_bench(args) -> int:
    """Single-request latency (batch 1, L = 15, V = 151936 bf16 with planted
    peaks, B = 64): one round = ddtree_build (stage 1, selection, fused mask)
    + ddtree_accept. Device time per round from events around many
    back-to-back rounds; host-visible latency (enqueue to synchronize) per
    round, median and spread; the same for the round captured as a HIP graph
    and replayed (reported beside the eager figures, which stay the value)."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.CONFIGS[2]
    L, V, B = c["L"], c["V"], c["B"]
    dev = torch.device("cuda:0")
    x = gen.make_logits(2, 0)
    Y = gen.drafter_draws(2, 0, x, c["dtype"])
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    tree = pkg.ddtree_build(xd, B)
    torch.cuda.synchronize()
    tgt = torch.from_numpy(gen.node_targets_from_depths(
        Y, tree["depths"].cpu().numpy(), tree["num_nodes"].cpu().numpy(), B)).to(dev)
    acc = pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"], tgt, L)

    def rnd():
        pkg.ddtree_build(xd, B, out=tree)
        pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"], tgt, L, out=acc)

    n = max(args.steps, 1000)
    for _ in range(max(args.warmup, 20)):
        rnd()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        rnd()
    b.record()
    torch.cuda.synchronize()
    dev_us = a.elapsed_time(b) * 1e3 / n
    host = []
    for _ in range(n):
        t0 = time.perf_counter()
        rnd()
        torch.cuda.synchronize()
        host.append((time.perf_counter() - t0) * 1e6)
    host = np.array(host)
    # the same round captured once as a HIP graph and replayed: no per-launch
    # host work (the library records no memsets; inputs and outputs stay put)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rnd()
    for _ in range(max(args.warmup, 20)):
        graph.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    gdev_us = a.elapsed_time(b) * 1e3 / n
    ghost = []
    for _ in range(n):
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        ghost.append((time.perf_counter() - t0) * 1e6)
    ghost = np.array(ghost)
    res = {
        "metric": "build+mask+accept latency at batch 1, V=151936, L=15, B=64",
        "value": round(float(np.median(host)), 2), "unit": "us", "n_gpus": 1, "steps": n,
        "warmup": max(args.warmup, 20), "ms_per_step": round(float(np.median(host)) / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32/f64",
        "data": "synthetic",
        "config": {"workload": "batch1_L15_V151936_B64_bf16_logits", "batch": 1, "L": L, "V": V,
                   "B": B},
        "host_latency_us": {"p10": round(float(np.percentile(host, 10)), 2),
                            "p50": round(float(np.median(host)), 2),
                            "p90": round(float(np.percentile(host, 90)), 2)},
        "device_us_per_round": round(dev_us, 2),
        "graph_replay": {"host_latency_us": {"p10": round(float(np.percentile(ghost, 10)), 2),
                                             "p50": round(float(np.median(ghost)), 2),
                                             "p90": round(float(np.percentile(ghost, 90)), 2)},
                         "device_us_per_round": round(gdev_us, 2)},
    }
    print(json.dumps(res), flush=True)
    return 0


# Verifier cache of the KV-compaction workload: Qwen3-8B's attention shape
# (36 layers, 8 KV heads, head dim 128, bf16), 1024 tokens of context.
KV_LAYERS, KV_HEADS, KV_DH, KV_PAST = 36, 8, 128, 1024


def kv_bench(args) -> int:
    """KV-cache compaction after a batch-64 round: the trees and accepted paths
    of the batch-64 workload, a verifier cache of the shape above; one step =
    one ddtree_compact_kv call (in place)."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.CONFIGS[3]
    batch, L, B = c["batch"], c["L"], c["B"]
    dev = torch.device("cuda:0")
    x = gen.make_logits(3, 0)
    Y = gen.drafter_draws(3, 0, x, c["dtype"])
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    tree = pkg.ddtree_build(xd, B)
    torch.cuda.synchronize()
    tgt = gen.node_targets_from_depths(Y, tree["depths"].cpu().numpy(),
                                       tree["num_nodes"].cpu().numpy(), B)
    acc = pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"],
                            torch.from_numpy(tgt).to(dev), L)
    cap = KV_PAST + B + 1
    shape = (KV_LAYERS, batch, KV_HEADS, cap, KV_DH)
    kc = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    vc = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    past = torch.full((batch,), KV_PAST, dtype=torch.int32, device=dev)
    new_len = torch.empty((batch,), dtype=torch.int32, device=dev)
    an, al = acc["accepted_nodes"], acc["accept_len"]
    for _ in range(args.warmup):
        pkg.ddtree_compact_kv(kc, vc, past, an, al, new_len)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        pkg.ddtree_compact_kv(kc, vc, past, an, al, new_len)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = a.elapsed_time(b) * 1e3 / args.steps
    moved = int(al.sum().item())
    row_bytes = KV_DH * 2
    alg_bytes = moved * KV_LAYERS * KV_HEADS * 2 * row_bytes * 2  # K and V rows, read + write
    gbps = alg_bytes / (us / 1e6) / 1e9
    res = {
        "metric": "KV-cache compaction time per round at batch 64 (accepted paths of the "
                  "batch-64 draft-tree workload)",
        "value": round(us, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (bit copy)", "data": "synthetic",
        "config": {"workload": "kv_compact_batch64_layers36_kvheads8_dh128_past1024",
                   "batch": batch, "layers": KV_LAYERS, "kv_heads": KV_HEADS, "head_dim": KV_DH,
                   "past": KV_PAST, "cap": cap, "accepted_rows": moved},
        "roofline": {"bound": "hbm", "kernel": "kv_compact_kernel", "achieved": round(gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "avg_launch_us": round(us, 2), "bytes_per_launch": alg_bytes,
                     "traffic": None},
        "wall_s": round(wall, 3),
    }
    print(json.dumps(res), flush=True)
    return 0


def read_probe_bench(args) -> int:
    """Stage 1's load path alone over the batch-64 workload's rotated buffers
    (960 rows of 303,872 bytes): the read ceiling stage 1 is measured against."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.CONFIGS[3]
    rows, V = c["batch"] * c["L"], c["V"]
    dev = torch.device("cuda:0")
    x = gen.make_logits(3, 0)
    x_dev = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    bufs = [x_dev] + [x_dev.clone() for _ in range(args.buffers - 1)]
    gbps, us = read_ceiling(pkg, torch, bufs, rows, V * 2, max(args.steps, 1))
    print(json.dumps({"probe": "read ceiling (ddtree_read_probe)", "rows": rows,
                      "row_bytes": V * 2, "launches_timed": max(args.steps, 1),
                      "avg_launch_us": round(us, 2), "gbps": round(gbps, 1),
                      "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}), flush=True)
    return 0


def ts_load_probe_bench(args) -> int:
    """TreeSpark's head-evaluation loads alone (ddtree_ts_load_probe) at the
    README shape (V = 151936, H = 2560, 128 parents): W alone and W with the
    parents' embedding rows in each load pattern, for 128 distinct parent
    tokens and for 8 (each repeated 16 times). Launches interleaved by round."""
    import numpy as np
    import torch

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    c = gen.TREESPARK
    V, H = c["V"], c["H"]
    dev = torch.device("cuda:0")
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=dev)
    E = torch.zeros((V, H), dtype=torch.bfloat16, device=dev)
    toks = {128: [(i * 1187 + 13) % V for i in range(128)],
            8: [((i % 8) * 1187 + 13) % V for i in range(128)]}
    toks = {n: torch.tensor(t, dtype=torch.int32, device=dev) for n, t in toks.items()}
    names = {0: "W alone (nt)", 1: "W (nt) + rows in MFMA layout", 2: "W (nt) + rows as lines",
             3: "W (sc1 nt) + rows as lines", 4: "W alone (sc1 nt)",
             5: "W (nt) + half the rows as lines",
             6: "W (nt) + rows as lines, 256-row tiles of eight waves",
             7: "W (nt) + rows as lines, 256-row tiles, one persistent workgroup per CU"}
    cases = [(v, 128) for v in range(8)] + [(1, 8), (2, 8), (3, 8), (6, 8), (7, 8)]
    sink = torch.empty(256, dtype=torch.int32, device=dev)
    for v, n in cases:
        pkg.ddtree_ts_load_probe(W, E, toks[n], v, sink)
    torch.cuda.synchronize()
    rounds = max(args.steps // 10, 5)
    times = {cs: [] for cs in cases}
    for _ in range(rounds):
        for cs in cases:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(5):
                pkg.ddtree_ts_load_probe(W, E, toks[cs[1]], cs[0], sink)
            b.record()
            torch.cuda.synchronize()
            times[cs].append(a.elapsed_time(b) / 5 * 1e3)
    wbytes = V * H * 2
    res = []
    for (v, n), t in times.items():
        us = float(np.median(t))
        res.append({"variant": v, "loads": names[v], "distinct_parent_rows": n,
                    "median_launch_us": round(us, 1), "w_gbps": round(wbytes / us / 1e3, 1)})
    print(json.dumps({"probe": "TreeSpark head-evaluation loads (ddtree_ts_load_probe)",
                      "V": V, "H": H, "parents": 128, "launches_per_case": 5 * rounds,
                      "cases": res}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--buffers", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--treespark", action="store_true",
                    help="time treespark_expand on the TreeSpark workload instead (own JSON line)")
    ap.add_argument("--sparkling", action="store_true",
                    help="time sparkling_build on the SparklingTree workload instead (own JSON line)")
    ap.add_argument("--dspark", action="store_true",
                    help="time dspark_budget on 256 requests x 16 guesses instead (own JSON line)")
    ap.add_argument("--beam", action="store_true",
                    help="time sparkling_beam on the SparklingTree workload instead (own JSON line)")
    ap.add_argument("--kv-compact", action="store_true",
                    help="time ddtree_compact_kv after a batch-64 round instead (own JSON line)")
    ap.add_argument("--workload", choices=("c3", "c2", "c5"), default="c3",
                    help="c3: batch 64, B 128 (default, the headline); c2: batch 1, B 64 latency "
                         "of build + mask + accept; c5: batch 256, B 256 (own JSON lines)")
    ap.add_argument("--ts-load-probe", action="store_true",
                    help="TreeSpark's head-evaluation loads alone, by load pattern and W policy")
    ap.add_argument("--read-probe", action="store_true",
                    help="only time the read probe over the batch-64 buffers (own JSON line)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): every draft tree is "
              "independent, so more GPUs would each run this same per-GPU workload on their "
              "own requests; multi-GPU runs are not part of this build.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_probe:
        # A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it
        # calibrates the per-dispatch byte counts of the kernels.
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return 0

    import draft_tree_construction_depth_amd as pkg
    from draft_tree_construction_depth_amd import gen

    if args.treespark:
        return treespark_bench(args)
    if args.kv_compact:
        return kv_bench(args)
    if args.sparkling:
        return sparkling_bench(args)
    if args.dspark:
        return dspark_bench(args)
    if args.beam:
        return beam_bench(args)
    if args.workload == "c2":
        return latency_bench(args)
    if args.read_probe:
        return read_probe_bench(args)
    if args.ts_load_probe:
        return ts_load_probe_bench(args)
    cfg = 5 if args.workload == "c5" else 3

    c = gen.CONFIGS[cfg]
    batch, L, V, B = c["batch"], c["L"], c["V"], c["B"]
    K = min(B, V)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x = gen.make_logits(cfg, 0)
    Y = gen.drafter_draws(cfg, 0, x, c["dtype"])
    x_dev = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    bufs = [x_dev] + [x_dev.clone() for _ in range(args.buffers - 1)]

    rows = batch * L
    tables = dict(ids=torch.empty((rows, K), dtype=torch.int32, device=dev),
                  vals=torch.empty((rows, K), dtype=torch.float32, device=dev),
                  lse=torch.empty((rows,), dtype=torch.float64, device=dev))
    tv = tables["vals"].view(batch, L, K)
    ti = tables["ids"].view(batch, L, K)
    tz = tables["lse"].view(batch, L)
    ws_size = pkg.lib().ddtree_row_topk_workspace_size(rows, V, K, pkg.DDT_BF16)
    ws = torch.zeros(ws_size, dtype=torch.uint8, device=dev)

    # One untimed round gives the tree shape; the per-node target tokens (the
    # target model's argmax at each node, a stand-in) follow from it. Its
    # trees, masks and walks are checked against the oracle after timing.
    pkg.ddtree_row_topk(bufs[0], K, out=tables, ws=ws)
    tree = pkg.ddtree_select(tv, ti, tz, B)
    torch.cuda.synchronize()
    tgt = gen.node_targets_from_depths(Y, tree["depths"].cpu().numpy(),
                                       tree["num_nodes"].cpu().numpy(), B)
    tgt_dev = torch.from_numpy(tgt).to(dev)
    acc = pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"], tgt_dev, L)
    torch.cuda.synchronize()
    first = {k: v.cpu().numpy() for k, v in {**tree, **acc}.items()}
    first["mask"] = first["mask"].view(np.uint64)

    def step(i):
        pkg.ddtree_row_topk(bufs[i % len(bufs)], K, out=tables, ws=ws)
        pkg.ddtree_select(tv, ti, tz, B, out=tree)
        pkg.ddtree_accept(tree["tree_tokens"], tree["parents"], tree["num_nodes"], tgt_dev, L,
                          out=acc)

    for i in range(args.warmup):
        step(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    trees_per_s = batch * args.steps / (total_ms / 1e3)

    # Stage 1 alone, after the timed loop: KERNEL_SAMPLES launches over the
    # rotated buffers, each between its own pair of events on the launch
    # stream (the library launches on torch's current stream).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(KERNEL_SAMPLES)]
    for i, (a, b) in enumerate(evs):
        a.record()
        pkg.ddtree_row_topk(bufs[i % len(bufs)], K, out=tables, ws=ws)
        b.record()
    torch.cuda.synchronize()
    s1_us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    s1_avg_us = float(s1_us.mean())
    ceiling_gbps, probe_us = read_ceiling(pkg, torch, bufs, rows, V * 2, KERNEL_SAMPLES)

    logits_bytes = batch * L * V * 2
    # Algorithmic bytes of the whole step (logits once, tree outputs, mask,
    # targets read, walk outputs).
    W = (B + 1 + 63) // 64
    step_bytes = logits_bytes + batch * (B * 12 + B * 4 + 4 + (B + 1) * W * 8
                                         + (B + 1) * 4 + (L + 2) * 4)
    achieved = logits_bytes / (s1_avg_us * 1e-6) / 1e9
    traffic = measured_traffic() if cfg == 3 else None

    result = {
        "metric": METRIC if cfg == 3 else
        "draft trees/sec at batch 256, V=151936, L=15, B=256; achieved HBM GB/s vs peak",
        "value": round(trees_per_s, 1),
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32/f64",
        "data": "synthetic",
        "config": {"workload": f"batch{batch}_L{L}_V{V}_B{B}_bf16_logits", "batch": batch,
                   "L": L, "V": V, "B": B, "input_buffers": len(bufs)},
        "whole_step_gbps": round(step_bytes * args.steps / (total_ms / 1e3) / 1e9, 1),
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": "stage1 (ddtree_row_topk)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "avg_launch_us": round(s1_avg_us, 2),
                     "median_launch_us": round(float(np.median(s1_us)), 2),
                     "launches_timed": len(s1_us),
                     "read_ceiling_gbps": round(ceiling_gbps, 1),
                     "read_ceiling_launch_us": round(probe_us, 2),
                     "frac_of_read_ceiling": round(achieved / ceiling_gbps, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        cb, o = cpu_baseline(x, Y, B, L)
        result["cpu_baseline"] = {k: (round(v, 2) if isinstance(v, float) else v)
                                  for k, v in cb.items()}
        result["parity"] = parity_of_run(first, o, tgt, B, L)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
