#!/usr/bin/env python3
"""Throughput of tree-indexed sparse attention decode on one MI355X.

A step is one pass of the whole hot path over one batch: tree_build over the
KV cache, then tree_route and tree_attend for every query head (one decode
step).  The default workload is GQA decode in bf16 with 32,768 keys per KV
head (batch 4, 32 query / 8 KV heads, d = 128, branching 8, leaf block 64,
3 levels, beam 8), inputs drawn from the seeded generator and resident in
HBM before timing starts.

Prints ONE JSON line on stdout; details go to stderr.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


SUMMARY_ROW_BYTES = {"f32": lambda d: 4 * d, "bf16": lambda d: 2 * d,
                     "fp8": lambda d: d + 4}   # fp8: the codes and the row's scale


def algorithmic_bytes(w, summary_dtype: str = "f32"):
    """Bytes the method must move (see the byte model in the design notes);
    a summary row is 4d bytes as float32, 2d as bfloat16, d + 4 as fp8."""
    s = w.elem_bytes
    d, b, W, L = w.head_dim, w.branching, w.beam, w.leaf_block
    heads = w.batch * w.kv_heads
    nodes = sum(b ** l for l in range(1, w.levels + 1))
    row = SUMMARY_ROW_BYTES[summary_dtype](d)
    build = heads * (w.n_keys * d * s + nodes * row)
    cand = b + sum(min(W, b ** (l - 1)) * b for l in range(2, w.levels + 1))
    route_q = cand * row + d * s + 4 * W
    attend_q = W * L * d * s * 2 + d * s + 4 * W + 4 * d
    return {"build": build, "route": w.queries * route_q, "attend": w.queries * attend_q,
            "candidates_per_query": cand}


COPY_BYTES = 256 << 20
FLUSH_BYTES = 1 << 30  # 4x the 256 MB Infinity Cache, 32x the L2s together
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{}.json")
BUILD_SOURCE = os.path.join(ROOT, "tree_indexed_sparse_build_amd", "csrc", "build.hip")


def _source_digest() -> str:
    """Digest of build.hip's code (comments and blank space ignored)."""
    import hashlib
    import re
    with open(BUILD_SOURCE) as f:
        code = re.sub(r"//[^\n]*", "", f.read())
    code = re.sub(r"\s+", " ", code).strip()
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per tree_build launch from the committed counter summary,
    or None when there is none or the build kernel changed since."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("build_source_sha256_16") != _source_digest():
        return None
    return t.get("build_bytes_per_launch")


def traffic_from_counters(workload: str, fetch_csv: str, write_csv: str) -> dict:
    """Scales rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the
    k_build dispatches by what the same counters read for the 256 MiB
    reference copy (COPY_BYTES read and written), and writes the summary."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                name = r["Kernel_Name"]
                vals.setdefault(name, []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, key, how="mean"):
        ks = [k for k in vals if key in k]
        if not ks:
            raise SystemExit(f"no dispatch matching {key!r} in the counter file")
        xs = [v for k in ks for v in vals[k]]
        return (max(xs) if how == "max" else sum(xs) / len(xs)), ks

    # the reference copy is the largest copy dispatch (input uploads are smaller)
    f_copy, _ = pick(fetch, "copyBuffer", "max")
    w_copy, _ = pick(write, "copyBuffer", "max")
    f_build, _ = pick(fetch, "k_build<")
    w_build, _ = pick(write, "k_build<")
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    out = {
        "workload": workload,
        "kernel": "k_build (first kernel of tree_build)",
        "fetch_kib_per_dispatch": f_build, "write_kib_per_dispatch": w_build,
        "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "build_bytes_per_launch": f_build * 1024.0 * f_scale + w_build * 1024.0 * w_scale,
        "build_source_sha256_16": _source_digest(),
    }
    with open(TRAFFIC_FILE.format(workload), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def cpu_baseline(w, x, min_seconds: float = 10.0, max_reps: int = 500):
    """The CPU oracle, as it stands, on whole steps of the same workload."""
    from oracle import tis_oracle as O
    from threadpoolctl import threadpool_limits
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            O.decode(x["Q"], x["K"], x["V"], w.dtype, w.branching, w.leaf_block, w.levels,
                     w.beam)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or reps >= max_reps:
                break
    return {"value": reps * w.queries / el, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole steps (build over all {w.batch * w.kv_heads} KV heads, "
                      f"route + attend of all {w.queries} queries) of the same workload, "
                      f"numpy fp64, BLAS limited to 1 thread, {el:.1f} s"}


def per_launch(torch, fn, reps):
    """Average duration (s) of fn's launch: reps launches back to back
    between one event pair (event overhead spread over reps launches)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def reduced_summaries(tis, torch, w, Q, K, V, reps, warmup, summary_dtype):
    """The step with summaries stored as bfloat16 or fp8 (the same means
    rounded once to the narrower type): build and fused decode durations, and
    the decode's rate on its own algorithmic bytes (each routing level reads
    a half or about a quarter of the float32 bytes)."""
    plan = tis.DecodePlan(Q, K, V, w.branching, w.leaf_block, w.levels, w.beam,
                          summary_dtype=summary_dtype)
    for _ in range(warmup):
        plan.build()
        plan.decode()

    def step():
        plan.build()
        plan.decode()
    step_s = per_launch(torch, step, reps)
    build_s = per_launch(torch, plan.build, reps)
    decode_s = per_launch(torch, plan.decode, reps)
    by = algorithmic_bytes(w, summary_dtype)
    dec = by["route"] + by["attend"]
    return {"regime": f"as the headline step, summaries stored as {summary_dtype}",
            "step_us": step_s * 1e6, "queries_per_s_step": w.queries / step_s,
            "build_us": build_s * 1e6, "build_gbs": by["build"] / build_s / 1e9,
            "decode_us": decode_s * 1e6, "decode_queries_per_s": w.queries / decode_s,
            "decode_gbs": dec / decode_s / 1e9, "decode_frac": dec / decode_s / 1e9 / HBM_PEAK_GBS,
            "decode_bytes": dec}


def threshold_retrieval(tis, torch, w, Q, K, V, reps, warmup, k_ranks=(64, 512)):
    """Bounding-sphere threshold retrieval on the step's data: the radii pass
    over K, then the fused threshold decode at thresholds halfway between
    each query's k-th and (k+1)-th best key score (set up with a dense torch
    matmul, not timed)."""
    tree = tis.tree_build(K, w.branching, w.leaf_block, w.levels)
    radii = tis.tree_radii(K, tree)
    for _ in range(warmup):
        tis.tree_radii(K, tree)
    radii_s = per_launch(torch, lambda: tis.tree_radii(K, tree), reps)
    nodes = sum(w.branching ** l for l in range(1, w.levels + 1))
    radii_bytes = w.batch * w.kv_heads * (w.n_keys * w.head_dim * w.elem_bytes
                                          + nodes * w.head_dim * 4 + nodes * 4)
    max_nodes = min(w.n_leaves, tis.TIS_MAX_SURVIVORS)
    out = {"radii_us": radii_s * 1e6, "radii_gbs": radii_bytes / radii_s / 1e9,
           "radii_bytes": radii_bytes, "max_nodes": max_nodes, "thresholds": []}
    G = w.group
    for k in k_ranks:
        tau = torch.empty((w.batch, w.q_heads), dtype=torch.float32, device=Q.device)
        for bi in range(w.batch):
            for h in range(w.kv_heads):
                s = Q[bi, h * G:(h + 1) * G].float() @ K[bi, h].float().t()
                top = torch.topk(s, k + 1, dim=1).values
                tau[bi, h * G:(h + 1) * G] = (top[:, k - 1] + top[:, k]) / 2
        o = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=Q.device)
        _, _, cnt = tis.tree_decode_threshold(Q, K, V, tree, radii, tau, max_nodes,
                                              return_indices=True)
        for _ in range(warmup):
            tis.tree_decode_threshold(Q, K, V, tree, radii, tau, max_nodes, out=o)
        dec_s = per_launch(torch, lambda: tis.tree_decode_threshold(
            Q, K, V, tree, radii, tau, max_nodes, out=o), reps)
        c = cnt.float()
        kept_bytes = float(c.clamp(min=0).sum()) * w.leaf_block * w.head_dim * w.elem_bytes * 2
        out["thresholds"].append({
            "k": k, "decode_us": dec_s * 1e6, "queries_per_s": w.queries / dec_s,
            "leaves_kept_mean": float(c.mean()), "leaves_kept_max": int(c.max()),
            "overflow": int((cnt < 0).sum()), "gathered_gbs": kept_bytes / dec_s / 1e9})
    return out


def causal_prefill_bench(tis, torch, w, Q, K, V, reps, warmup, max_positions=4096):
    """Causal prefill of the first P = min(N, max_positions) keys: every
    position a query over the tree of its prefix (queries: the workload's,
    one per head, plus seeded per-position noise).  Times the whole call
    (partial means + routing + causal attention) and counts the keys each
    query reads."""
    P = min(w.n_keys, max_positions)
    g = torch.Generator(device=Q.device).manual_seed(1234)
    qf = Q.float()[:, :, None, :] + torch.randn((w.batch, w.q_heads, P, w.head_dim),
                                                generator=g, device=Q.device)
    Qp = qf.to(Q.dtype).contiguous()
    ct = tis.CacheTree(K, V, w.branching, w.leaf_block)
    ct.append(P)
    out = torch.empty((w.batch, w.q_heads, P, w.head_dim), dtype=torch.float32, device=Q.device)
    _, idx = ct.causal_prefill(Qp, w.beam, return_indices=True)
    for _ in range(warmup):
        ct.causal_prefill(Qp, w.beam, out=out)
    reps = max(3, min(reps, 20))
    t = per_launch(torch, lambda: ct.causal_prefill(Qp, w.beam, out=out), reps)
    pos = torch.arange(P, device=Q.device).view(1, 1, P, 1)
    blk = idx.long()
    size = torch.clamp(pos + 1 - blk * w.leaf_block, max=w.leaf_block)
    reads = torch.where(blk >= 0, size, torch.zeros_like(size)).sum(-1).double()
    queries = w.batch * w.q_heads * P
    return {"positions": P, "queries": queries, "us": t * 1e6, "queries_per_s": queries / t,
            "keys_read_mean": float(reads.mean()), "dense_causal_keys_mean": (P + 1) / 2}


def cache_states(torch, dev, plan, reps, back_to_back):
    """Durations in two cache states.  cold: 1 GiB read first, which leaves
    none of the inputs in the Infinity Cache or an L2 and no dirty lines to
    write back (a flush by writing would charge its write-backs to the timed
    kernel); steady: cold, then one read of the summaries, as when the tree
    stays hot across decode steps.  Each is the median of `reps` lone
    launches between their own events, compared with lone warm launches
    timed the same way (nothing in between): the difference is what the
    cache state costs, and adding it to the back-to-back duration removes
    the event and dispatch overhead a lone launch carries."""
    import numpy as np
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def one(fn, state):
        if state != "warm":
            flush.sum()
        if state == "steady":
            plan.summaries.sum()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    out = {}
    for name, fn in (("build", plan.build), ("decode", plan.decode)):
        lone = {}
        for state in ("warm", "cold", "steady"):
            if name == "build" and state == "steady":
                continue
            one(fn, state)
            lone[state] = float(np.median([one(fn, state) for _ in range(reps)]))
        for state, us in lone.items():
            out[f"{name}_{state}_lone_us"] = us
            if state != "warm":
                out[f"{name}_{state}_us"] = back_to_back[name] + us - lone["warm"]
    del flush
    return out


def distinct_route_bytes(tis, w, Q, K):
    """Summary bytes the route must read when each distinct row is counted
    once per KV head (its G query heads run on one XCD and share its L2):
    the rows of every scored level's candidates, from the route's trace.
    Levels whose nodes all fit in the beam are kept without scoring; the
    first level that cuts scores all of its nodes, later ones the children
    of the nodes each query kept."""
    import numpy as np
    tree = tis.tree_build(K, w.branching, w.leaf_block, w.levels)
    _, tr = tis.tree_route(Q, tree, w.beam, trace=True)
    tr = tr.cpu().numpy()
    b, lv, W, G = w.branching, w.levels, w.beam, w.group
    rows = 0
    for bb in range(w.batch):
        for h in range(w.kv_heads):
            grp = tr[bb, h * G:(h + 1) * G]  # [G, levels, W]
            for l in range(1, lv + 1):
                if b ** l <= W:
                    continue  # kept whole, not scored
                if b ** (l - 1) <= W:
                    rows += b ** l  # the first level that cuts: all of its nodes
                    continue
                kept = np.unique(grp[:, l - 2][grp[:, l - 2] >= 0])
                rows += len(kept) * b  # distinct parents kept by the group, b children each
    return rows * w.head_dim * 4


def cache_decode_loop(tis, w, K, V, Q, steps, warmup):
    """The decode loop over a growing cache of the same shape: the tree over
    the first keys of the cache is filled by one long append, then every
    step appends one key per head (tis_cache_tree_append) and decodes every
    query (tis_cache_tree_decode).  Times: the long append, one-key appends
    back to back, decodes back to back, whole steps back to back, and the
    same step as one fused call (tis_cache_tree_append_decode)."""
    import torch
    need = 4 * (steps + warmup) + 8
    prefill = w.n_keys - need
    if prefill < 1:
        return None
    ct = tis.CacheTree(K, V, w.branching, w.leaf_block)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=K.device)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us

    ct.append(prefill)  # warm the kernel once, then time a fresh prefill
    ct.reset()
    prefill_us = timed(lambda: ct.append(prefill), 1)
    decode = ct.bind_decode(Q, w.beam, out)
    step = lambda: (ct.append(1), decode())
    for _ in range(warmup):
        step()
    step_us = timed(step, steps)
    append_us = timed(lambda: ct.append(1), steps)
    decode_us = timed(decode, steps)
    fused = ct.bind_decode(Q, w.beam, out, append=True)
    for _ in range(warmup):
        fused()
    fused_us = timed(fused, steps)
    kbytes = prefill * w.batch * w.kv_heads * w.head_dim * w.elem_bytes
    return {"regime": "tree over the first n keys of a cache of the workload's size; "
                      "one key appended per head per step",
            "n_keys_at_end": ct.n_keys, "levels": ct.levels,
            "prefill_keys": prefill, "prefill_us": prefill_us,
            "prefill_gbs": kbytes / (prefill_us * 1e-6) / 1e9,
            "append1_us": append_us, "decode_us": decode_us, "step_us": step_us,
            "queries_per_s": w.queries / (step_us * 1e-6),
            "fused_step_us": fused_us, "fused_queries_per_s": w.queries / (fused_us * 1e-6)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-loop", action="store_true",
                    help="skip the growing-cache decode loop measurement")
    ap.add_argument("--no-bf16-summaries", action="store_true",
                    help="skip the measurement of the step with bfloat16 and fp8 summaries")
    ap.add_argument("--no-threshold", action="store_true",
                    help="skip the bounding-sphere threshold retrieval measurement")
    ap.add_argument("--prefill-positions", type=int, default=4096,
                    help="positions of the causal prefill measurement (at most the workload's keys)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the causal prefill measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (the reference "
                         "dispatch for scaling HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of "
                         "a --calibrate-copy run into profiles/traffic_<workload>.json and exit")
    args = ap.parse_args(argv)
    if args.traffic_from:
        print(json.dumps(traffic_from_counters(args.workload, *args.traffic_from)))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); every tree is "
              "independent per (batch, KV head), so N GPUs would each run their own share "
              "with no exchange", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import workloads
    import tree_indexed_sparse_build_amd as tis

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    w = workloads.get(args.workload)
    t0 = time.time()
    x = workloads.generate(w)
    log(f"workload {w.name}: generated in {time.time() - t0:.1f}s; {tis.version()}; "
        f"device {torch.cuda.get_device_name(0)}")
    dev = torch.device("cuda", 0)
    Q = tis.from_storage(x["Q"], w.dtype, dev)
    K = tis.from_storage(x["K"], w.dtype, dev)
    V = tis.from_storage(x["V"], w.dtype, dev)
    plan = tis.DecodePlan(Q, K, V, w.branching, w.leaf_block, w.levels, w.beam)
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        plan.build()
        plan.decode()  # route + attend of every query in one launch

    def step_separate():
        plan.build()
        plan.route()
        plan.attend()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K_ = args.steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    # timed region 1: whole steps back to back (the headline)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    start.record()
    for _ in range(K_):
        step()
    end.record()
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    h2 = time.perf_counter()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K_
    # the same steps replayed from a HIP graph (one capture of build + decode):
    # the replays must reproduce the eager outputs bit for bit
    out_eager = plan.out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        plan.out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(plan.out, out_eager):
            raise RuntimeError("graph replay does not reproduce the eager step")
    torch.cuda.synchronize()
    start.record()
    for _ in range(K_):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms_step_graph = start.elapsed_time(end) / K_
    # the same steps with route and attend as separate calls (reference)
    torch.cuda.synchronize()
    start.record()
    for _ in range(K_):
        step_separate()
    end.record()
    torch.cuda.synchronize()
    ms_step_separate = start.elapsed_time(end) / K_
    # timed region 2: each kernel K times back to back between one event pair
    # (its average launch duration; event overhead is spread over K launches)
    t_build = np.array([per_launch(torch, plan.build, K_)])
    t_route = np.array([per_launch(torch, plan.route, K_)])
    t_attend = np.array([per_launch(torch, plan.attend, K_)])
    t_decode = per_launch(torch, plan.decode, K_)

    by = algorithmic_bytes(w)
    build_gbs = by["build"] / t_build.mean() / 1e9
    decode_s = t_decode
    idx = plan.indices.cpu().numpy()
    uniq = 0
    for bb in range(w.batch):
        for h in range(w.kv_heads):
            uniq += len(np.unique(idx[bb, h * w.group:(h + 1) * w.group]))
    attend_dedup = uniq * w.leaf_block * w.head_dim * w.elem_bytes * 2
    route_dedup = distinct_route_bytes(tis, w, Q, K)
    # the query rows read and the kept leaves written, once per query
    qio = w.queries * (w.head_dim * w.elem_bytes + 4 * w.beam)
    dec_dedup = route_dedup + attend_dedup + qio
    log(f"step {ms_step * 1e3:.1f} us (host enqueue {(h1 - h0) / K_ * 1e6:.1f} us/step, "
        f"wall {(h2 - h0) / K_ * 1e6:.1f} us/step); replayed from a graph "
        f"{ms_step_graph * 1e3:.1f} us; with separate route + attend calls "
        f"{ms_step_separate * 1e3:.1f} us")
    log(f"build  {t_build.mean() * 1e6:8.2f} us  {build_gbs:8.1f} GB/s "
        f"({build_gbs / HBM_PEAK_GBS:.1%} of 8 TB/s) on {by['build'] / 1e6:.1f} MB")
    log(f"route  {t_route.mean() * 1e6:8.2f} us  {by['route'] / t_route.mean() / 1e9:8.1f} GB/s "
        f"on {by['route'] / 1e6:.2f} MB ({by['candidates_per_query']} candidates/query)")
    log(f"attend {t_attend.mean() * 1e6:8.2f} us  {by['attend'] / t_attend.mean() / 1e9:8.1f} "
        f"GB/s on {by['attend'] / 1e6:.2f} MB per-query sum; "
        f"{attend_dedup / t_attend.mean() / 1e9:.1f} GB/s on {attend_dedup / 1e6:.2f} MB of "
        f"distinct blocks per KV head")
    dec_bytes = by["route"] + by["attend"]
    log(f"decode (fused route + attend) {decode_s * 1e6:.2f} us -> "
        f"{w.queries / decode_s:.3e} queries/s, {dec_bytes / decode_s / 1e9:.1f} GB/s "
        f"({dec_bytes / decode_s / 1e9 / HBM_PEAK_GBS:.1%}) on {dec_bytes / 1e6:.2f} MB "
        f"per-query sum, {dec_dedup / decode_s / 1e9:.1f} GB/s "
        f"({dec_dedup / decode_s / 1e9 / HBM_PEAK_GBS:.1%}) on {dec_dedup / 1e6:.2f} MB "
        f"distinct per KV head; "
        f"in the step (step - build): {ms_step * 1e3 - t_build.mean() * 1e6:.2f} us")

    states = cache_states(torch, dev, plan, 30,
                          {"build": t_build.mean() * 1e6, "decode": decode_s * 1e6})
    log(f"cache states (lone launches, median of 30; cold = 1 GiB read first, steady = cold + "
        f"summaries read; lone warm build {states['build_warm_lone_us']:.1f} us, decode "
        f"{states['decode_warm_lone_us']:.2f} us): build cold {states['build_cold_us']:.1f} us "
        f"({by['build'] / states['build_cold_us'] / 1e3:.0f} GB/s, "
        f"{by['build'] / states['build_cold_us'] / 1e3 / HBM_PEAK_GBS:.1%}); decode cold "
        f"{states['decode_cold_us']:.2f} us ({dec_bytes / states['decode_cold_us'] / 1e3:.0f} "
        f"GB/s, {dec_bytes / states['decode_cold_us'] / 1e3 / HBM_PEAK_GBS:.1%}), steady "
        f"{states['decode_steady_us']:.2f} us")

    pre = None
    if not args.no_prefill:
        pre = causal_prefill_bench(tis, torch, w, Q, K, V, K_, args.warmup,
                                   max_positions=args.prefill_positions)
        log(f"causal prefill of the first {pre['positions']} keys ({pre['queries']} queries): "
            f"{pre['us']:.1f} us -> {pre['queries_per_s']:.3e} queries/s; keys read per query "
            f"{pre['keys_read_mean']:.2f} on average (dense causal "
            f"{pre['dense_causal_keys_mean']:.1f})")

    thr = None
    if not args.no_threshold:
        thr = threshold_retrieval(tis, torch, w, Q, K, V, K_, args.warmup)
        log(f"bounding spheres: radii {thr['radii_us']:.1f} us ({thr['radii_gbs']:.0f} GB/s on "
            f"{thr['radii_bytes'] / 1e6:.1f} MB); " + "; ".join(
                f"threshold at the {t['k']}-th best score: decode {t['decode_us']:.2f} us -> "
                f"{t['queries_per_s']:.3e} queries/s, leaves kept mean "
                f"{t['leaves_kept_mean']:.1f} max {t['leaves_kept_max']} of {w.n_leaves}, "
                f"overflow {t['overflow']}"
                for t in thr["thresholds"]))

    bf = None
    if not args.no_bf16_summaries:
        bf = {}
        for sd in ("bf16", "fp8"):
            r = reduced_summaries(tis, torch, w, Q, K, V, K_, args.warmup, sd)
            bf[sd] = r
            log(f"{sd} summaries: step {r['step_us']:.1f} us ({r['queries_per_s_step']:.3e} "
                f"queries/s); build {r['build_us']:.2f} us ({r['build_gbs']:.0f} GB/s); decode "
                f"{r['decode_us']:.2f} us -> {r['decode_queries_per_s']:.3e} queries/s, "
                f"{r['decode_gbs']:.0f} GB/s ({r['decode_frac']:.1%}) on "
                f"{r['decode_bytes'] / 1e6:.2f} MB")

    traffic = load_traffic(w.name)

    cache = None
    if not args.no_cache_loop:
        cache = cache_decode_loop(tis, w, K, V, Q, K_, args.warmup)
        log(f"growing cache: prefill append of {cache['prefill_keys']} keys/head "
            f"{cache['prefill_us']:.1f} us ({cache['prefill_gbs']:.1f} GB/s); append of 1 key "
            f"{cache['append1_us']:.2f} us; decode {cache['decode_us']:.2f} us; decode step "
            f"(append + decode) {cache['step_us']:.2f} us -> {cache['queries_per_s']:.3e} queries/s; "
            f"fused step {cache['fused_step_us']:.2f} us -> "
            f"{cache['fused_queries_per_s']:.3e} queries/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w, x)
        log(f"cpu oracle {cpu['value']:.2f} queries/s ({cpu['sample']})")

    line = {
        "metric": "decode queries/sec + achieved HBM GB/s (% roofline) at N=32K\u20131M keys",
        "value": w.queries / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs; fp64 build sums and route scores; fp32 attention"
        if w.dtype == "bf16" else "f32 inputs; fp64 build sums and route scores; fp32 attention",
        "data": "synthetic (seeded clustered-Gaussian keys, see workloads.py)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "n_keys": w.n_keys,
                   "branching": w.branching, "leaf_block": w.leaf_block, "levels": w.levels,
                   "beam": w.beam,
                   "step": "tree_build + tree_decode (tree_route and tree_attend in one launch)"},
        "roofline": {"kernel": "tree_build", "bound": "hbm", "achieved": build_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": build_gbs / HBM_PEAK_GBS,
                     "traffic": traffic},
        "decode": {"regime": "fused route + attend launches back to back on the step's data",
                   "us": decode_s * 1e6, "queries_per_s": w.queries / decode_s,
                   "gbs": dec_bytes / decode_s / 1e9,
                   "frac": dec_bytes / decode_s / 1e9 / HBM_PEAK_GBS,
                   "in_step_us": ms_step * 1e3 - t_build.mean() * 1e6,
                   "step_us_separate_calls": ms_step_separate * 1e3,
                   "step_us_graph_replay": ms_step_graph * 1e3,
                   "route_us": t_route.mean() * 1e6, "attend_us": t_attend.mean() * 1e6,
                   "attend_gbs_per_query_bytes": by["attend"] / t_attend.mean() / 1e9,
                   "attend_gbs_distinct_blocks": attend_dedup / t_attend.mean() / 1e9,
                   "bytes_per_query_sum": dec_bytes, "bytes_distinct": dec_dedup,
                   "gbs_distinct": dec_dedup / decode_s / 1e9,
                   "frac_distinct": dec_dedup / decode_s / 1e9 / HBM_PEAK_GBS,
                   "cache_states": dict(states, regime="cold: 1 GiB read first; steady: cold, "
                                        "then the summaries read once; *_lone_us: median of "
                                        "30 lone launches between events; *_cold_us and "
                                        "*_steady_us: back-to-back duration + (lone in that "
                                        "state - lone warm)")},
        "cpu_baseline": cpu,
        "cache_decode_loop": cache,
        "reduced_summaries": bf,
        "threshold_retrieval": thr,
        "causal_prefill": pre,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
