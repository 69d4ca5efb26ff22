#!/usr/bin/env python3
"""Throughput of tree-indexed sparse attention decode on one MI355X.

A step is one pass of the whole hot path over one batch: tree_build over the
KV cache, then tree_route and tree_attend for every query head (one fused
decode launch).  The headline workload is GQA decode in bf16 with 32,768 keys
per KV head (batch 4, 32 query / 8 KV heads, d = 128, branching 8, leaf block
64, 3 levels, beam 8).  Each timed step starts from cold caches: a 1 GiB
streaming read before it (not counted) leaves none of its inputs in the L2s
or the Infinity Cache.  Inputs come from the seeded generator and are
resident in HBM before timing starts.

The same run measures the other large workloads (262,144 keys, 1,048,576
keys, the six-level planted tree): the cold build, and the decode cold
(caches emptied), steady (caches emptied, then the summaries read once, as
in a decode loop that keeps the tree hot) and warm (back-to-back launches
replayed from a graph), each as queries/s and as GB/s on the bytes the method
must move, per query and counting each distinct row and block once per KV
head.  Beside them: the streaming-read ceiling and the dependent-load latency
measured by the library's probes, and from them a latency floor per decode.

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
HEADLINE = "gqa_32k"
OTHERS = ("gqa_256k", "long_1m", "deep_planted")
FLUSH_BYTES = 1 << 30  # 4x the 256 MB Infinity Cache, 32x the L2s together
COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{}.json")
BUILD_SOURCE = os.path.join(ROOT, "tree_indexed_sparse_build_amd", "csrc", "build.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


SUMMARY_ROW_BYTES = {"f32": lambda d: 4 * d, "bf16": lambda d: 2 * d,
                     "fp8": lambda d: d + 4}   # fp8: the codes and the row's scale


def first_cut(w) -> int:
    """First level with more nodes than the beam (levels above keep all)."""
    l0 = 1
    while l0 < w.levels and w.branching ** l0 <= w.beam:
        l0 += 1
    return l0


def algorithmic_bytes(w, summary_dtype: str = "f32"):
    """Bytes the method must move: the build reads K once and writes every
    summary once; a query's route reads the summary row of every candidate
    it scores (plus its query row and kept leaves), its attention the K and V
    rows of its kept leaf blocks (plus query, indices and output).  A summary
    row is 4d bytes as float32, 2d as bfloat16, d + 4 as fp8."""
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


def distinct_bytes(tis, w, Q, K):
    """Decode bytes when each distinct summary row and leaf block is counted
    once per (batch, KV head), as its query heads read them through one L2:
    the rows of every scored level's candidates (from the route's trace; the
    first level that cuts scores all of its nodes, later ones the children of
    the nodes the group kept), the K and V rows of the distinct kept leaves,
    and each query's own row, kept leaves and output.  Also returns the leaf
    union fraction: distinct kept leaves per (batch, KV head), summed, over
    the queries' kept leaves (1.0: the G query heads of a group share none;
    1 / G: all keep the same), the most that gathering each leaf of a
    group's union once could save of the gather's bytes."""
    import numpy as np
    tree = tis.tree_build(K, w.branching, w.leaf_block, w.levels)
    idx, tr = tis.tree_route(Q, tree, w.beam, trace=True)
    tr, idx = tr.cpu().numpy(), idx.cpu().numpy()
    b, lv, W, G, d = w.branching, w.levels, w.beam, w.group, w.head_dim
    rows = blocks = 0
    for bb in range(w.batch):
        for h in range(w.kv_heads):
            grp = tr[bb, h * G:(h + 1) * G]
            for l in range(1, lv + 1):
                if b ** l <= W:
                    continue  # kept whole, not scored
                if b ** (l - 1) <= W:
                    rows += b ** l
                    continue
                kept = np.unique(grp[:, l - 2][grp[:, l - 2] >= 0])
                rows += len(kept) * b
            blocks += len(np.unique(idx[bb, h * G:(h + 1) * G]))
    per_query = d * w.elem_bytes + 4 * W + 4 * d
    kept = int((idx >= 0).sum())
    return (rows * d * 4 + blocks * w.leaf_block * d * w.elem_bytes * 2 + w.queries * per_query,
            blocks / max(kept, 1))


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
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, key, how="mean"):
        ks = [k for k in vals if key in k]
        if not ks:
            raise SystemExit(f"no dispatch matching {key!r} in the counter file")
        xs = [v for k in ks for v in vals[k]]
        return (max(xs) if how == "max" else sum(xs) / len(xs)), ks

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


def trace_summary(db_path: str, out_path: str, title: str, command: str,
                  segments: str = "") -> None:
    """Writes a kernel-trace summary (markdown) from a rocprofv3 database:
    per workload segment, kernel and grid size, the launches and their mean /
    median / min / max duration, grouped by what ran just before on the
    stream (a 1 GiB probe read = cold; another probe read = the summaries
    read after one, steady; the same kernel = back to back).  Segments begin
    at the marker reads of (k + 1) MiB (64 (k + 1) workgroups) the benchmark
    launches before the k-th workload; `segments` names them, comma-separated."""
    import sqlite3
    import statistics
    names = [n for n in segments.split(",") if n]
    con = sqlite3.connect(db_path)
    rows = list(con.execute("select name, start, end, grid_x, workgroup_x, queue_id "
                            "from kernels order by start"))
    groups = {}
    prev = {}
    seg = "-"
    for name, s, e, gx, wx, q in rows:
        short = name.replace("(anonymous namespace)::", "").replace("tis::", "")
        short = short.replace("void ", "", 1).split("(")[0]
        wgs = gx // max(wx, 1)
        if "k_probe_read" in short and wgs < 4096 and wgs % 64 == 0 and wgs // 64 <= len(names) \
                and (e - s) < 50e3:
            k = wgs // 64 - 1
            if names and (prev.get(q) is None or "k_probe_read" not in prev[q][0]):
                seg = names[k]
                prev[q] = None
                continue
        p = prev.get(q)
        if p is None:
            before = "-"
        elif "k_probe_read" in p[0]:
            # the 1 GiB flush takes ~150-250 us, a summaries read far less
            before = "probe read of 1 GiB (cold)" if p[2] > 100.0 else "probe read of the summaries"
        elif p[0] == short:
            before = "same kernel"
        else:
            before = p[0].split("<")[0]
        key = (seg, short, wgs, wx, before)
        groups.setdefault(key, []).append((e - s) / 1e3)
        prev[q] = (short, wgs, (e - s) / 1e3)
    lines = [f"# {title}", "", "Command (run from the repository root):", "", "```",
             command, "```", "",
             "rocprofv3 kernel trace; durations in microseconds (kernel begin to end). "
             "`before` is the dispatch that ran just before on the stream.", "",
             "| workload | kernel | workgroups x threads | before | launches | mean | median | "
             "min | max |",
             "|---|---|---|---|---|---|---|---|---|"]
    order = {n: i for i, n in enumerate(["-"] + names)}
    # "{workload}" in out_path: one file per workload segment
    outs = {n: out_path.replace("{workload}", n) for n in names} if "{workload}" in out_path \
        else None
    body = {}
    for (seg, short, wgs, wx, before), ds in sorted(
            groups.items(), key=lambda kv: (order.get(kv[0][0], 99), -sum(kv[1]))):
        if not (short.startswith("k_") or "probe" in short):
            continue
        body.setdefault(seg, []).append(
            f"| {seg} | `{short}` | {wgs} x {wx} | {before} | {len(ds)} | "
            f"{statistics.fmean(ds):.2f} | {statistics.median(ds):.2f} | {min(ds):.2f} | "
            f"{max(ds):.2f} |")
    if outs is None:
        with open(out_path, "w") as f:
            f.write("\n".join(lines + [r for seg in body for r in body[seg]]) + "\n")
        return
    for n, path in outs.items():
        head = [ln.replace(title, f"{title}: {n}") if ln == f"# {title}" else ln for ln in lines]
        with open(path, "w") as f:
            f.write("\n".join(head + body.get(n, [])) + "\n")


def counters_summary(csv_path: str, out_path: str, title: str, command: str,
                     kernels: str) -> None:
    """Writes a markdown summary of a rocprofv3 --pmc counter file: for each
    kernel whose name holds one of `kernels` (comma-separated), by grid and
    workgroup size, the dispatches and the mean of every counter per
    dispatch."""
    import csv
    keys = [k for k in kernels.split(",") if k]
    vals = {}
    counters = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not any(k in name for k in keys):
                continue
            short = name.replace("(anonymous namespace)::", "").replace("tis::", "")
            short = short.replace("void ", "", 1).split("(")[0]
            c = r["Counter_Name"]
            if c not in counters:
                counters.append(c)
            key = (short, r.get("Grid_Size", "?"), r.get("Workgroup_Size", "?"))
            vals.setdefault(key, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    lines = [f"# {title}", "", "Command (run from the repository root):", "", "```", command,
             "```", "", "Mean per dispatch of each counter (rocprofv3 --pmc).", "",
             "| kernel | grid x workgroup (threads) | dispatches | " + " | ".join(counters) + " |",
             "|---|---|---|" + "---|" * len(counters)]
    for (short, g, w), cs in sorted(vals.items()):
        n = max(len(v) for v in cs.values())
        cells = []
        for c in counters:
            xs = cs.get(c, [])
            m = sum(xs) / len(xs) if xs else float("nan")
            cells.append(f"{m:.4g}" if abs(m) < 1e6 else f"{m:.4e}")
        lines.append(f"| `{short}` | {g} x {w} | {n} | " + " | ".join(cells) + " |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")


# --------------------------------------------------------------- probes --

class Probes:
    """The library's measurement probes on torch buffers: a 1 GiB streaming
    read (the read ceiling, and the cache flush before cold timings) and a
    dependent-load chase (latency of one round trip)."""

    def __init__(self, tis, torch, dev):
        self.torch = torch
        self.lib = tis.ops.lib()
        self.dev = dev
        self.buf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        self._check = tis.ops.check
        self._stream = tis.ops._stream

    def read(self, t=None, nbytes=None, nontemporal=False):
        t = self.buf if t is None else t
        n = t.numel() * t.element_size() if nbytes is None else nbytes
        n -= n % 16
        self._check(self.lib.tis_probe_read(t.data_ptr(), n, int(nontemporal),
                                            self.sink.data_ptr(), self._stream(self.dev)))

    def flush(self):
        self.read()

    def marker(self, k: int):
        """A probe read of (k + 1) MiB: a dispatch of 64 (k + 1) workgroups
        that marks, in a kernel trace, where the measurement of the k-th
        workload begins."""
        self.read(nbytes=(k + 1) << 20)

    def read_ceiling(self, reps=4, nbytes=4 << 30):
        """GB/s of back-to-back reads of a 4 GiB buffer (16 times the
        Infinity Cache, so each read finds nothing of its data cached)."""
        torch = self.torch
        buf = torch.ones(nbytes, dtype=torch.uint8, device=self.dev)
        out = {}
        for nt in (False, True):
            self.read(buf, nontemporal=nt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                self.read(buf, nontemporal=nt)
            e1.record()
            torch.cuda.synchronize()
            out["nontemporal" if nt else "plain"] = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del buf
        return out

    def chase(self, footprint: int, hops: int, cold: bool, seed: int = 7):
        """Microseconds per dependent load on a random cycle through
        footprint / 128 cache-line slots, `hops` links from one start: cold
        (caches emptied first, so every hop goes to HBM, through TLB misses
        across the footprint) or warm (the same links walked just before, so
        the hops find whichever cache holds hops * 128 bytes of lines).
        Per hop = (time of `hops` hops - time of none) / hops."""
        import numpy as np
        torch = self.torch
        n = footprint // 4
        slots = n // 32
        rng = np.random.default_rng(seed)
        perm = rng.permutation(slots).astype(np.int64)
        nxt = np.zeros(n, dtype=np.uint32)
        nxt[perm * 32] = np.roll(perm, -1) * 32
        dnext = torch.from_numpy(nxt.view(np.int32)).to(self.dev)
        out = torch.zeros(1, dtype=torch.int32, device=self.dev)
        start = int(perm[0] * 32)

        def run(h):
            self._check(self.lib.tis_probe_chase(dnext.data_ptr(), n, start, h, out.data_ptr(),
                                                 self._stream(self.dev)))

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(h):
            if cold:
                self.flush()
            else:
                run(hops)
            e0.record()
            run(h)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3

        timed(hops)
        t_h = float(np.median([timed(hops) for _ in range(5)]))
        t_0 = float(np.median([timed(0) for _ in range(5)]))
        del dnext
        return (t_h - t_0) / hops


# ------------------------------------------------------------- timings --

def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def graph_time(torch, fn, per_graph=20, replays=5):
    """Microseconds per call of fn, from a graph holding `per_graph` calls
    back to back, replayed `replays` times between events (median)."""
    import numpy as np
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    ts = []
    for _ in range(replays):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / per_graph)
    del g
    return float(np.median(ts))


def graph_diff(torch, prep, fn, per_graph=10, replays=5):
    """Microseconds of fn in the cache state prep() leaves: a graph of
    `per_graph` times (prep, fn) and a graph of `per_graph` times prep alone
    are replayed between events, and the difference of their median times
    is divided by per_graph.  The launches run back to back inside each
    graph, so no host gap or event sits between prep and fn, and the result
    is close to fn's kernel durations."""
    import numpy as np

    def capture(body):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            body()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                body()
        return g

    def both():
        prep()
        fn()
    ga, gb = capture(both), capture(prep)
    e0, e1 = _events(torch, 2)

    def once(g):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3
    ga.replay()
    gb.replay()
    torch.cuda.synchronize()
    # the two graphs alternate, so a drift of the clock or of the memory
    # system's state over the measurement falls on both alike
    ta, tb = [], []
    for _ in range(replays):
        ta.append(once(ga))
        tb.append(once(gb))
    t = (float(np.median(ta)) - float(np.median(tb))) / per_graph
    del ga, gb
    return t


def decode_regimes(torch, probes, plan):
    """Decode durations (us): cold (caches emptied by a 1 GiB read), steady
    (emptied, then the summaries read once: a decode loop that keeps the
    tree hot while keys and values come from HBM) and warm (back to back:
    repeated decodes of the same queries, whose blocks stay in the L2s)."""
    def steady_prep():
        probes.flush()
        probes.read(plan.summaries)
    # the decode is short beside the flush (about 190 us), so its cold
    # figures take more launches a graph and more replays than the rest
    return {"cold_us": graph_diff(torch, probes.flush, plan.decode, per_graph=20, replays=9),
            "steady_us": graph_diff(torch, steady_prep, plan.decode, per_graph=20, replays=9),
            "warm_us": graph_time(torch, plan.decode)}


def attend_comparison(torch, probes, plan):
    """The attention alone over the routed leaves, per query (tree_attend)
    and with the query heads of a KV head together (tree_attend_grouped),
    cold and warm (us); the grouped output's largest difference from the
    per-query one."""
    plan.route()
    plan.attend()
    torch.cuda.synchronize()
    ref = plan.out.clone()
    res = {"per_query_cold_us": graph_diff(torch, probes.flush, plan.attend, per_graph=20,
                                           replays=9),
           "per_query_warm_us": graph_time(torch, plan.attend, replays=3)}
    if plan.ws_grouped is not None:
        plan.attend_grouped()
        torch.cuda.synchronize()
        res["grouped_max_abs_diff"] = float((plan.out - ref).abs().max().item())
        res["grouped_cold_us"] = graph_diff(torch, probes.flush, plan.attend_grouped,
                                            per_graph=20, replays=9)
        res["grouped_warm_us"] = graph_time(torch, plan.attend_grouped, replays=3)
    return res


TIMELINE_SLOTS, TIMELINE_WAVES = 24, 16


def timeline_phases(st, khz: int, scored: int) -> dict:
    """Phase times (us from the launch's first wave entry) of one decode's
    timeline st [workgroups, 16 waves, 24 slots]: for each phase the median
    and the latest over the waves that passed it (the walking waves for the
    levels).  'K arrived' and 'V used' are each wave's first unit."""
    import numpy as np
    st = st.astype(np.int64)
    t0 = st[:, :, 0][st[:, :, 0] > 0].min()
    names = [(0, "entry", None)]
    for j in range(min(scored, 8)):
        names += [(8 + 2 * j, f"level {j + 1} scored", 8), (9 + 2 * j, f"level {j + 1} ranked", 8)]
    names += [(1, "descent done", None), (2, "first K load issued", None),
              (3, "K arrived", None), (4, "V used", None), (5, "units done", None),
              (6, "partials merged", None), (7, "end", None)]
    out = {}
    for k, nm, waves in names:
        v = st[:, :waves, k] if waves else st[:, :, k]
        v = v[v > 0]
        if v.size:
            us = (v - t0) * 1e3 / khz
            out[nm] = {"median_us": float(np.median(us)), "max_us": float(us.max())}
    return out


def decode_timeline(torch, probes, plan, w) -> dict:
    """Where a decode's time goes: the instrumented decode's phase stamps
    after a cache flush (cold) and right after two decodes (warm)."""
    lib = plan._lib
    khz = int(lib.tis_wall_clock_khz(torch.cuda.current_device()))
    if khz <= 0 or plan.summary_dtype == "fp8":
        return {}
    tl = torch.zeros(plan.timeline_bytes() // 8, dtype=torch.int64, device=plan.device)
    scored = w.levels - first_cut(w) + 1
    res = {"clock_khz": khz}
    for regime in ("cold", "warm"):
        plan.decode()
        plan.decode()
        if regime == "cold":
            probes.flush()
        tl.zero_()
        plan.decode_timeline(tl)
        torch.cuda.synchronize()
        st = tl.cpu().numpy().reshape(-1, TIMELINE_WAVES, TIMELINE_SLOTS)
        res[regime] = timeline_phases(st, khz, scored)
    return res


def decode_floor(w, ceil_gbs, hop_us, dec_bytes):
    """Latency floor of one decode: the scored levels and the gather form a
    chain of dependent round trips (the first level's rows, each later
    level's rows, then the leaf blocks), and the bytes cannot move faster
    than the streaming-read ceiling."""
    hops = w.levels - first_cut(w) + 2
    return hops * hop_us + dec_bytes / (ceil_gbs * 1e3)


def measure_workload(tis, torch, probes, w, ceil_gbs, hop_us, reps, headline=False, K=0, W=0,
                     index=0):
    """Cold build, decode regimes and bytes for one workload; with headline
    set, also the timed region of K cold steps (build + decode)."""
    import workloads
    t0 = time.time()
    probes.marker(index)
    x = workloads.generate(w, workers=min(16, os.cpu_count() or 1))
    dev = probes.dev
    Q, K_, V = (tis.from_storage(x[k], w.dtype, dev) for k in ("Q", "K", "V"))
    log(f"{w.name}: generated and uploaded in {time.time() - t0:.1f}s")
    plan = tis.DecodePlan(Q, K_, V, w.branching, w.leaf_block, w.levels, w.beam)
    by = algorithmic_bytes(w)
    dec_bytes = by["route"] + by["attend"]
    res = {"queries": w.queries, "n_keys": w.n_keys,
           "bytes": {"build": by["build"], "decode_per_query_sum": dec_bytes,
                     "route_per_query_sum": by["route"], "attend_per_query_sum": by["attend"],
                     "candidates_per_query": by["candidates_per_query"]}}
    step = None
    if headline:
        # the timed region: K cold steps (a 1 GiB read, then build and
        # decode), replayed from one graph between events, less the same K
        # reads alone
        def step_fn():
            plan.build()
            plan.decode()
        for _ in range(W):
            probes.flush()
            step_fn()
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        step_us = graph_diff(torch, probes.flush, step_fn, per_graph=K, replays=3)
        h1 = time.perf_counter()
        step = {"steps": K, "step_us_mean": step_us, "region_wall_s": h1 - h0}
    bc = graph_diff(torch, probes.flush, plan.build, per_graph=max(5, min(K, 20)), replays=7)
    if not headline:
        # the build then one decode, back to back (the decode finds the tree
        # the build just wrote): the literal sequence of the 1M-key workload
        def bd():
            plan.build()
            plan.decode()
        res["decode_after_build_us"] = graph_diff(torch, probes.flush, bd, per_graph=5,
                                                  replays=3) - bc
    res["build"] = {"cold_us": bc, "cold_gbs": by["build"] / (bc * 1e3),
                    "cold_frac": by["build"] / (bc * 1e3) / HBM_PEAK_GBS,
                    "warm_us": graph_time(torch, plan.build, per_graph=5, replays=3)}
    res["build"]["warm_frac"] = by["build"] / (res["build"]["warm_us"] * 1e3) / HBM_PEAK_GBS
    # the same bytes as the build's K, streamed by the read probe (cold): the
    # read ceiling at this size, ramp and tail included
    kread = graph_diff(torch, probes.flush, lambda: probes.read(K_, nontemporal=True),
                       per_graph=max(5, min(K, 20)), replays=7)
    kbytes = K_.numel() * K_.element_size()
    res["build"]["k_read_cold_us"] = kread
    res["build"]["k_read_cold_gbs"] = kbytes / (kread * 1e3)
    res["build"]["frac_of_k_read"] = kread / bc
    dr = decode_regimes(torch, probes, plan)
    dist, union = distinct_bytes(tis, w, Q, K_)
    floor = decode_floor(w, ceil_gbs, hop_us, dec_bytes)
    dec = {"regimes": dr, "bytes_distinct": dist, "leaf_union_fraction": union, "floor_us": floor,
           "floor_model": f"{w.levels - first_cut(w) + 2} dependent HBM round trips + "
                          "per-query-sum bytes at the read ceiling"}
    for r in ("cold", "steady", "warm"):
        t = dr[f"{r}_us"]
        dec[r] = {"us": t, "queries_per_s": w.queries / (t * 1e-6),
                  "gbs": dec_bytes / (t * 1e3), "frac": dec_bytes / (t * 1e3) / HBM_PEAK_GBS,
                  "gbs_distinct": dist / (t * 1e3),
                  "frac_distinct": dist / (t * 1e3) / HBM_PEAK_GBS,
                  "floor_ratio": t / floor}
    dec["timeline"] = decode_timeline(torch, probes, plan, w)
    res["decode"] = dec
    res["attend_only"] = attend_comparison(torch, probes, plan)
    if step is not None:
        res["step"] = step
    log(f"{w.name}: build cold {bc:.1f} us ({res['build']['cold_frac']:.1%} of 8 TB/s on "
        f"{by['build'] / 1e6:.1f} MB; {kread / bc:.1%} of a cold streaming read of K, "
        f"{kread:.1f} us), warm {res['build']['warm_us']:.1f} us; leaf union "
        f"{union:.2f}; decode cold "
        f"{dr['cold_us']:.2f} / steady {dr['steady_us']:.2f} / warm {dr['warm_us']:.2f} us "
        f"({dec['cold']['frac']:.1%} / {dec['steady']['frac']:.1%} / {dec['warm']['frac']:.1%} "
        f"on {dec_bytes / 1e6:.2f} MB per-query sum; {dec['cold']['frac_distinct']:.1%} cold on "
        f"{dist / 1e6:.2f} MB distinct); floor {floor:.2f} us; attend alone cold per query "
        f"{res['attend_only']['per_query_cold_us']:.2f} us, grouped "
        f"{res['attend_only'].get('grouped_cold_us', float('nan')):.2f} us")
    tlc = dec["timeline"].get("cold", {})
    if tlc:
        log(f"{w.name}: cold decode timeline (median / latest wave, us): " + "; ".join(
            f"{k} {v['median_us']:.2f}/{v['max_us']:.2f}" for k, v in tlc.items()))
    return res, (x, Q, K_, V, plan)


# ----------------------------------------------------- the other legs --

def cpu_baseline(w, x, min_seconds: float = 10.0, max_reps: int = 500):
    """The CPU oracle, as it stands, on whole steps of the same workload."""
    from oracle import tis_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
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
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": reps * w.queries / el, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_affinity_cpus": affinity,
            "blas_threads_default": blas[0] if blas else None,
            "sample": f"{reps} whole steps (build over all {w.batch * w.kv_heads} KV heads, "
                      f"route + attend of all {w.queries} queries) of the same workload, "
                      f"numpy fp64 on one thread (BLAS limited to 1; the oracle's other work "
                      f"is single-threaded numpy), {el:.1f} s"}


def per_launch(torch, fn, reps):
    """Average duration (s) of fn's launch: reps launches back to back
    between one event pair."""
    e0, e1 = _events(torch, 2)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def reduced_summaries(tis, torch, w, Q, K, V, summary_dtype):
    """The step with summaries stored as bfloat16 or fp8 (the same means
    rounded once to the narrower type): warm build and decode durations
    (graph replay) and the decode's rate on its own algorithmic bytes."""
    plan = tis.DecodePlan(Q, K, V, w.branching, w.leaf_block, w.levels, w.beam,
                          summary_dtype=summary_dtype)
    plan.build()
    plan.decode()
    build_us = graph_time(torch, plan.build, per_graph=5, replays=3)
    decode_us = graph_time(torch, plan.decode)
    by = algorithmic_bytes(w, summary_dtype)
    dec = by["route"] + by["attend"]
    return {"regime": f"warm (graph replay), summaries stored as {summary_dtype}",
            "build_us": build_us, "build_gbs": by["build"] / (build_us * 1e3),
            "decode_us": decode_us, "decode_queries_per_s": w.queries / (decode_us * 1e-6),
            "decode_gbs": dec / (decode_us * 1e3),
            "decode_frac": dec / (decode_us * 1e3) / HBM_PEAK_GBS, "decode_bytes": dec}


def threshold_retrieval(tis, torch, w, Q, K, V, reps, k_ranks=(64, 512)):
    """Bounding-sphere threshold retrieval on the step's data: the radii pass
    over K, then the fused threshold decode at thresholds halfway between
    each query's k-th and (k+1)-th best key score (set up with a dense torch
    matmul, not timed)."""
    tree = tis.tree_build(K, w.branching, w.leaf_block, w.levels)
    radii = tis.tree_radii(K, tree)
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
        dec_s = per_launch(torch, lambda: tis.tree_decode_threshold(
            Q, K, V, tree, radii, tau, max_nodes, out=o), reps)
        c = cnt.float()
        kept_bytes = float(c.clamp(min=0).sum()) * w.leaf_block * w.head_dim * w.elem_bytes * 2
        out["thresholds"].append({
            "k": k, "decode_us": dec_s * 1e6, "queries_per_s": w.queries / dec_s,
            "leaves_kept_mean": float(c.mean()), "leaves_kept_max": int(c.max()),
            "overflow": int((cnt < 0).sum()), "gathered_gbs": kept_bytes / dec_s / 1e9})
    return out


def causal_prefill_bench(tis, torch, w, Q, K, V, reps, max_positions=4096):
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
    ct.causal_prefill(Qp, w.beam, out=out)
    t = per_launch(torch, lambda: ct.causal_prefill(Qp, w.beam, out=out), max(3, min(reps, 10)))
    pos = torch.arange(P, device=Q.device).view(1, 1, P, 1)
    blk = idx.long()
    size = torch.clamp(pos + 1 - blk * w.leaf_block, max=w.leaf_block)
    reads = torch.where(blk >= 0, size, torch.zeros_like(size)).sum(-1).double()
    queries = w.batch * w.q_heads * P
    return {"positions": P, "queries": queries, "us": t * 1e6, "queries_per_s": queries / t,
            "keys_read_mean": float(reads.mean()), "dense_causal_keys_mean": (P + 1) / 2}


def cache_decode_loop(tis, torch, w, K, V, Q, steps):
    """The decode loop over a growing cache of the same shape: the tree over
    the first keys of the cache is filled by one long append, then every
    step appends one key per head and decodes every query, as two calls and
    as the fused call (tis_cache_tree_append_decode).  Appends change the
    tree, so these launches run eagerly, back to back."""
    need = 4 * (steps + 4) + 8
    prefill = w.n_keys - need
    if prefill < 1:
        return None
    ct = tis.CacheTree(K, V, w.branching, w.leaf_block)
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=torch.float32, device=K.device)

    def timed(fn, reps):
        return per_launch(torch, fn, reps) * 1e6

    ct.append(prefill)
    ct.reset()
    prefill_us = timed(lambda: ct.append(prefill), 1)
    decode = ct.bind_decode(Q, w.beam, out)
    step = lambda: (ct.append(1), decode())
    for _ in range(2):
        step()
    step_us = timed(step, steps)
    append_us = timed(lambda: ct.append(1), steps)
    decode_us = timed(decode, steps)
    fused = ct.bind_decode(Q, w.beam, out, append=True)
    for _ in range(2):
        fused()
    fused_us = timed(fused, steps)
    kbytes = prefill * w.batch * w.kv_heads * w.head_dim * w.elem_bytes
    return {"regime": "tree over the first n keys of a cache of the workload's size; "
                      "one key appended per head per step; eager launches back to back",
            "n_keys_at_end": ct.n_keys, "levels": ct.levels,
            "prefill_keys": prefill, "prefill_us": prefill_us,
            "prefill_gbs": kbytes / (prefill_us * 1e-6) / 1e9,
            "append1_us": append_us, "decode_us": decode_us, "step_us": step_us,
            "queries_per_s": w.queries / (step_us * 1e-6),
            "fused_step_us": fused_us, "fused_queries_per_s": w.queries / (fused_us * 1e-6)}


# ----------------------------------------------------------------- main --

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed cold steps of the headline")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="the headline workload")
    ap.add_argument("--others", default=",".join(OTHERS),
                    help="comma-separated workloads also measured ('none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the growing-cache loop, reduced-precision summaries, bounding "
                         "spheres and causal prefill legs")
    ap.add_argument("--prefill-positions", type=int, default=4096,
                    help="positions of the causal prefill leg (at most the workload's keys)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (the reference "
                         "dispatch for scaling HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files (FETCH_SIZE, WRITE_SIZE) of "
                         "a --calibrate-copy run into profiles/traffic_<workload>.json and exit")
    ap.add_argument("--trace-summary", nargs=5,
                    metavar=("DB", "OUT_MD", "TITLE", "COMMAND", "SEGMENTS"),
                    help="write a markdown kernel-trace summary of a rocprofv3 database (its "
                         "workload segments named by SEGMENTS, comma-separated) and exit")
    ap.add_argument("--counters-from", nargs=5,
                    metavar=("CSV", "OUT_MD", "TITLE", "COMMAND", "KERNELS"),
                    help="write a markdown summary of a rocprofv3 --pmc counter file for the "
                         "kernels named by KERNELS (comma-separated substrings) and exit")
    args = ap.parse_args(argv)
    if args.counters_from:
        counters_summary(*args.counters_from)
        return 0
    if args.traffic_from:
        print(json.dumps(traffic_from_counters(args.workload, *args.traffic_from)))
        return 0
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); every tree is "
              "independent per (batch, KV head), so N GPUs would each run their own share "
              "with no exchange", file=sys.stderr)
        return 2

    import torch
    import workloads
    import tree_indexed_sparse_build_amd as tis

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    log(f"{tis.version()}; device {torch.cuda.get_device_name(0)}")
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    probes = Probes(tis, torch, dev)
    ceil = probes.read_ceiling()
    # cold: 2,000 hops over a 1 GiB footprint after the caches are emptied;
    # Infinity Cache: 131,072 warm hops (16 MB of lines, more than an XCD's
    # 4 MB L2, far less than the 256 MB cache); L2: 2,000 warm hops (256 KB)
    hop = {"hbm_cold": probes.chase(FLUSH_BYTES, 2000, cold=True),
           "infinity_cache_warm": probes.chase(64 << 20, 131072, cold=False),
           "l2_warm": probes.chase(1 << 20, 2000, cold=False)}
    log(f"read ceiling {ceil['plain']:.0f} GB/s plain, {ceil['nontemporal']:.0f} GB/s "
        f"nontemporal (4 GiB, back to back); dependent load {hop['hbm_cold']:.3f} us cold "
        f"(1 GiB footprint), {hop['infinity_cache_warm']:.3f} us (Infinity Cache), "
        f"{hop['l2_warm']:.3f} us (L2)")
    ceil_gbs = max(ceil.values())

    w = workloads.get(args.workload)
    K_ = args.steps
    head, (x, Q, K, V, plan) = measure_workload(tis, torch, probes, w, ceil_gbs, hop["hbm_cold"],
                                                reps=K_, headline=True, K=K_, W=args.warmup)
    step = head["step"]
    by = algorithmic_bytes(w)
    build_gbs = head["build"]["cold_gbs"]

    extras = {}
    if not args.no_extras:
        extras["causal_prefill"] = causal_prefill_bench(tis, torch, w, Q, K, V, K_,
                                                        max_positions=args.prefill_positions)
        p = extras["causal_prefill"]
        log(f"causal prefill of the first {p['positions']} keys ({p['queries']} queries): "
            f"{p['us']:.1f} us -> {p['queries_per_s']:.3e} queries/s; keys read per query "
            f"{p['keys_read_mean']:.2f} (dense causal {p['dense_causal_keys_mean']:.1f})")
        extras["threshold_retrieval"] = threshold_retrieval(tis, torch, w, Q, K, V, K_)
        t = extras["threshold_retrieval"]
        log(f"bounding spheres: radii {t['radii_us']:.1f} us; " + "; ".join(
            f"k={r['k']}: decode {r['decode_us']:.2f} us, leaves kept {r['leaves_kept_mean']:.1f}"
            f", overflow {r['overflow']}" for r in t["thresholds"]))
        extras["reduced_summaries"] = {sd: reduced_summaries(tis, torch, w, Q, K, V, sd)
                                       for sd in ("bf16", "fp8")}
        for sd, r in extras["reduced_summaries"].items():
            log(f"{sd} summaries (warm): build {r['build_us']:.1f} us, decode {r['decode_us']:.2f}"
                f" us ({r['decode_frac']:.1%} on {r['decode_bytes'] / 1e6:.2f} MB)")
        extras["cache_decode_loop"] = cache_decode_loop(tis, torch, w, K, V, Q, K_)
        c = extras["cache_decode_loop"]
        if c:
            log(f"growing cache: prefill append {c['prefill_us']:.1f} us; append 1 "
                f"{c['append1_us']:.2f} us; decode {c['decode_us']:.2f} us; fused step "
                f"{c['fused_step_us']:.2f} us")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w, x)
        log(f"cpu oracle {cpu['value']:.2f} queries/s ({cpu['sample']})")
    del x, Q, K, V, plan
    torch.cuda.empty_cache()

    others = {}
    names = [] if args.others in ("", "none") else [n for n in args.others.split(",") if n]
    for k, name in enumerate(names, start=1):
        r, bufs = measure_workload(tis, torch, probes, workloads.get(name), ceil_gbs,
                                   hop["hbm_cold"], reps=10, index=k)
        others[name] = r
        del bufs
        torch.cuda.empty_cache()

    d = head["decode"]
    line = {
        "metric": "decode queries/sec + achieved HBM GB/s (% roofline) at N=32K–1M keys",
        "value": w.queries / (step["step_us_mean"] * 1e-6),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": step["step_us_mean"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 inputs; fp64 build sums and route scores; fp32 attention",
        "data": "synthetic (seeded clustered-Gaussian keys, see workloads/__init__.py)",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim, "n_keys": w.n_keys,
                   "branching": w.branching, "leaf_block": w.leaf_block, "levels": w.levels,
                   "beam": w.beam,
                   "step": "tree_build + tree_decode (tree_route and tree_attend in one launch)",
                   "cache_state": "cold: a 1 GiB streaming read before each timed step, not "
                                  "counted (the K steps, each after its read, are replayed "
                                  "from one graph between events; the same K reads alone are "
                                  "timed the same way and subtracted)"},
        "roofline": {"kernel": "k_build (tree_build)", "bound": "hbm", "achieved": build_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": build_gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic(w.name), "regime": "cold (caches emptied first)",
                     "launch_us_mean": head["build"]["cold_us"],
                     "warm_frac": head["build"]["warm_frac"],
                     "read_ceiling_frac": build_gbs / ceil_gbs,
                     "frac_of_k_read": head["build"]["frac_of_k_read"]},
        "decode": {"queries_per_s_cold": d["cold"]["queries_per_s"],
                   "queries_per_s_steady": d["steady"]["queries_per_s"],
                   "queries_per_s_warm": d["warm"]["queries_per_s"],
                   "frac_cold": d["cold"]["frac"], "frac_steady": d["steady"]["frac"],
                   "frac_warm": d["warm"]["frac"],
                   "frac_distinct_cold": d["cold"]["frac_distinct"],
                   "regime_note": "cold: caches emptied; steady: emptied, then the summaries "
                                  "read once (a decode loop keeping the tree hot); warm: "
                                  "back-to-back launches replayed from a graph"},
        "ceilings": {"read_gbs": ceil, "dependent_load_us": hop},
        "workloads": dict({w.name: head}, **others),
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
