"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Every case draws seeded inputs from `workloads`, runs tree_build, tree_route
(with trace) and tree_attend on the GPU, and compares with the oracle under
the rules in tests/parity.py.  Reduced cases keep each workload's generator,
branching, leaf block, beam and head grouping at fewer levels / heads; the
full-size cases run the five page-shaped workloads at their real sizes in
the launch configuration the benchmark times.
"""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import pytest

import workloads
from oracle import tis_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()  # raises if libtis.so is missing
    return t


def grouped_supported(w) -> bool:
    """The grouped attend takes up to 64 query heads per KV head and 512
    slots per group."""
    return w.group <= 64 and w.group * w.beam <= 512


def run_gpu(t, w, x, oracle_idx=None, summary_dtype="f32"):
    dev = "cuda"
    K = t.from_storage(x["K"], w.dtype, dev)
    V = t.from_storage(x["V"], w.dtype, dev)
    Q = t.from_storage(x["Q"], w.dtype, dev)
    tree = t.tree_build(K, w.branching, w.leaf_block, w.levels, summary_dtype=summary_dtype)
    idx, tr = t.tree_route(Q, tree, w.beam, trace=True)
    out = t.tree_attend(Q, K, V, idx, w.leaf_block)
    res = {"tree": tree, "idx": idx, "trace": tr, "out": out}
    if oracle_idx is not None:
        oi = torch.from_numpy(np.ascontiguousarray(oracle_idx, dtype=np.int32)).to(dev)
        res["out_oracle_idx"] = t.tree_attend(Q, K, V, oi, w.leaf_block)
    res["fused_out"], res["fused_idx"] = t.tree_decode(Q, K, V, tree, w.beam, return_indices=True)
    if grouped_supported(w):
        res["grouped_out"] = t.tree_attend_grouped(Q, K, V, idx, w.leaf_block)
    else:
        with pytest.raises(t.TisError, match="TIS_E_UNSUPPORTED"):
            t.tree_attend_grouped(Q, K, V, idx, w.leaf_block)
    torch.cuda.synchronize()
    res["levels"] = [tree.level(l).float().cpu().numpy() for l in range(1, w.levels + 1)]
    for k in ("idx", "trace", "out", "out_oracle_idx", "fused_out", "fused_idx", "grouped_out"):
        if k in res:
            res[k] = res[k].cpu().numpy()
    return res


def check_case(t, w, x=None, label="", summary_dtype="f32", max_excused=None):
    t0 = time.time()
    if x is None:
        x = workloads.generate(w)
    _say(f"{label or w.name}: generated in {time.time() - t0:.1f}s "
         f"(B={w.batch} Hq={w.q_heads} Hkv={w.kv_heads} d={w.head_dim} N={w.n_keys} "
         f"b={w.branching} L={w.leaf_block} lv={w.levels} W={w.beam} {w.dtype}; "
         f"{summary_dtype} summaries)")
    ob = O.tree_build(x["K"], w.dtype, w.branching, w.leaf_block, w.levels,
                      summary_dtype=summary_dtype)
    orr = O.tree_route(x["Q"], w.dtype, ob["stored"], w.branching, w.beam)
    _say(f"{label or w.name}: oracle build+route done at {time.time() - t0:.1f}s")
    g = run_gpu(t, w, x, oracle_idx=orr["indices"], summary_dtype=summary_dtype)
    eq, tot, worst = parity.compare_summaries(g["levels"], ob["stored"],
                                              summary_dtype=summary_dtype)
    exact, tie, nq = parity.compare_indices(g["idx"], orr, max_excused=max_excused)
    parity.compare_trace(g["trace"], orr)
    o_or = O.tree_attend(x["Q"], x["K"], x["V"], w.dtype, orr["indices"], w.leaf_block)
    err1 = parity.compare_outputs(g["out_oracle_idx"], o_or, w.dtype)
    # every query's output is also checked on the leaves the GPU chose
    o_g = O.tree_attend(x["Q"], x["K"], x["V"], w.dtype, g["idx"], w.leaf_block)
    err2 = parity.compare_outputs(g["out"], o_g, w.dtype)
    # the fused decode keeps the same leaves and attends over them
    assert np.array_equal(g["fused_idx"], g["idx"]), "fused decode kept other leaves"
    err3 = parity.compare_outputs(g["fused_out"], o_g, w.dtype)
    # the grouped attend over the same leaves
    err4 = (parity.compare_outputs(g["grouped_out"], o_g, w.dtype)
            if "grouped_out" in g else float("nan"))
    _say(f"{label or w.name}: summaries bit-equal {eq}/{tot} (worst {worst} ulp); "
         f"indices exact {exact}/{nq}, tie-exposed mismatches {tie}; "
         f"attend max-abs {err1:.2e} (oracle idx) {err2:.2e} (gpu idx) {err3:.2e} (fused) "
         f"{err4:.2e} (grouped); "
         f"min cut gap {float(np.min(orr['gap'])):.2e}; {time.time() - t0:.1f}s")
    return x, ob, orr, g


# ---------------------------------------------------------------- reduced --
REDUCED = [
    ("alhr_1k", None, None),          # the full 1,024-key case is already small
    ("gqa_32k", 2, 2),
    ("gqa_256k", 2, 2),
    ("long_1m", 3, 1),
    ("deep_planted", 4, 2),
]


@pytest.mark.parametrize("name,levels,kvh", REDUCED, ids=[r[0] for r in REDUCED])
def test_reduced_workload(tis, name, levels, kvh):
    w = workloads.get(name) if levels is None else workloads.small(name, levels=levels,
                                                                   kv_heads=kvh)
    check_case(tis, w)


def _custom(name, dtype, b, L, lv, W, d=128, B=1, Hkv=2, G=3, gen="normal", seed=11):
    return workloads.Workload(name, dtype, B, Hkv * G, Hkv, d, b, L, lv, W, gen, seed=seed)


EDGE = [
    # ragged leaf blocks against the 2/4/8 rows one wave-wide load covers
    _custom("ragged_f32_d64", "f32", 3, 5, 3, 4, d=64),
    _custom("ragged_bf16_d64", "bf16", 3, 5, 3, 4, d=64),
    _custom("ragged_bf16_d128", "bf16", 3, 7, 3, 5, d=128, B=2),
    _custom("ragged_f32_d128", "f32", 5, 3, 2, 7, d=128),
    # one level: block top-k then softmax on the kept blocks
    _custom("single_level", "bf16", 16, 8, 1, 5),
    _custom("single_level_wide", "f32", 64, 4, 1, 4, d=64),
    # widest candidate set (beam * branching = 256) and beam 1
    _custom("cand_256", "bf16", 16, 4, 2, 16),
    _custom("beam_1", "bf16", 4, 16, 4, 1),
    # beam = every leaf: the final attention is dense
    _custom("full_beam", "f32", 2, 8, 4, 16, d=64),
    # long leaf blocks (several batches of rows per wave)
    _custom("long_leaf", "bf16", 2, 200, 2, 2),
    # deep binary tree: the last chunk of each level-1 subtree climbs 4
    # levels above the chunk roots
    _custom("deep_binary", "bf16", 2, 4, 9, 6, d=64, Hkv=3, G=1),
    # the deepest tree the library takes: 16 levels (binary, leaf blocks of
    # one key, 65,536 keys); a level-1 subtree too wide for the build's LDS,
    # so the levels above the chunk roots take one small launch each
    _custom("max_levels_16", "f32", 2, 1, 16, 3, d=64, Hkv=1, G=2),
    # many heads, GQA group 8, batch 3
    _custom("gqa8_batch3", "bf16", 4, 32, 3, 6, B=3, Hkv=2, G=8),
    # few queries with long key sets: each query split over several
    # workgroups (64 x 64 keys, 6 queries -> 32 parts each), merged after
    _custom("split_long_gather", "bf16", 4, 64, 4, 64, Hkv=2, G=3),
    _custom("split_long_gather_f32", "f32", 8, 128, 2, 32, d=64, Hkv=1, G=2),
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
def test_edge_geometry(tis, w):
    check_case(tis, w)


def test_full_beam_is_dense_attention(tis):
    w = _custom("dense_check", "bf16", 4, 16, 2, 16, d=128)
    x = workloads.generate(w)
    g = run_gpu(tis, w, x)
    assert np.all(g["idx"] == np.arange(16, dtype=np.int32))
    k = O.widen(x["K"], w.dtype)
    v = O.widen(x["V"], w.dtype)
    q = O.widen(x["Q"], w.dtype)
    for hq in range(w.q_heads):
        kk, vv = k[0, hq // w.group], v[0, hq // w.group]
        s = kk @ q[0, hq] / math.sqrt(w.head_dim)
        p = np.exp(s - s.max())
        want = p @ vv / p.sum()
        assert np.max(np.abs(g["out"][0, hq] - want)) <= parity.ATTEND_TOL["bf16"]


def test_attend_slot_rules(tis):
    """Duplicates count once, negative slots are empty, an all-empty row is
    zero, an out-of-range block makes the row NaN (and nothing else)."""
    w = _custom("slots", "bf16", 4, 16, 2, 4, Hkv=1, G=6)
    x = workloads.generate(w)
    n_blocks = w.n_keys // w.leaf_block
    idx = np.array([[[3, 3, 7, -1],
                     [-1, -1, -1, -1],
                     [0, 1, 2, 15],
                     [5, n_blocks, 1, 2],
                     [9, -5, 9, 9],
                     [15, 14, 13, 12]]], dtype=np.int32)
    K = tis.from_storage(x["K"], w.dtype)
    V = tis.from_storage(x["V"], w.dtype)
    Q = tis.from_storage(x["Q"], w.dtype)
    out = tis.tree_attend(Q, K, V, torch.from_numpy(idx).cuda(), w.leaf_block).cpu().numpy()
    safe = idx.copy()
    safe[0, 3] = -1  # the oracle refuses out-of-range blocks; compare the other rows
    want = O.tree_attend(x["Q"], x["K"], x["V"], w.dtype, safe, w.leaf_block)
    for r in (0, 2, 4, 5):
        assert np.max(np.abs(out[0, r] - want[0, r])) <= parity.ATTEND_TOL["bf16"]
    assert np.all(out[0, 1] == 0.0)
    assert np.all(np.isnan(out[0, 3]))


def test_grouped_attend_slot_rules(tis):
    """The grouped attend applies the slot rules per head: a leaf kept by
    several heads of the group, repeats and negatives within a head, an
    empty head, an out-of-range block in one head only."""
    w = _custom("slots_grouped", "bf16", 4, 16, 2, 4, Hkv=1, G=6)
    x = workloads.generate(w)
    n_blocks = w.n_keys // w.leaf_block
    idx = np.array([[[3, 3, 7, -1],
                     [-1, -1, -1, -1],
                     [0, 1, 2, 15],
                     [5, n_blocks, 1, 2],
                     [9, -5, 9, 9],
                     [15, 14, 13, 12]]], dtype=np.int32)
    K = tis.from_storage(x["K"], w.dtype)
    V = tis.from_storage(x["V"], w.dtype)
    Q = tis.from_storage(x["Q"], w.dtype)
    out = tis.tree_attend_grouped(Q, K, V, torch.from_numpy(idx).cuda(),
                                  w.leaf_block).cpu().numpy()
    safe = idx.copy()
    safe[0, 3] = -1
    want = O.tree_attend(x["Q"], x["K"], x["V"], w.dtype, safe, w.leaf_block)
    for r in (0, 2, 4, 5):
        assert np.max(np.abs(out[0, r] - want[0, r])) <= parity.ATTEND_TOL["bf16"]
    assert np.all(out[0, 1] == 0.0)
    assert np.all(np.isnan(out[0, 3]))


GROUPED_CASES = [
    # 32 and 48 heads per KV head: two and four blocks of 16 heads
    _custom("grouped_g32", "bf16", 4, 32, 2, 4, Hkv=1, G=32),
    _custom("grouped_g48_f32", "f32", 4, 16, 3, 8, d=64, Hkv=2, G=48),
    # 16 heads, ragged leaf blocks (not a multiple of 16 keys)
    _custom("grouped_g16_ragged", "bf16", 8, 24, 2, 8, Hkv=2, G=16),
    # 256 groups: one workgroup per group, no split
    _custom("grouped_unsplit", "bf16", 2, 16, 2, 2, B=64, Hkv=4, G=2),
    _custom("grouped_unsplit_f32", "f32", 2, 32, 2, 2, d=64, B=32, Hkv=8, G=3),
]


@pytest.mark.parametrize("w", GROUPED_CASES, ids=[w.name for w in GROUPED_CASES])
def test_grouped_geometry(tis, w):
    check_case(tis, w)


def test_deterministic(tis):
    w = workloads.small("gqa_256k", levels=2, kv_heads=2)
    x = workloads.generate(w)
    a = run_gpu(tis, w, x)
    b = run_gpu(tis, w, x)
    for la, lb in zip(a["levels"], b["levels"]):
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))


def test_planted_blocks_retrieved(tis):
    w = workloads.small("deep_planted", levels=4, kv_heads=2)
    x = workloads.generate(w)
    g = run_gpu(tis, w, x)
    hit = [x["planted"][0, h] in g["idx"][0, h] for h in range(w.q_heads)]
    assert all(hit), f"planted block missed by {hit.count(False)} queries"


def test_errors_through_binding(tis):
    K = torch.zeros((1, 1, 96, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tis.TisError, match="TIS_E_SHAPE"):
        tis.tree_build(K, 2, 16, 3)  # 2^3 * 16 = 128 != 96
    K = torch.zeros((1, 1, 128, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tis.TisError, match="TIS_E_UNSUPPORTED"):
        tis.tree_build(K, 2, 16, 3)
    K = torch.zeros((1, 2, 128, 64), dtype=torch.float32, device="cuda")
    tree = tis.tree_build(K, 2, 16, 3)
    Q = torch.zeros((1, 3, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(tis.TisError, match="TIS_E_SHAPE"):
        tis.tree_route(Q, tree, 2)  # 3 q heads over 2 KV heads
    Q = torch.zeros((1, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(tis.TisError, match="TIS_E_SHAPE"):
        tis.tree_route(Q, tree, 9)  # beam > 8 leaves
    torch.cuda.synchronize()


# ------------------------------------------------------ random geometries --
def _random_geometries(n=24, seed=2024):
    """Seeded small geometries across branching, depth, leaf size, beam, head
    dim, input type and GQA group, kept small enough for the oracle: they
    reach the build's single-kernel and climbing plans, unscored levels,
    beams from 1 to every leaf, and split and unsplit attention."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        b = int(rng.choice([2, 3, 4, 5, 8]))
        lv = int(rng.integers(1, 6))
        L = int(rng.choice([1, 3, 4, 8, 16, 32, 64, 96]))
        leaves = b ** lv
        if leaves * L > (1 << 15) or leaves > 4096:
            continue
        W = int(rng.integers(1, min(leaves, 256 // b) + 1))
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f32", "bf16"]))
        B = int(rng.integers(1, 3))
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4, 8]))
        name = f"rand{len(out)}_b{b}_lv{lv}_L{L}_W{W}_d{d}_{dtype}_B{B}_{Hkv}x{G}"
        out.append(workloads.Workload(name, dtype, B, Hkv * G, Hkv, d, b, L, lv, W, "normal",
                                      seed=100 + len(out)))
    return out


RANDOM = _random_geometries()


@pytest.mark.parametrize("w", RANDOM, ids=[w.name for w in RANDOM])
def test_random_geometry(tis, w):
    check_case(tis, w)


# -------------------------------------------------------------- full size --
# bfloat16 summaries: the build rounds every mean straight from fp64 and the
# walk reads 8 summary elements per 16-byte load (both head dims, the
# single-launch builds, builds that climb above the chunk roots, splits)
BF16_SUMMARY_CASES = [
    workloads.small("gqa_32k", levels=2, kv_heads=2),
    workloads.small("deep_planted", levels=4, kv_heads=2),
    workloads.small("long_1m", levels=3, kv_heads=1),
    _custom("bf16s_ragged_f32_d64", "f32", 3, 5, 3, 4, d=64),
    _custom("bf16s_single_level", "bf16", 16, 8, 1, 5),
    _custom("bf16s_cand_256", "bf16", 16, 4, 2, 16),
    _custom("bf16s_deep_binary", "bf16", 2, 4, 9, 6, d=64, Hkv=3, G=1),
    _custom("bf16s_split", "bf16", 4, 64, 4, 64, Hkv=2, G=3),
]


@pytest.mark.parametrize("w", BF16_SUMMARY_CASES, ids=[w.name for w in BF16_SUMMARY_CASES])
def test_bf16_summaries(tis, w):
    check_case(tis, w, label=f"{w.name} (bf16 summaries)", summary_dtype="bf16")


# fp8 summaries (full tree): per-row scales from a wave-wide max in the
# build's leaf and node stores, the LDS levels and the climb above the chunk
# roots; the walk reads 8 codes a lane and scales each row's partial dot
FP8_SUMMARY_CASES = [
    workloads.small("gqa_32k", levels=2, kv_heads=2),
    workloads.small("deep_planted", levels=4, kv_heads=2),
    workloads.small("long_1m", levels=3, kv_heads=1),
    _custom("fp8s_ragged_f32_d64", "f32", 3, 5, 3, 4, d=64),
    _custom("fp8s_single_level", "bf16", 16, 8, 1, 5),
    _custom("fp8s_cand_256", "bf16", 16, 4, 2, 16),
    _custom("fp8s_deep_binary", "bf16", 2, 4, 9, 6, d=64, Hkv=3, G=1),
    _custom("fp8s_split", "bf16", 4, 64, 4, 64, Hkv=2, G=3),
]


@pytest.mark.parametrize("w", FP8_SUMMARY_CASES, ids=[w.name for w in FP8_SUMMARY_CASES])
def test_fp8_summaries(tis, w):
    check_case(tis, w, label=f"{w.name} (fp8 summaries)", summary_dtype="fp8")


@pytest.mark.timeout(900)
def test_fp8_summaries_full_gqa_32k(tis):
    w = workloads.get("gqa_32k")
    check_case(tis, w, label="gqa_32k (full size, fp8 summaries)", summary_dtype="fp8")


@pytest.mark.timeout(900)
def test_bf16_summaries_full_gqa_32k(tis):
    w = workloads.get("gqa_32k")
    check_case(tis, w, label="gqa_32k (full size, bf16 summaries)", summary_dtype="bf16")


FULL = ["alhr_1k", "gqa_32k", "gqa_256k", "deep_planted", "long_1m"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(tis, name):
    w = workloads.get(name)
    # full size: no mismatch may be excused
    x, ob, orr, g = check_case(tis, w, label=f"{name} (full size)", max_excused=0)
    if w.generator == "planted":
        hit = np.array([[x["planted"][bb, h] in g["idx"][bb, h] for h in range(w.q_heads)]
                        for bb in range(w.batch)])
        _say(f"{name}: planted blocks retrieved by {int(hit.sum())}/{hit.size} queries")
        assert hit.all()


def test_workspace_reuse_across_geometries(tis):
    """One cached workspace serves calls of different shapes in turn, and
    contents left by earlier calls never leak into later results: beyond the
    arrival counters (the first 16 KiB of a build workspace, 1 KiB of an
    attend or decode one, zero between calls) nothing in a workspace matters
    on entry, and every call leaves those counters zero whatever its shape."""
    cases = [
        _custom("ws_a", "bf16", 4, 16, 4, 16, Hkv=2, G=2, seed=21),   # few queries, wide beam
        _custom("ws_b", "bf16", 4, 16, 4, 8, Hkv=2, G=16, seed=22),   # many queries
        _custom("ws_c", "bf16", 2, 8, 8, 4, d=64, Hkv=1, G=4, seed=23),  # deep: build climbs
        _custom("ws_d", "bf16", 8, 8, 3, 16, Hkv=4, G=8, seed=24),
        _custom("ws_split", "bf16", 4, 64, 4, 64, Hkv=2, G=3, seed=26),  # 6 queries, split
        _custom("ws_a2", "bf16", 4, 16, 4, 16, Hkv=2, G=2, seed=25),
    ]
    counters = {"build": 16384, "attend": 1024, "decode": 1024}
    splits_seen = climbs_seen = 0
    for w in cases:
        for (_, kind), ws in tis.ops._workspaces.items():
            ws.fill_(0x7F)  # garbage (large finite doubles) must not matter
            ws[:counters.get(kind, 0)].zero_()
        lib = tis.ops.lib()
        splits_seen += lib.tis_decode_workspace_bytes(
            w.batch, w.q_heads, w.head_dim, w.beam, w.leaf_block) > 0
        climbs_seen += lib.tis_build_workspace_bytes(
            w.batch, w.kv_heads, w.n_keys, w.head_dim, w.branching, w.leaf_block, w.levels) > 0
        check_case(tis, w)
        torch.cuda.synchronize()
        for (_, kind), ws in tis.ops._workspaces.items():
            n = min(counters.get(kind, 0), ws.numel())
            assert not ws[:n].any(), f"{w.name}: {kind} counters left nonzero"
    assert splits_seen >= 1 and climbs_seen >= 1


GRAPH_CASES = [
    _custom("graph_split", "bf16", 4, 64, 4, 64, Hkv=2, G=3, seed=31),   # split, merged in the kernel
    _custom("graph_deep", "bf16", 2, 4, 9, 6, d=64, Hkv=3, G=1, seed=32),  # build climbs 4 levels
    workloads.small("deep_planted", levels=4, kv_heads=2),                # build climbs
    _custom("graph_per_level", "f32", 2, 1, 16, 3, d=64, Hkv=1, G=2, seed=33),  # per-level kernels
]


@pytest.mark.parametrize("w", GRAPH_CASES, ids=[w.name for w in GRAPH_CASES])
def test_graph_replay_matches_eager(tis, w):
    """A step (build, fused decode, route, attend) captured into a HIP graph
    reproduces the eager results bit for bit on every replay, with other
    eager work on the same buffers between the replays."""
    x = workloads.generate(w)
    dev = "cuda"
    Q = tis.from_storage(x["Q"], w.dtype, dev)
    K = tis.from_storage(x["K"], w.dtype, dev)
    V = tis.from_storage(x["V"], w.dtype, dev)
    plan = tis.DecodePlan(Q, K, V, w.branching, w.leaf_block, w.levels, w.beam)

    def step():
        plan.build()
        plan.decode()
        fused = plan.out.clone()
        plan.route()
        plan.attend()
        return fused

    fused_eager = step()
    torch.cuda.synchronize()
    ref = {"summ": plan.summaries.clone(), "idx": plan.indices.clone(),
           "out": plan.out.clone(), "fused": fused_eager}
    _say(f"{w.name}: eager step done")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        fused_g = step()
    for rep in range(3):
        # eager work that overwrites every output between the replays
        plan.summaries.fill_(float("nan"))
        plan.indices.fill_(-7)
        plan.out.fill_(float("nan"))
        fused_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.summaries.view(torch.int32), ref["summ"].view(torch.int32)), rep
        assert torch.equal(plan.indices, ref["idx"]), rep
        assert torch.equal(plan.out.view(torch.int32), ref["out"].view(torch.int32)), rep
        assert torch.equal(fused_g.view(torch.int32), ref["fused"].view(torch.int32)), rep
        _say(f"{w.name}: replay {rep} matches the eager step")
