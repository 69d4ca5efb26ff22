"""Parity of the growing-cache tree (tis_cache_tree_* through the C-ABI) with
the CPU oracle for a tree over the first n keys of a cache.

A cache is filled by a sequence of appends that crosses leaf, node and depth
boundaries; after each append the GPU tree, kept incrementally, must equal
the oracle's tree of the same n keys (summaries within 1 ulp, reported
bit-equal counts), route the same leaves (cut gaps under 1e-5 counted), and
its fused decode must attend within the input type's tolerance.  At a full
size the cache tree must agree bit for bit with the full-tree calls.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import workloads
from oracle import tis_grow_oracle as GO
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[cache]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()
    return t


def _inputs(dtype, b, L, d, Hkv, G, capacity, gen="normal", seed=7, name="cache"):
    """Seeded cache of `capacity` keys per head: the first `capacity` rows of a
    full-tree workload deep enough to hold them."""
    lv = GO.depth_for(capacity, b, L)
    # mixture: 128 keys per cluster, as in the 32K-key GQA workload
    clusters = b ** lv * L // 128 if gen == "mixture" else 0
    w = workloads.Workload(name, dtype, 1, Hkv * G, Hkv, d, b, L, lv, 1, gen,
                           clusters=clusters, seed=seed)
    x = workloads.generate(w)
    return {k: np.ascontiguousarray(x[k][:, :, :capacity]) if k in ("K", "V") else x[k]
            for k in ("K", "V", "Q")}


def _check(tis, ct, x, Qd, dtype, n, b, L, beam, label):
    sd = ct.summary_dtype
    ob = GO.grow_build(x["K"], dtype, n, b, L, summary_dtype=sd)
    lv = ob["levels"]
    assert ct.levels == lv and ct.n_keys == n
    g_levels = [ct.level(l).float().cpu().numpy() for l in range(1, lv + 1)]
    eq, tot, worst = parity.compare_summaries(g_levels, ob["stored"], summary_dtype=sd)
    orr = GO.grow_route(x["Q"], dtype, ob["stored"], n, b, L, beam)
    idx, tr = ct.route(Qd, beam, trace=True)
    out, didx = ct.decode(Qd, beam, return_indices=True)
    torch.cuda.synchronize()
    idx, tr, out, didx = idx.cpu().numpy(), tr.cpu().numpy(), out.cpu().numpy(), didx.cpu().numpy()
    w_out = orr["indices"].shape[-1]
    assert np.all(idx[..., w_out:] == -1), "padding past the kept leaves"
    exact, tie, nq = parity.compare_indices(idx[..., :w_out], orr)
    parity.compare_trace(tr, orr)
    assert np.array_equal(didx, idx), "fused decode kept other leaves"
    o_g = GO.grow_attend(x["Q"], x["K"], x["V"], dtype, idx, n, L)
    err = parity.compare_outputs(out, o_g, dtype)
    gaps = orr["gap"][np.isfinite(orr["gap"])]
    _say(f"{label} n={n} lv={lv}: summaries bit-equal {eq}/{tot} (worst {worst} ulp); "
         f"indices exact {exact}/{nq}, tie-exposed {tie}; decode max-abs {err:.2e}; "
         f"min cut gap {float(gaps.min()) if gaps.size else float('inf'):.2e}")
    return eq, tot


SEQUENCES = [
    # (label, dtype, b, L, d, Hkv, G, capacity, beam, first appends[, summary type])
    ("tiny_f32", "f32", 3, 5, 64, 2, 2, 405, 4, [1, 1, 3, 1, 4, 5, 9, 1, 20, 1, 44, 1, 90]),
    ("bf16_d128", "bf16", 4, 16, 128, 2, 3, 1000, 6, [1, 15, 1, 47, 1, 191, 1, 100, 300]),
    ("beam_wide", "bf16", 2, 8, 64, 1, 4, 300, 16, [1, 2, 5, 8, 16, 1, 31, 64, 1, 127]),
    ("leaf_1", "f32", 2, 1, 64, 1, 2, 100, 3, [1, 1, 1, 1, 4, 8, 16, 1, 31, 1]),
    ("branch_8_f32", "f32", 8, 4, 128, 2, 2, 600, 5, [7, 1, 24, 1, 224, 1, 255, 2]),
    # bfloat16 summaries, both head dims
    ("bf16s_d128", "bf16", 4, 16, 128, 2, 3, 1000, 6, [1, 15, 1, 47, 1, 191, 1, 100, 300],
     "bf16"),
    ("bf16s_f32_d64", "f32", 3, 5, 64, 2, 2, 405, 4, [1, 1, 3, 1, 4, 5, 9, 1, 20, 1, 44, 1, 90],
     "bf16"),
]


@pytest.mark.parametrize("case", SEQUENCES, ids=[c[0] for c in SEQUENCES])
def test_append_sequence_matches_oracle(tis, case):
    label, dtype, b, L, d, Hkv, G, cap, beam, chunks = case[:10]
    sd = case[10] if len(case) > 10 else "f32"
    t0 = time.time()
    x = _inputs(dtype, b, L, d, Hkv, G, cap, seed=len(label))
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L, summary_dtype=sd)
    n = 0
    rest = cap - sum(chunks)
    assert rest >= 0
    for c in chunks + ([rest] if rest else []):
        ct.append(c)
        n += c
        _check(tis, ct, x, Qd, dtype, n, b, L, beam, label)
    assert n == cap
    _say(f"{label}: {len(chunks) + (1 if rest else 0)} appends checked in {time.time() - t0:.1f}s")


LONG = [
    # (label, dtype, summary type, b, L, d, Hkv, G, capacity, beam, appends)
    # long appends run in chunks (the nodes of the smallest height with 512
    # or more keys, at most 64 leaves), then heights above them per head;
    # appends start mid-leaf and mid-node, and short ones come in between
    ("b4_bf16", "bf16", "f32", 4, 16, 128, 2, 2, 16000, 6, [5, 3000, 1, 1500, 7, 11000]),
    ("b8_f32_d64", "f32", "f32", 8, 32, 64, 2, 2, 20000, 5, [100, 5000, 3, 9000]),
    ("b2_bf16s", "bf16", "bf16", 2, 16, 128, 1, 3, 5000, 4, [1, 700, 2049, 1]),
    ("leaf_1", "f32", "f32", 2, 1, 64, 1, 2, 3000, 3, [10, 1000, 1, 1500]),
    # chunks are the top height: no heights above them
    ("top_chunks", "bf16", "f32", 3, 5, 64, 2, 2, 405, 4, [7, 200, 1]),
    # appends that start and end on chunk boundaries (512 keys here), the
    # last one up to a full cache
    ("aligned", "bf16", "f32", 8, 64, 128, 1, 4, 8 ** 3 * 64, 8, [512, 1024, 1536]),
]


@pytest.mark.parametrize("case", LONG, ids=[c[0] for c in LONG])
def test_long_appends_match_oracle(tis, case):
    label, dtype, sd, b, L, d, Hkv, G, cap, beam, chunks = case
    t0 = time.time()
    x = _inputs(dtype, b, L, d, Hkv, G, cap, seed=len(label) + 11)
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L, summary_dtype=sd)
    n = 0
    halves = set()
    for c in chunks + [cap - sum(chunks)]:
        ct.append(c)
        n += c
        halves.add(ct.c.state_half)
        _check(tis, ct, x, Qd, dtype, n, b, L, beam, label)
    # the tree goes on growing from the state the long appends left
    ct.reset()
    ct.append(cap - 3)
    for _ in range(3):
        ct.append_decode(Qd, beam)
    _check(tis, ct, x, Qd, dtype, cap, b, L, beam, label + " refill")
    _say(f"{label}: long appends checked (state halves used {sorted(halves)}) in "
         f"{time.time() - t0:.1f}s")


def test_reset_then_refill_matches(tis):
    """A reset empties the tree whatever it held; refilling gives the same tree."""
    dtype, b, L, d, cap, beam = "bf16", 3, 4, 64, 200, 3
    x = _inputs(dtype, b, L, d, 2, 2, cap, seed=41)
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L)
    ct.append(150)
    ct.reset()
    assert (ct.n_keys, ct.levels) == (0, 0)
    ct.state.fill_(0)  # (already zero) the refill must not depend on old summaries
    ct.summaries.fill_(float("nan"))
    for c in (37, 1, 62):
        ct.append(c)
    _check(tis, ct, x, Qd, dtype, 100, b, L, beam, "refill")


@pytest.mark.parametrize("sd", ["f32", "bf16"])
def test_full_cache_equals_full_tree_calls(tis, sd):
    """With n = b^lv * L the cache tree is the full tree: the same summaries
    and the same decode output, bit for bit, as tree_build + tree_decode."""
    w = workloads.small("gqa_32k", levels=2, kv_heads=2)
    x = workloads.generate(w)
    dtype, b, L = w.dtype, w.branching, w.leaf_block
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L, summary_dtype=sd)
    ct.append(w.n_keys - 129)
    for _ in range(129):
        ct.append(1)
    tree = tis.tree_build(Kd, b, L, w.levels, summary_dtype=sd)
    out_c, idx_c = ct.decode(Qd, w.beam, return_indices=True)
    out_f, idx_f = tis.tree_decode(Qd, Kd, Vd, tree, w.beam, return_indices=True)
    torch.cuda.synchronize()
    for l in range(1, w.levels + 1):
        a = ct.level(l).float().cpu().numpy()
        f = tree.level(l).float().cpu().numpy()
        assert np.array_equal(a.view(np.uint32), f.view(np.uint32)), l
    assert torch.equal(idx_c, idx_f)
    assert torch.equal(out_c.view(torch.int32), out_f.view(torch.int32))
    _check(tis, ct, x, Qd, dtype, w.n_keys, b, L, w.beam, "full")


def test_decode_loop_on_a_gqa_cache(tis):
    """The decode-loop shape: a clustered GQA cache prefilled in one append,
    then one key per step; checked every few steps, across a leaf boundary."""
    b, L, d, Hkv, G, beam = 8, 64, 128, 2, 4, 8
    cap = 8 ** 3 * 64
    x = _inputs("bf16", b, L, d, Hkv, G, cap, gen="mixture", seed=3)
    Kd = tis.from_storage(x["K"], "bf16", "cuda")
    Vd = tis.from_storage(x["V"], "bf16", "cuda")
    Qd = tis.from_storage(x["Q"], "bf16", "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L)
    n = cap - 100
    ct.append(n)
    _check(tis, ct, x, Qd, "bf16", n, b, L, beam, "gqa prefill")
    for step in range(1, 41):
        ct.append(1)
        n += 1
        if step % 8 == 0 or n % L == 0:
            _check(tis, ct, x, Qd, "bf16", n, b, L, beam, f"gqa step {step}")


def test_split_decode_few_queries_long_gathers(tis):
    """Few queries with long gathers split each query over workgroups; the
    kept count may be below the beam early on (empty parts)."""
    dtype, b, L, d, Hkv, G, beam = "bf16", 4, 64, 128, 2, 1, 64
    cap = 4 ** 4 * 64
    x = _inputs(dtype, b, L, d, Hkv, G, cap, seed=51)
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L)
    n = 0
    for c in (700, 1, 2000, 3000, 1, 5000):
        ct.append(c)
        n += c
        _check(tis, ct, x, Qd, dtype, n, b, L, beam, "split")
