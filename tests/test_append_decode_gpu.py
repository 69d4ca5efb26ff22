"""Parity of the fused one-key append + decode of a growing cache
(tis_cache_tree_append_decode through the C-ABI).

Each step adds key n to the tree and decodes over the tree of n + 1 keys.
Checked at every step against the CPU oracle's tree of n + 1 keys (kept
leaves exact, cut gaps under 1e-5 counted; output within the input type's
tolerance of the oracle's attention over the GPU's leaves), and against a
second cache driven by the separate calls (append of one key, then decode):
the same leaves and, where the leaves agree, the same output bit for bit;
at the end, the same summaries for every node ever written and the same
open-node sums, bit for bit.
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
    print("[append_decode]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()
    return t


def _inputs(dtype, b, L, d, Hkv, G, capacity, gen="normal", seed=7, B=1):
    lv = GO.depth_for(capacity, b, L)
    clusters = b ** lv * L // 128 if gen == "mixture" else 0
    w = workloads.Workload("append_decode", dtype, B, Hkv * G, Hkv, d, b, L, lv, 1, gen,
                           clusters=clusters, seed=seed)
    x = workloads.generate(w)
    return {k: np.ascontiguousarray(x[k][:, :, :capacity]) if k in ("K", "V") else x[k]
            for k in ("K", "V", "Q")}


def _heights(ct):
    """Stored heights of a cache tree and the keys under one node of each."""
    c = ct.c
    H = 1  # the depth of a full cache: fewest H with L b^H >= capacity
    while c.leaf_block * c.branching ** H < c.capacity:
        H += 1
    return [c.leaf_block * c.branching ** h for h in range(H)]


def _same_tree(ct, ref):
    """Every written summary row (the nodes over the first n keys at every
    stored height) and the open-node sums in use agree bit for bit."""
    n = ct.n_keys
    assert n == ref.n_keys and ct.levels == ref.levels
    for h, span in enumerate(_heights(ct)):
        rows = -(-n // span)
        a = ct.height_block(h)[:, :, :rows].contiguous().view(torch.int16 if
                                                               ct.summary_dtype == "bf16"
                                                               else torch.int32)
        r = ref.height_block(h)[:, :, :rows].contiguous().view(a.dtype)
        assert torch.equal(a, r), f"height {h} summaries differ"
    c = ct.c
    half = c.batch * c.kv_heads * len(_heights(ct)) * c.head_dim  # doubles in one state half
    s_f = ct.state[c.state_half * half:][:half]
    s_r = ref.state[ref.c.state_half * half:][:half]
    assert torch.equal(s_f.view(torch.int64), s_r.view(torch.int64)), "open-node sums differ"


def _step_check(x, dtype, n, b, L, beam, idx, out, sd):
    """Oracle check of one step over the tree of n keys; returns (exact, tie,
    queries, max-abs)."""
    ob = GO.grow_build(x["K"], dtype, n, b, L, summary_dtype=sd)
    orr = GO.grow_route(x["Q"], dtype, ob["stored"], n, b, L, beam)
    w_out = orr["indices"].shape[-1]
    assert np.all(idx[..., w_out:] == -1), "padding past the kept leaves"
    exact, tie, nq = parity.compare_indices(idx[..., :w_out], orr)
    o_g = GO.grow_attend(x["Q"], x["K"], x["V"], dtype, idx, n, L)
    err = parity.compare_outputs(out, o_g, dtype)
    return exact, tie, nq, err


STEPS = [
    # (label, dtype, summary type, b, L, d, Hkv, G, capacity, beam, keys before, steps)
    # from an empty cache: the first key, leaf and node closings, depth growth
    # at 15, 45 and 135 keys
    ("empty_start_f32", "f32", "f32", 3, 5, 64, 2, 2, 405, 4, 0, 140),
    # bf16 keys, d 128, across 256 keys (depth 2 -> 3) and a level-1 closing
    ("bf16_d128_depth", "bf16", "f32", 4, 16, 128, 2, 3, 1000, 6, 240, 40),
    # bfloat16 summaries
    ("bf16s_d128", "bf16", "bf16", 4, 16, 128, 2, 3, 1000, 6, 240, 40),
    ("bf16s_f32_d64", "f32", "bf16", 3, 5, 64, 2, 2, 405, 4, 0, 60),
    # one-key leaves: every step closes a leaf, depth grows at each power of 2
    ("leaf_1", "f32", "f32", 2, 1, 64, 1, 2, 300, 3, 0, 140),
    # many children, wide beam (no cut until the last levels)
    ("branch_8_wide", "bf16", "f32", 8, 4, 128, 2, 2, 600, 20, 20, 70),
    # few queries with long gathers: each query split over workgroups
    ("split", "bf16", "f32", 4, 64, 128, 2, 1, 4 ** 4 * 64, 64, 4000, 70),
]


@pytest.mark.parametrize("case", STEPS, ids=[c[0] for c in STEPS])
def test_append_decode_steps(tis, case):
    label, dtype, sd, b, L, d, Hkv, G, cap, beam, n0, steps = case
    t0 = time.time()
    x = _inputs(dtype, b, L, d, Hkv, G, cap, seed=len(label) + 3)
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L, summary_dtype=sd)
    ref = tis.CacheTree(Kd, Vd, b, L, summary_dtype=sd)
    if n0:
        ct.append(n0)
        ref.append(n0)
    tot = dict(exact=0, tie=0, nq=0, err=0.0, same=0)
    half0 = ct.c.state_half  # a long prefix append may have switched halves already
    for s in range(steps):
        n = ct.n_keys + 1
        out_f, idx_f = ct.append_decode(Qd, beam, return_indices=True)
        ref.append(1)
        out_r, idx_r = ref.decode(Qd, beam, return_indices=True)
        torch.cuda.synchronize()
        assert ct.n_keys == n and ct.c.state_half == (half0 + s + 1) % 2
        idx_f, idx_r = idx_f.cpu().numpy(), idx_r.cpu().numpy()
        out_f, out_r = out_f.cpu().numpy(), out_r.cpu().numpy()
        exact, tie, nq, err = _step_check(x, dtype, n, b, L, beam, idx_f, out_f, sd)
        tot["exact"] += exact
        tot["tie"] += tie
        tot["nq"] += nq
        tot["err"] = max(tot["err"], err)
        same = np.all(idx_f == idx_r, axis=-1)
        tot["same"] += int(same.sum())
        # where both kept the same leaves, the attention is the same code on
        # the same inputs
        assert np.array_equal(out_f[same].view(np.uint32), out_r[same].view(np.uint32))
    _same_tree(ct, ref)
    _say(f"{label}: {steps} steps from {n0} keys to {ct.n_keys} (depth {ct.levels}); indices "
         f"exact {tot['exact']}/{tot['nq']}, tie-exposed {tot['tie']}; same leaves as the "
         f"separate calls {tot['same']}/{tot['nq']}; max-abs {tot['err']:.2e}; "
         f"{time.time() - t0:.1f}s")


def test_append_decode_mixed_with_appends_and_reset(tis):
    """The fused step switches state halves; multi-key appends update the half
    in use in place; a reset returns to half 0.  Any mix gives the tree the
    separate calls give."""
    dtype, b, L, d, cap, beam = "bf16", 3, 4, 64, 400, 3
    x = _inputs(dtype, b, L, d, 2, 2, cap, seed=29)
    Kd = tis.from_storage(x["K"], dtype, "cuda")
    Vd = tis.from_storage(x["V"], dtype, "cuda")
    Qd = tis.from_storage(x["Q"], dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L)
    ref = tis.CacheTree(Kd, Vd, b, L)
    plan = [("f", 3), ("a", 7), ("f", 2), ("a", 20), ("f", 1), ("a", 1), ("f", 13), ("reset", 0),
            ("f", 5), ("a", 100), ("f", 9), ("a", 36), ("f", 4)]
    checked = 0
    for op, k in plan:
        if op == "reset":
            ct.reset()
            ref.reset()
            assert ct.c.state_half == 0
            continue
        if op == "a":
            ct.append(k)
            ref.append(k)
            continue
        for _ in range(k):
            out_f, idx_f = ct.append_decode(Qd, beam, return_indices=True)
            ref.append(1)
            out_r, idx_r = ref.decode(Qd, beam, return_indices=True)
            torch.cuda.synchronize()
            n = ct.n_keys
            exact, tie, nq, err = _step_check(x, dtype, n, b, L, beam, idx_f.cpu().numpy(),
                                              out_f.cpu().numpy(), "f32")
            assert exact + tie == nq
            checked += 1
        _same_tree(ct, ref)
    _say(f"mixed plan: {checked} fused steps checked, trees equal after each run of steps, "
         f"n = {ct.n_keys}")


def test_append_decode_gqa_loop(tis):
    """The decode-loop shape of the 32K-key GQA workload (b 8, L 64, d 128,
    group 4, beam 8, clustered keys): a prefill append, then one fused step
    per token across leaf boundaries; the oracle every 10 steps and at each
    leaf closing, the separate calls at every step."""
    b, L, d, Hkv, G, beam = 8, 64, 128, 2, 4, 8
    cap = 8 ** 3 * 64
    x = _inputs("bf16", b, L, d, Hkv, G, cap, gen="mixture", seed=3)
    Kd = tis.from_storage(x["K"], "bf16", "cuda")
    Vd = tis.from_storage(x["V"], "bf16", "cuda")
    Qd = tis.from_storage(x["Q"], "bf16", "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L)
    ref = tis.CacheTree(Kd, Vd, b, L)
    ct.append(cap - 130)
    ref.append(cap - 130)
    out = torch.empty((1, Hkv * G, d), dtype=torch.float32, device="cuda")
    step = ct.bind_decode(Qd, beam, out, append=True)
    oracle_checks = 0
    for s in range(130):
        step()
        ref.append(1)
        out_r, idx_r = ref.decode(Qd, beam, return_indices=True)
        torch.cuda.synchronize()
        n = ct.n_keys
        assert n == cap - 129 + s
        if s % 10 == 0 or n % L == 0 or n == cap:
            exact, tie, nq, err = _step_check(x, "bf16", n, b, L, beam, idx_r.cpu().numpy(),
                                              out.cpu().numpy(), "f32")
            assert exact + tie == nq
            oracle_checks += 1
        assert torch.equal(out.view(torch.int32), out_r.view(torch.int32)), f"step {s}"
    _same_tree(ct, ref)
    with pytest.raises(tis.TisError):
        step()  # the cache is full
    _say(f"gqa loop: 130 bound fused steps to a full cache, bit-equal to the separate calls at "
         f"every step, {oracle_checks} oracle checks")
