"""Pins for the CPU oracle, independent of the oracle's own formulas.

Each test checks the oracle against something other than itself: closed forms,
invariants, exact rational brute force on tiny trees, and reductions to
textbook routines (dense softmax attention, single-level block top-k). The
definitions pinned are those of the ZHA abstract (Subquadratic Attention with a
Hierarchical Tree-Structured Indexer: summaries over the KV cache, top-down
traversal, final attention over the retrieved subset) under the readings that
the oracle's module docstring lists.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import tis_oracle as O
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _bf16(x):
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------------------
# build: closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_build_constant_keys(dtype):
    b, L, lv, d = 3, 5, 3, 8
    N = b ** lv * L
    c = 1.5
    Kf = np.full((2, 2, N, d), c, dtype=np.float32)
    K = Kf if dtype == "f32" else _bf16(Kf)
    t = O.tree_build(K, dtype, b, L, lv)
    for l in range(1, lv + 1):
        s = t["stored"][l - 1]
        assert s.shape == (2, 2, b ** l, d) and s.dtype == np.float32
        assert np.all(s == np.float32(c))


def test_build_block_constant_integers():
    """K[t, i] = floor(t / L) + i: node n of level l covers leaves
    [n*c, (n+1)*c) with c = b**(lv-l), so its mean is n*c + (c-1)/2 + i."""
    b, L, lv, d = 2, 4, 5, 6
    N = b ** lv * L
    t_idx = np.arange(N)[:, None]
    Kf = (t_idx // L + np.arange(d)[None, :]).astype(np.float32)
    K = Kf[None, None]
    t = O.tree_build(K, "f32", b, L, lv)
    for l in range(1, lv + 1):
        c = b ** (lv - l)
        n = np.arange(b ** l)[:, None]
        expect = n * c + (c - 1) / 2.0 + np.arange(d)[None, :]
        np.testing.assert_array_equal(t["mean"][l - 1][0, 0], expect)
        np.testing.assert_array_equal(t["stored"][l - 1][0, 0], expect.astype(np.float32))


def test_build_position_keys():
    """K[t, i] = t: node n of level l has mean n*M_l + (M_l - 1)/2."""
    b, L, lv, d = 4, 8, 4, 3
    N = b ** lv * L
    Kf = np.repeat(np.arange(N, dtype=np.float32)[:, None], d, axis=1)
    t = O.tree_build(Kf[None, None], "f32", b, L, lv)
    for l in range(1, lv + 1):
        M = N // b ** l
        expect = np.arange(b ** l) * M + (M - 1) / 2.0
        assert np.all(t["mean"][l - 1][0, 0] == expect[:, None])


def test_build_rounds_once():
    """Leaf {1, 2^-24, 2^-24, 0}: the exact mean 0.25 + 2^-25 is a float32, so
    the stored summary must hold it exactly; accumulating in float32 would
    lose the small terms (1 + 2^-24 rounds to 1) and give 0.25."""
    L, b, lv, d = 4, 2, 1, 1
    leaf = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 0.0], dtype=np.float32)
    Kf = np.concatenate([leaf, leaf[::-1]])[:, None]
    t = O.tree_build(Kf[None, None], "f32", b, L, lv)
    want = np.float32(0.25 + 2.0 ** -25)
    assert want != np.float32(0.25)
    assert np.all(t["stored"][0][0, 0, :, 0] == want)
    # and a mean that is not a float32 is rounded to nearest (even on ties)
    Kf2 = np.array([1.0, 2.0 ** -25, 0.0, 0.0, 0, 0, 0, 0], dtype=np.float32)[:, None]
    t2 = O.tree_build(Kf2[None, None], "f32", 2, 4, 1)
    # exact mean 0.25 + 2^-27 lies between 0.25 and 0.25+2^-25, nearer 0.25
    assert t2["stored"][0][0, 0, 0, 0] == np.float32(0.25)
    assert t2["mean"][0][0, 0, 0, 0] == 0.25 + 2.0 ** -27


def test_build_recursive_equals_direct():
    """The recursive mean of child means equals the direct mean of the keys."""
    w = workloads.small("gqa_32k", levels=2, kv_heads=2)
    x = workloads.generate(w)
    t = O.tree_build(x["K"], w.dtype, w.branching, w.leaf_block, w.levels)
    leaf = t["mean"][-1]
    cur = leaf
    for l in range(w.levels - 1, 0, -1):
        B, H, n, d = cur.shape
        cur = cur.reshape(B, H, n // w.branching, w.branching, d).mean(axis=3)
        np.testing.assert_allclose(cur, t["mean"][l - 1], rtol=1e-12, atol=1e-12)
    # and the leaf level against a plain per-block mean of the widened keys
    kf = workloads.bf16_bits_to_f32(x["K"]).astype(np.float64)
    B, H, N, d = kf.shape
    direct = kf.reshape(B, H, N // w.leaf_block, w.leaf_block, d).mean(axis=3)
    np.testing.assert_allclose(leaf, direct, rtol=1e-12, atol=1e-12)


def test_widen_bf16_exact():
    vals = np.array([1.0, -2.5, 3.140625, 1e-20, 65280.0], dtype=np.float32)
    bits = _bf16(vals)
    w = O.widen(bits, "bf16")
    # these values are exactly representable in bf16
    np.testing.assert_array_equal(w[[0, 1, 2, 4]], vals[[0, 1, 2, 4]].astype(np.float64))
    # 1e-20 rounds to the nearest bf16
    assert abs(w[3] - 1e-20) / 1e-20 < 2 ** -8


# ---------------------------------------------------------------------------
# route: exact rational brute force on tiny trees
# ---------------------------------------------------------------------------

def _exact_scores(Kint, q, b, L, lv):
    """Fraction score of every node of every level, straight from the raw keys:
    score(n) = (1/M) * sum over keys t under n of q . k_t."""
    N = Kint.shape[0]
    per_key = [sum(int(q[i]) * int(Kint[t, i]) for i in range(len(q))) for t in range(N)]
    out = []
    for l in range(1, lv + 1):
        M = N // b ** l
        out.append([Fraction(sum(per_key[n * M:(n + 1) * M]), M) for n in range(b ** l)])
    return out


def _beam_by_definition(scores, b, W):
    """Independent simulation: at each level sort the children of the kept
    nodes by (-score, index) with Python's sort and keep the first W."""
    kept = [None]
    trace = []
    for l, sc in enumerate(scores, start=1):
        cands = list(range(b)) if l == 1 else [p * b + c for p in kept for c in range(b)]
        cands.sort(key=lambda n: (-sc[n], n))
        kept = cands[:W]
        trace.append(sorted(kept))
    return trace


def _tiny_case(rng, b, L, lv, d, scale_to_integers):
    N = b ** lv * L
    K = rng.integers(-2, 3, size=(N, d))
    if scale_to_integers:
        K = K * (N // b)          # every node mean is then an integer
    q = rng.integers(-2, 3, size=d)
    return K, q


@pytest.mark.parametrize("b,L,lv,d,scaled", [
    (2, 1, 4, 3, False), (2, 2, 3, 4, False), (4, 2, 2, 3, False),
    (2, 4, 2, 2, False), (3, 1, 3, 3, True), (3, 2, 2, 4, True), (4, 3, 2, 2, True),
    (2, 3, 4, 2, True),
])
def test_route_brute_force_every_beam(b, L, lv, d, scaled):
    rng = np.random.default_rng([b, L, lv, d, int(scaled)])
    for rep in range(6):
        K, q = _tiny_case(rng, b, L, lv, d, scaled)
        sc = _exact_scores(K, q, b, L, lv)
        tree = O.tree_build(K.astype(np.float32)[None, None], "f32", b, L, lv)
        for W in range(1, b ** lv + 1):
            r = O.tree_route(q.astype(np.float32)[None, None], "f32", tree["stored"], b, W)
            want = _beam_by_definition(sc, b, W)
            for l in range(lv):
                got = [int(v) for v in r["trace"][0, 0, l] if v >= 0]
                assert got == want[l], (W, l)
            assert list(r["indices"][0, 0]) == want[-1]
            # closed-form candidate count: b + sum_{l>=2} min(W, b^(l-1)) * b
            assert r["scored"][0, 0] == b + sum(min(W, b ** (l - 1)) * b for l in range(2, lv + 1))


@pytest.mark.parametrize("b,L,lv,d", [(2, 2, 4, 3), (3, 2, 3, 3), (4, 1, 3, 4)])
def test_route_wide_beam_is_global_top_leaves(b, L, lv, d):
    """beam >= b^(lv-1) keeps every node above the leaves, so the result is the
    global top-W leaves by (score desc, index asc) -- via numpy's lexsort on
    leaf scores computed directly from the keys."""
    rng = np.random.default_rng([7, b, L, lv, d])
    for rep in range(5):
        K, q = _tiny_case(rng, b, L, lv, d, True)
        N = K.shape[0]
        leaf_scores = (K.astype(np.float64) @ q).reshape(-1, L).mean(axis=1)
        tree = O.tree_build(K.astype(np.float32)[None, None], "f32", b, L, lv)
        for W in range(b ** (lv - 1), b ** lv + 1):
            r = O.tree_route(q.astype(np.float32)[None, None], "f32", tree["stored"], b, W)
            order = np.lexsort((np.arange(b ** lv), -leaf_scores))
            assert list(r["indices"][0, 0]) == sorted(order[:W].tolist())


def test_route_beam1_is_greedy_chain():
    rng = np.random.default_rng(11)
    b, L, lv, d = 3, 2, 4, 5
    for rep in range(10):
        K, q = _tiny_case(rng, b, L, lv, d, True)
        sc = _exact_scores(K, q, b, L, lv)
        node = None
        for l in range(lv):
            kids = list(range(b)) if node is None else [node * b + c for c in range(b)]
            best = max(sc[l][n] for n in kids)
            node = min(n for n in kids if sc[l][n] == best)
        tree = O.tree_build(K.astype(np.float32)[None, None], "f32", b, L, lv)
        r = O.tree_route(q.astype(np.float32)[None, None], "f32", tree["stored"], b, 1)
        assert r["indices"][0, 0].tolist() == [node]


def test_route_ties_go_to_lowest_index():
    """Identical blocks everywhere: every score ties, so the kept set is the
    lowest indices; with two copies of a winning block the lower copy wins."""
    b, L, lv, d = 2, 2, 3, 4
    N = b ** lv * L
    K = np.ones((N, d), dtype=np.float32)
    q = np.ones(d, dtype=np.float32)
    tree = O.tree_build(K[None, None], "f32", b, L, lv)
    for W in (1, 2, 3, 5):
        r = O.tree_route(q[None, None], "f32", tree["stored"], b, W)
        # level by level the lowest-indexed children win: leaves 0..W-1
        assert r["indices"][0, 0].tolist() == list(range(W))
    # duplicate a strong block at leaves 5 and 6 (same level-1 parent, node 1,
    # and different level-2 parents 2 and 3); beam 1 must reach leaf 5
    K2 = np.zeros((N, d), dtype=np.float32)
    K2[5 * L:6 * L] = 3.0
    K2[6 * L:7 * L] = 3.0
    tree2 = O.tree_build(K2[None, None], "f32", b, L, lv)
    r = O.tree_route(q[None, None], "f32", tree2["stored"], b, 1)
    assert r["indices"][0, 0].tolist() == [5]


def test_route_gqa_and_batch_mapping():
    """Each (batch, KV head) gets its own strong leaf; with beam 1 every query
    head h must reach the leaf of KV head h // (Hq/Hkv) in its own batch row."""
    B, Hkv, G, b, L, lv, d = 2, 3, 2, 2, 2, 3, 4
    N = b ** lv * L
    K = np.zeros((B, Hkv, N, d), dtype=np.float32)
    strong = np.array([[1, 6, 3], [4, 2, 7]])
    for bi in range(B):
        for h in range(Hkv):
            K[bi, h, strong[bi, h] * L:(strong[bi, h] + 1) * L] = 5.0
    Q = np.ones((B, Hkv * G, d), dtype=np.float32)
    tree = O.tree_build(K, "f32", b, L, lv)
    r = O.tree_route(Q, "f32", tree["stored"], b, 1)
    for bi in range(B):
        for hq in range(Hkv * G):
            assert r["indices"][bi, hq].tolist() == [strong[bi, hq // G]]


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(b=st.integers(2, 4), L=st.integers(1, 3), lv=st.integers(1, 3),
       d=st.integers(1, 4), W=st.integers(1, 64), seed=st.integers(0, 2 ** 31))
def test_route_topw_definition_property(b, L, lv, d, W, seed):
    """At every level the kept set is exactly the W best children of the
    previous kept set: no dropped candidate beats a kept one under
    (score desc, index asc), scored exactly from raw keys."""
    W = min(W, b ** lv)
    rng = np.random.default_rng(seed)
    K, q = _tiny_case(rng, b, L, lv, d, True)
    sc = _exact_scores(K, q, b, L, lv)
    tree = O.tree_build(K.astype(np.float32)[None, None], "f32", b, L, lv)
    r = O.tree_route(q.astype(np.float32)[None, None], "f32", tree["stored"], b, W)
    prev = None
    for l in range(lv):
        kept = [int(v) for v in r["trace"][0, 0, l] if v >= 0]
        cands = list(range(b)) if prev is None else [p * b + c for p in prev for c in range(b)]
        assert set(kept) <= set(cands)
        assert len(kept) == min(W, len(cands))
        dropped = set(cands) - set(kept)
        for k in kept:
            for c in dropped:
                assert (sc[l][k], -k) > (sc[l][c], -c)
        prev = kept


# ---------------------------------------------------------------------------
# route + attend: textbook reductions
# ---------------------------------------------------------------------------

def _dense_softmax_attention(q, K, V, scale):
    s = scale * (K @ q)
    return scipy.special.softmax(s) @ V


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_full_beam_is_dense_attention(dtype):
    """beam = all leaves selects every leaf, and the final attention is plain
    dense softmax attention (scipy softmax + matmul)."""
    rng = np.random.default_rng(5)
    b, L, lv, d, Hkv, G = 2, 4, 3, 16, 2, 3
    N = b ** lv * L
    Kf = rng.standard_normal((1, Hkv, N, d)).astype(np.float32)
    Vf = rng.standard_normal((1, Hkv, N, d)).astype(np.float32)
    Qf = rng.standard_normal((1, Hkv * G, d)).astype(np.float32)
    conv = (lambda a: a) if dtype == "f32" else _bf16
    K, V, Q = conv(Kf), conv(Vf), conv(Qf)
    res = O.decode(Q, K, V, dtype, b, L, lv, b ** lv)
    assert np.all(res["route"]["indices"] == np.arange(b ** lv))
    k64, v64, q64 = (O.widen(a, dtype) for a in (K, V, Q))
    for hq in range(Hkv * G):
        want = _dense_softmax_attention(q64[0, hq], k64[0, hq // G], v64[0, hq // G],
                                        1 / math.sqrt(d))
        np.testing.assert_allclose(res["out"][0, hq], want, rtol=1e-12, atol=1e-13)


def test_single_level_is_block_topk():
    """levels = 1: the route is block top-k on block-mean scores followed by
    softmax on the selected tokens (the NSA / InfLLMv2 description)."""
    rng = np.random.default_rng(9)
    b, L, d, W = 16, 8, 8, 5
    N = b * L
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    res = O.decode(q[None, None], K[None, None], V[None, None], "f32", b, L, 1, W)
    block_scores = K.astype(np.float64).reshape(b, L, d).mean(axis=1) @ q.astype(np.float64)
    top = np.argpartition(-block_scores, W - 1)[:W]
    assert sorted(top.tolist()) == res["route"]["indices"][0, 0].tolist()
    rows = np.concatenate([np.arange(j * L, (j + 1) * L) for j in sorted(top)])
    want = _dense_softmax_attention(q.astype(np.float64), K[rows].astype(np.float64),
                                    V[rows].astype(np.float64), 1 / math.sqrt(d))
    np.testing.assert_allclose(res["out"][0, 0], want, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# attend: invariants and edge cases
# ---------------------------------------------------------------------------

def _rand_attend_case(seed, dtype="f32"):
    rng = np.random.default_rng(seed)
    B, Hkv, G, N, d, L = 2, 2, 2, 64, 8, 4
    K = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    Q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    idx = np.stack([np.stack([rng.choice(N // L, 5, replace=False) for _ in range(Hkv * G)])
                    for _ in range(B)]).astype(np.int32)
    return K, V, Q, idx, L


def test_attend_constant_values():
    K, V, Q, idx, L = _rand_attend_case(1)
    V[:] = 0.75
    o = O.tree_attend(Q, K, V, "f32", idx, L)
    np.testing.assert_allclose(o, 0.75, rtol=0, atol=1e-15)


def test_attend_zero_keys_is_mean_of_selected_values():
    K, V, Q, idx, L = _rand_attend_case(2)
    K[:] = 0
    o = O.tree_attend(Q, K, V, "f32", idx, L)
    for bi in range(Q.shape[0]):
        for hq in range(Q.shape[1]):
            hk = hq // 2
            rows = np.concatenate([np.arange(j * L, (j + 1) * L) for j in idx[bi, hq]])
            np.testing.assert_allclose(o[bi, hq], V[bi, hk, rows].astype(np.float64).mean(0),
                                       rtol=1e-13, atol=1e-14)


def test_attend_convex_hull_and_permutation():
    K, V, Q, idx, L = _rand_attend_case(3)
    o = O.tree_attend(Q, K, V, "f32", idx, L)
    perm = idx[..., ::-1].copy()
    o2 = O.tree_attend(Q, K, V, "f32", perm, L)
    np.testing.assert_allclose(o, o2, rtol=1e-14, atol=1e-15)
    for bi in range(Q.shape[0]):
        for hq in range(Q.shape[1]):
            rows = np.concatenate([np.arange(j * L, (j + 1) * L) for j in idx[bi, hq]])
            v = V[bi, hq // 2, rows]
            assert np.all(o[bi, hq] >= v.min(0) - 1e-12)
            assert np.all(o[bi, hq] <= v.max(0) + 1e-12)


def test_attend_padding_duplicates_empty_and_range():
    K, V, Q, idx, L = _rand_attend_case(4)
    o = O.tree_attend(Q, K, V, "f32", idx, L)
    padded = np.concatenate([idx, -np.ones_like(idx[..., :2]), idx[..., :1]], axis=-1)
    np.testing.assert_allclose(O.tree_attend(Q, K, V, "f32", padded, L), o, rtol=1e-14, atol=1e-15)
    empty = -np.ones_like(idx)
    assert np.all(O.tree_attend(Q, K, V, "f32", empty, L) == 0)
    bad = idx.copy()
    bad[0, 0, 0] = K.shape[2] // L
    with pytest.raises(ValueError):
        O.tree_attend(Q, K, V, "f32", bad, L)


def test_attend_softmax_shift_invariance():
    """Adding one vector u to every key adds scale*q.u to every score, which
    softmax ignores. Keys are multiples of 2^-10 so that k + u is exact in
    float32."""
    K, V, Q, idx, L = _rand_attend_case(6)
    K = (np.round(K * 1024) / 1024).astype(np.float32)
    o = O.tree_attend(Q, K, V, "f32", idx, L)
    u = np.array([2.0, -1.0, 0.5, 3.0, 0.0, -4.0, 1.0, 2.0], dtype=np.float32)
    o2 = O.tree_attend(Q, K + u, V, "f32", idx, L)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# counts on the page-shaped workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,scored", [("alhr_1k", 22), ("gqa_32k", 136), ("gqa_256k", 328),
                                         ("long_1m", 456), ("deep_planted", 148)])
def test_candidate_count_closed_form(name, scored):
    w = workloads.get(name)
    b, W = w.branching, w.beam
    assert b + sum(min(W, b ** (l - 1)) * b for l in range(2, w.levels + 1)) == scored
    assert w.n_keys == b ** w.levels * w.leaf_block


def test_alhr_workload_reads_32_keys_per_query():
    """The 1,024-token binary-tree workload (64 leaves of 16, 6 levels, beam 2)
    reads exactly beam x leaf_block = 32 keys per query, scores 22 summaries,
    and every kept leaf descends from kept nodes at every level."""
    w = workloads.get("alhr_1k")
    x = workloads.generate(w)
    res = O.decode(x["Q"], x["K"], x["V"], w.dtype, w.branching, w.leaf_block, w.levels, w.beam)
    idx = res["route"]["indices"]
    tr = res["route"]["trace"]
    assert idx.shape == (1, 64, 2)
    assert np.all(res["route"]["scored"] == 22)
    for hq in range(64):
        sel = idx[0, hq]
        assert len(set(sel.tolist())) == 2 and np.all((sel >= 0) & (sel < 64))
        assert len(sel) * w.leaf_block == 32
        for l in range(1, w.levels + 1):
            anc = set((sel // w.branching ** (w.levels - l)).tolist())
            assert anc <= set(int(v) for v in tr[0, hq, l - 1] if v >= 0)
