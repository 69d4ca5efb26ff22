"""Pins for the growing-cache oracle (oracle/tis_grow_oracle.py).

Each test checks it against something other than its own formulas: the
already pinned full-tree oracle at full sizes, a bottom-up brute-force tree
built from explicit key lists with exact rationals, an independent beam
simulation over that tree, numpy's lexsort on leaf scores, dense softmax
attention, and closed forms.  The definitions are the readings listed in
the module's docstring (depth grows when the cache outgrows the tree; nodes
cover their key range cut at the cache length).
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import tis_oracle as O
from oracle import tis_grow_oracle as GO
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ---------------------------------------------------------------------------
# depth
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b,L", [(2, 1), (2, 16), (3, 5), (8, 64), (4, 64)])
def test_depth_grows_exactly_past_each_full_tree(b, L):
    assert GO.depth_for(1, b, L) == 1
    for lv in range(1, 7):
        full = b ** lv * L
        assert GO.depth_for(full, b, L) == lv
        assert GO.depth_for(full + 1, b, L) == lv + 1
        if full > 1:
            below = lv if full - 1 > b ** (lv - 1) * L else max(lv - 1, 1)
            assert GO.depth_for(full - 1, b, L) == below


# ---------------------------------------------------------------------------
# full sizes: the same results as the full-tree oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b,L,lv,W", [(2, 4, 3, 3), (3, 2, 3, 4), (4, 5, 2, 6), (8, 8, 2, 8)])
def test_full_size_matches_full_tree_oracle(dtype, b, L, lv, W):
    rng = np.random.default_rng([b, L, lv, W])
    N, d, Hkv, G = b ** lv * L, 8, 2, 3
    Kf = rng.standard_normal((1, Hkv, N, d)).astype(np.float32)
    Vf = rng.standard_normal((1, Hkv, N, d)).astype(np.float32)
    Qf = rng.standard_normal((1, Hkv * G, d)).astype(np.float32)
    conv = (lambda a: a) if dtype == "f32" else workloads.f32_to_bf16_bits
    K, V, Q = conv(Kf), conv(Vf), conv(Qf)
    t = O.tree_build(K, dtype, b, L, lv)
    g = GO.grow_build(K, dtype, N, b, L)
    assert g["levels"] == lv
    for l in range(lv):
        assert np.array_equal(g["stored"][l].view(np.uint32), t["stored"][l].view(np.uint32))
    r = O.tree_route(Q, dtype, t["stored"], b, W)
    rg = GO.grow_route(Q, dtype, g["stored"], N, b, L, W)
    for k in ("indices", "trace", "gap", "scored"):
        assert np.array_equal(rg[k], r[k]), k
    a = O.tree_attend(Q, K, V, dtype, r["indices"], L)
    ag = GO.grow_attend(Q, K, V, dtype, rg["indices"], N, L)
    assert np.array_equal(a, ag)


# ---------------------------------------------------------------------------
# build: bottom-up brute force with exact rationals
# ---------------------------------------------------------------------------

def _brute_tree(Kint, n_keys, b, L):
    """Bottom-up: leaves are the blocks of L consecutive keys (the last one
    short), each level above groups b consecutive nodes of the level below
    (the last group short), until one group would hold everything.  Returns
    the per-level lists of key-index lists, root level first."""
    leaves = [list(range(j, min(j + L, n_keys))) for j in range(0, n_keys, L)]
    levels = [leaves]
    while True:
        below = levels[0]
        if len(below) <= b:
            break
        levels.insert(0, [sum(below[i:i + b], []) for i in range(0, len(below), b)])
    return levels


def _exact_means(Kint, keys):
    d = Kint.shape[1]
    return [Fraction(int(sum(int(Kint[t, i]) for t in keys)), len(keys)) for i in range(d)]


@pytest.mark.parametrize("b,L", [(2, 1), (2, 3), (3, 2), (4, 1), (3, 4)])
def test_build_matches_bottom_up_brute_force(b, L):
    rng = np.random.default_rng([b, L])
    d = 3
    for n_keys in list(range(1, 3 * b * b * L + 2)):
        Kint = rng.integers(-4, 5, size=(n_keys + 3, d))     # capacity > n_keys
        g = GO.grow_build(Kint.astype(np.float32)[None, None], "f32", n_keys, b, L)
        brute = _brute_tree(Kint, n_keys, b, L)
        assert g["levels"] == len(brute), n_keys
        for l, nodes in enumerate(brute):
            assert g["stored"][l].shape[2] == len(nodes), (n_keys, l)
            for n, keys in enumerate(nodes):
                want = _exact_means(Kint, keys)
                got = g["mean"][l][0, 0, n]
                for i in range(d):
                    assert abs(Fraction(float(got[i])) - want[i]) <= abs(want[i]) * Fraction(1, 2 ** 52)
                # stored = the fp64 mean rounded once to float32
                assert np.array_equal(g["stored"][l][0, 0, n], got.astype(np.float32))


def test_build_position_keys_closed_form():
    """K[t, i] = t + i: a node covering keys [lo, hi) has mean (lo + hi - 1) / 2 + i."""
    b, L, d = 3, 4, 5
    C = 200
    K = (np.arange(C)[:, None] + np.arange(d)[None, :]).astype(np.float32)[None, None]
    for n_keys in (1, 2, 4, 5, 12, 13, 36, 37, 100, 108, 109, 150):
        g = GO.grow_build(K, "f32", n_keys, b, L)
        lv = g["levels"]
        for l in range(1, lv + 1):
            M = b ** (lv - l) * L
            for n in range(g["mean"][l - 1].shape[2]):
                lo, hi = n * M, min((n + 1) * M, n_keys)
                expect = (lo + hi - 1) / 2.0 + np.arange(d)
                assert np.array_equal(g["mean"][l - 1][0, 0, n], expect)


# ---------------------------------------------------------------------------
# route: independent beam simulation over the brute-force tree
# ---------------------------------------------------------------------------

def _brute_route(Kint, q, n_keys, b, L, W):
    """Beam over the bottom-up tree: children of node n at level l are the
    nodes of level l+1 whose keys it contains; a node's score is q times its
    stored summary (the exact mean, rounded to fp64 and then to fp32, as a
    stored summary is defined), evaluated exactly with rationals; Python sort
    on (-score, index); returns the kept lists per level, ascending."""
    tree = _brute_tree(Kint, n_keys, b, L)

    def score_of(keys):
        mean = _exact_means(Kint, keys)
        stored = [Fraction(float(np.float32(float(m)))) for m in mean]
        return sum(int(q[i]) * stored[i] for i in range(len(q)))

    score = [[score_of(keys) for keys in lvl] for lvl in tree]
    kept = None
    out = []
    for l, lvl in enumerate(tree):
        if kept is None:
            cands = list(range(len(lvl)))
        else:
            cands = [c for c in range(len(lvl))
                     if any(set(lvl[c]) <= set(tree[l - 1][p]) for p in kept)]
        cands.sort(key=lambda n: (-score[l][n], n))
        kept = cands[:W]
        out.append(sorted(kept))
    return out


@pytest.mark.parametrize("b,L", [(2, 1), (2, 2), (3, 2), (4, 1)])
def test_route_matches_brute_force_beam(b, L):
    rng = np.random.default_rng([11, b, L])
    d = 3
    for n_keys in range(1, 2 * b * b * L + 3):
        for rep in range(2):
            Kint = rng.integers(-3, 4, size=(n_keys, d))
            q = rng.integers(-3, 4, size=d)
            g = GO.grow_build(Kint.astype(np.float32)[None, None], "f32", n_keys, b, L)
            n_leaves = g["stored"][-1].shape[2]
            for W in range(1, n_leaves + 2):
                r = GO.grow_route(q.astype(np.float32)[None, None], "f32", g["stored"],
                                  n_keys, b, L, W)
                want = _brute_route(Kint, q, n_keys, b, L, W)
                for l in range(len(want)):
                    got = [int(v) for v in r["trace"][0, 0, l] if v >= 0]
                    assert got == want[l], (n_keys, W, l)
                assert r["indices"][0, 0].tolist() == want[-1]


@pytest.mark.parametrize("b,L", [(2, 3), (3, 2), (4, 2)])
def test_route_wide_beam_is_global_top_existing_leaves(b, L):
    """A beam no smaller than the existing nodes of every level above the
    leaves cuts nothing before the last level, so the result is the global
    top-W existing leaves by (score desc, index asc) -- numpy lexsort."""
    rng = np.random.default_rng([13, b, L])
    d = 4
    for n_keys in (b * L + 1, b * b * L - 1, b * b * L + L + 1, 2 * b * b * L + 1):
        K = rng.integers(-3, 4, size=(n_keys, d)).astype(np.float32)
        q = rng.integers(-3, 4, size=d).astype(np.float32)
        g = GO.grow_build(K[None, None], "f32", n_keys, b, L)
        e = [s.shape[2] for s in g["stored"]]
        leaf_scores = np.array([K[j * L:min((j + 1) * L, n_keys)].astype(np.float64).mean(axis=0) @ q
                                for j in range(e[-1])])
        for W in range(max(e[:-1]) if len(e) > 1 else 1, e[-1] + 1):
            r = GO.grow_route(q[None, None], "f32", g["stored"], n_keys, b, L, W)
            order = np.lexsort((np.arange(e[-1]), -leaf_scores))
            assert r["indices"][0, 0].tolist() == sorted(order[:W].tolist()), (n_keys, W)


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(b=st.integers(2, 4), L=st.integers(1, 3), n_keys=st.integers(1, 90),
       W=st.integers(1, 40), seed=st.integers(0, 2 ** 31))
def test_route_candidates_exist_and_beam_counts(b, L, n_keys, W, seed):
    """Every candidate scored exists (covers a key), the kept count is
    min(W, #candidates) at each level, and the output has min(W, #leaves)
    distinct leaves, each a descendant of the nodes kept above it."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n_keys, 3)).astype(np.float32)
    q = rng.standard_normal(3).astype(np.float32)
    g = GO.grow_build(K[None, None], "f32", n_keys, b, L)
    lv = g["levels"]
    r = GO.grow_route(q[None, None], "f32", g["stored"], n_keys, b, L, W)
    e = [s.shape[2] for s in g["stored"]]
    prev = None
    for l in range(lv):
        kept = [int(v) for v in r["trace"][0, 0, l] if v >= 0]
        cands = list(range(min(b, e[0]))) if prev is None else \
            [p * b + c for p in prev for c in range(b) if p * b + c < e[l]]
        M = b ** (lv - 1 - l) * L
        assert all(c * M < n_keys for c in cands)
        assert set(kept) <= set(cands) and len(kept) == min(W, len(cands))
        prev = kept
    assert len(set(r["indices"][0, 0].tolist())) == min(W, e[-1])


# ---------------------------------------------------------------------------
# attend: short last block
# ---------------------------------------------------------------------------

def test_attend_full_beam_is_dense_over_the_cache_prefix():
    rng = np.random.default_rng(17)
    b, L, d, Hkv, G, C = 3, 5, 8, 2, 2, 80
    Kf = rng.standard_normal((1, Hkv, C, d)).astype(np.float32)
    Vf = rng.standard_normal((1, Hkv, C, d)).astype(np.float32)
    Qf = rng.standard_normal((1, Hkv * G, d)).astype(np.float32)
    for n_keys in (1, 4, 16, 46, 77):
        g = GO.grow_build(Kf, "f32", n_keys, b, L)
        W = g["stored"][-1].shape[2]
        r = GO.grow_route(Qf, "f32", g["stored"], n_keys, b, L, W)
        o = GO.grow_attend(Qf, Kf, Vf, "f32", r["indices"], n_keys, L)
        for hq in range(Hkv * G):
            k = Kf[0, hq // G, :n_keys].astype(np.float64)
            v = Vf[0, hq // G, :n_keys].astype(np.float64)
            want = scipy.special.softmax(k @ Qf[0, hq].astype(np.float64) / math.sqrt(d)) @ v
            np.testing.assert_allclose(o[0, hq], want, rtol=1e-12, atol=1e-13)


def test_attend_zero_keys_is_mean_of_existing_selected_values():
    """K = 0: every score ties, so the output is the plain mean of the value
    rows of the selected blocks, the last block holding only its existing
    keys (counted by hand)."""
    rng = np.random.default_rng(19)
    L, d, C, n_keys = 4, 3, 40, 23          # blocks 0..5, block 5 holds keys 20..22
    K = np.zeros((1, 1, C, d), dtype=np.float32)
    V = rng.integers(-5, 6, size=(1, 1, C, d)).astype(np.float32)
    Q = np.ones((1, 1, d), dtype=np.float32)
    for sel in ([5], [0, 5], [1, 3, 5, -1], [2, 2, 4]):
        o = GO.grow_attend(Q, K, V, "f32", np.array([[sel]]), n_keys, L)
        rows = []
        for j in sorted(set(s for s in sel if s >= 0)):
            rows += [t for t in range(j * L, (j + 1) * L) if t < n_keys]
        want = V[0, 0, rows].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(o[0, 0], want, rtol=1e-14, atol=1e-14)
    with pytest.raises(ValueError):
        GO.grow_attend(Q, K, V, "f32", np.array([[[6]]]), n_keys, L)
