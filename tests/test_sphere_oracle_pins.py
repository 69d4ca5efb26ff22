"""Pins of the threshold-retrieval oracle (bounding spheres over the summary
tree).

The radius is pinned by exact rational arithmetic; the pruning by the
guarantee it exists for (no key whose score reaches tau is ever lost, so the
tree's answer equals dense halfspace attention), by an independent per-leaf
formulation of the survivors, by the special thresholds -inf / +inf, by
monotonicity in tau, and by the degenerate tree whose leaf spheres have
radius 0.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from oracle import tis_oracle as O
from oracle import tis_sphere_oracle as S


def _smallest_f32_with_square_at_least(D: Fraction) -> np.float32:
    """Brute force over float32 neighbours of sqrt(D), compared exactly."""
    r = np.float32(np.sqrt(float(D)))
    for _ in range(8):
        r = np.nextafter(r, np.float32(0)) if r > 0 else r
    while Fraction(float(r)) ** 2 < D:
        r = np.nextafter(r, np.float32(np.inf))
    return r


def test_round_up_radius_is_the_smallest_float32_whose_square_covers():
    rng = np.random.default_rng(1)
    D = np.concatenate([
        rng.uniform(0, 100, 3000),
        rng.uniform(0, 1, 1000) * 2.0 ** rng.integers(-60, 60, 1000),
        [0.0, 1.0, 2.0, 4.0, 1e-300],
    ])
    f = rng.standard_normal(1000).astype(np.float32)
    D = np.concatenate([D, f.astype(np.float64) ** 2,                    # exact squares
                        f.astype(np.float64) ** 2 * (1 + 2.0 ** -50)])   # just above
    got = S.round_up_radius(D)
    for x, r in zip(D, got):
        assert r == _smallest_f32_with_square_at_least(Fraction(float(x))), x
    # exact squares of float32 values come back unchanged
    assert np.array_equal(S.round_up_radius(f.astype(np.float64) ** 2), np.abs(f))
    with pytest.raises(ValueError):
        S.round_up_radius(np.array([-1.0]))


def _int_tree(b, L, lv, d, seed, B=1, H=2, span=9):
    rng = np.random.default_rng(seed)
    N = b ** lv * L
    K = rng.integers(-span, span + 1, size=(B, H, N, d)).astype(np.float32)
    return K


@pytest.mark.parametrize("b,L,lv", [(2, 4, 3), (4, 2, 2), (2, 1, 4)])
def test_radii_exact_on_integer_keys(b, L, lv):
    """Integer keys and power-of-two node sizes: the stored means are exact
    dyadic rationals, every squared distance is exact in float64, so the
    radius must be exactly the smallest float32 whose square covers the
    exact largest squared distance (computed here with Fractions)."""
    d = 5
    K = _int_tree(b, L, lv, d, seed=b * 10 + L)
    B, H, N, _ = K.shape
    tree = O.tree_build(K, "f32", b, L, lv)
    rad = S.node_radii(K, "f32", tree["stored"], b, L)
    for l in range(1, lv + 1):
        M = N // b ** l
        for bi in range(B):
            for h in range(H):
                for n in range(b ** l):
                    c = [Fraction(float(x)) for x in tree["stored"][l - 1][bi, h, n]]
                    Dx = max(sum((Fraction(float(k[i])) - c[i]) ** 2 for i in range(d))
                             for k in K[bi, h, n * M:(n + 1) * M])
                    assert rad["D"][l - 1][bi, h, n] == float(Dx)
                    assert rad["stored"][l - 1][bi, h, n] == _smallest_f32_with_square_at_least(Dx)


def test_every_key_lies_inside_its_stored_spheres():
    """Random float keys (inexact means): checked exactly with Fractions."""
    b, L, lv, d = 3, 5, 2, 6
    rng = np.random.default_rng(4)
    K = rng.standard_normal((1, 1, b ** lv * L, d)).astype(np.float32)
    tree = O.tree_build(K, "f32", b, L, lv)
    rad = S.node_radii(K, "f32", tree["stored"], b, L)
    N = K.shape[2]
    for l in range(1, lv + 1):
        M = N // b ** l
        for n in range(b ** l):
            c = [Fraction(float(x)) for x in tree["stored"][l - 1][0, 0, n]]
            r2 = Fraction(float(rad["stored"][l - 1][0, 0, n])) ** 2
            d2 = [sum((Fraction(float(k[i])) - c[i]) ** 2 for i in range(d))
                  for k in K[0, 0, n * M:(n + 1) * M]]
            assert max(d2) <= r2
            # and the radius is tight: one float32 step less no longer covers
            below = np.nextafter(rad["stored"][l - 1][0, 0, n], np.float32(0))
            assert max(d2) > Fraction(float(below)) ** 2 * (1 - Fraction(1, 2 ** 40))


def _case(b, L, lv, d, seed, G=2, H=2, dtype="f32"):
    rng = np.random.default_rng(seed)
    N = b ** lv * L
    K = rng.standard_normal((1, H, N, d)).astype(np.float32)
    V = rng.standard_normal((1, H, N, d)).astype(np.float32)
    Q = rng.standard_normal((1, H * G, d)).astype(np.float32) * 2
    tree = O.tree_build(K, dtype, b, L, lv)
    rad = S.node_radii(K, dtype, tree["stored"], b, L)
    return K, V, Q, tree, rad


def _tau_between_scores(Q, K, k_rank, G):
    """A threshold halfway between the k-th and (k+1)-th best scores of each
    query (float32), so exactly k keys reach it unless scores tie."""
    B, Hq, d = Q.shape
    tau = np.empty((B, Hq), dtype=np.float32)
    for bi in range(B):
        for hq in range(Hq):
            s = np.sort(K[bi, hq // G].astype(np.float64) @ Q[bi, hq].astype(np.float64))[::-1]
            tau[bi, hq] = np.float32((s[k_rank - 1] + s[k_rank]) / 2)
    return tau


@pytest.mark.parametrize("b,L,lv,k_rank", [(2, 4, 4, 1), (2, 4, 4, 7), (4, 8, 2, 20),
                                           (3, 5, 3, 40)])
def test_tree_answer_equals_dense_halfspace_attention(b, L, lv, k_rank):
    """No key that reaches tau is pruned: the threshold route + attend equal
    softmax over every key with q.k >= tau."""
    K, V, Q, tree, rad = _case(b, L, lv, 8, seed=k_rank)
    tau = _tau_between_scores(Q, K, k_rank, G=2)
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, tau, max_nodes=b ** lv)
    assert np.all(r["counts"] >= 0)
    a = S.threshold_attend(Q, K, V, "f32", r["indices"], r["counts"], L, tau)
    dense = S.halfspace_attend(Q, K, V, "f32", tau)
    assert np.all(a["selected"] >= 1)
    np.testing.assert_allclose(a["out"], dense, rtol=1e-12, atol=1e-12)
    # every leaf holding a key that reaches tau survived
    for hq in range(Q.shape[1]):
        s = K[0, hq // 2].astype(np.float64) @ Q[0, hq].astype(np.float64)
        need = set(np.nonzero(s >= tau[0, hq])[0] // L)
        have = set(r["indices"][0, hq, :r["counts"][0, hq]].tolist())
        assert need <= have


def test_survivors_match_a_per_leaf_formulation():
    """A leaf survives iff the bound of every node on its path from the root
    reaches tau (written leaf by leaf here, not level by level)."""
    b, L, lv = 2, 3, 5
    K, V, Q, tree, rad = _case(b, L, lv, 6, seed=9)
    qn = np.linalg.norm(Q.astype(np.float64), axis=-1)  # numpy's norm, not the oracle's
    for k_rank in (1, 5, 30):
        tau = _tau_between_scores(Q, K, k_rank, G=2)
        r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, tau, b ** lv)
        for hq in range(Q.shape[1]):
            q = Q[0, hq].astype(np.float64)
            alive = []
            for leaf in range(b ** lv):
                ok = True
                for l in range(1, lv + 1):
                    n = leaf // b ** (lv - l)
                    c = tree["stored"][l - 1][0, hq // 2, n].astype(np.float64)
                    bound = c @ q + qn[0, hq] * float(rad["stored"][l - 1][0, hq // 2, n])
                    ok = ok and bound >= float(tau[0, hq])
                alive.append(ok)
            want = np.nonzero(alive)[0]
            assert r["counts"][0, hq] == len(want)
            assert np.array_equal(r["indices"][0, hq, :len(want)], want)


def test_bound_is_never_below_a_key_score():
    b, L, lv = 4, 6, 3
    K, V, Q, tree, rad = _case(b, L, lv, 16, seed=21)
    qn = S.query_norm(Q, "f32")
    N = K.shape[2]
    for l in range(1, lv + 1):
        M = N // b ** l
        for hq in range(Q.shape[1]):
            q = Q[0, hq].astype(np.float64)
            c = tree["stored"][l - 1][0, hq // 2].astype(np.float64)
            bound = c @ q + qn[0, hq] * rad["stored"][l - 1][0, hq // 2].astype(np.float64)
            best = (K[0, hq // 2].astype(np.float64) @ q).reshape(b ** l, M).max(axis=1)
            assert np.all(best <= bound + 1e-9 * np.abs(bound))


def test_extreme_thresholds_and_monotonicity():
    b, L, lv = 2, 4, 3
    K, V, Q, tree, rad = _case(b, L, lv, 8, seed=3)
    Hq = Q.shape[1]
    lo = np.full((1, Hq), -np.inf, dtype=np.float32)
    hi = np.full((1, Hq), np.inf, dtype=np.float32)
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, lo, b ** lv)
    assert np.all(r["counts"] == b ** lv)
    a = S.threshold_attend(Q, K, V, "f32", r["indices"], r["counts"], L, lo)
    dense = O.tree_attend(Q, K, V, "f32", np.tile(np.arange(b ** lv), (1, Hq, 1)), L)
    np.testing.assert_allclose(a["out"], dense, rtol=1e-12, atol=1e-12)
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, hi, b ** lv)
    assert np.all(r["counts"] == 0) and np.all(r["indices"] == -1)
    a = S.threshold_attend(Q, K, V, "f32", r["indices"], r["counts"], L, hi)
    assert np.all(a["out"] == 0)
    prev = None
    for k_rank in (1, 3, 9, 20):
        tau = _tau_between_scores(Q, K, k_rank, G=2)
        r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, tau, b ** lv)
        sets = [set(r["indices"][0, h, :r["counts"][0, h]].tolist()) for h in range(Hq)]
        if prev is not None:
            assert all(p <= s for p, s in zip(prev, sets)), "a lower threshold lost a leaf"
        prev = sets


def test_overflow_is_reported():
    b, L, lv = 2, 4, 3
    K, V, Q, tree, rad = _case(b, L, lv, 8, seed=5)
    lo = np.full((1, Q.shape[1]), -np.inf, dtype=np.float32)
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, lo, max_nodes=b ** lv - 1)
    assert np.all(r["counts"] == -1) and np.all(r["indices"] == -1)
    a = S.threshold_attend(Q, K, V, "f32", r["indices"], r["counts"], L, lo)
    assert np.all(np.isnan(a["out"]))


def test_query_norm_closed_forms():
    """|q| of Pythagorean rows: (3, 4) -> 5, (2, 3, 6) -> 7, (1, 4, 8) -> 9,
    and a bf16 row (the pattern 0x4040 is 3.0, 0x4080 is 4.0) -> 5."""
    Q = np.zeros((1, 3, 3), dtype=np.float32)
    Q[0, 0, :2] = [3, 4]
    Q[0, 1] = [2, 3, 6]
    Q[0, 2] = [1, 4, 8]
    assert S.query_norm(Q, "f32").tolist() == [[5.0, 7.0, 9.0]]
    Qb = np.array([[[0x4040, 0x4080]]], dtype=np.uint16)
    assert S.query_norm(Qb, "bf16").tolist() == [[5.0]]


def test_radius_zero_leaves_prune_exactly():
    """Every leaf holds one repeated key: leaf spheres have radius 0, so a
    leaf survives exactly when its key reaches tau (no false positives at
    the leaves)."""
    b, L, lv, d = 2, 4, 4, 8
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((1, 1, b ** lv, d)).astype(np.float32)
    K = np.repeat(keys, L, axis=2)
    V = rng.standard_normal(K.shape).astype(np.float32)
    Q = rng.standard_normal((1, 3, d)).astype(np.float32)
    tree = O.tree_build(K, "f32", b, L, lv)
    rad = S.node_radii(K, "f32", tree["stored"], b, L)
    assert np.all(rad["stored"][-1] == 0)
    tau = _tau_between_scores(Q, K, 3 * L, G=3)
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, tau, b ** lv)
    for hq in range(3):
        s = keys[0, 0].astype(np.float64) @ Q[0, hq].astype(np.float64)
        want = np.nonzero(s >= tau[0, hq])[0]
        assert np.array_equal(r["indices"][0, hq, :r["counts"][0, hq]], want)


def test_bf16_inputs_and_bf16_summaries():
    """The sphere is about the stored centre whatever its type: with bfloat16
    summaries the radius grows to cover the rounding of the centre, and the
    answer is still the dense halfspace one."""
    b, L, lv, d = 4, 8, 2, 16
    rng = np.random.default_rng(12)
    bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    K = bits(rng.standard_normal((1, 2, b ** lv * L, d)))
    V = bits(rng.standard_normal((1, 2, b ** lv * L, d)))
    Q = bits(rng.standard_normal((1, 4, d)) * 2)
    for sd in ("f32", "bf16"):
        tree = O.tree_build(K, "bf16", b, L, lv, summary_dtype=sd)
        rad = S.node_radii(K, "bf16", tree["stored"], b, L)
        k64 = O.widen(K, "bf16")
        q64 = O.widen(Q, "bf16")
        tau = np.empty((1, 4), dtype=np.float32)
        for hq in range(4):
            s = np.sort(k64[0, hq // 2] @ q64[0, hq])[::-1]
            tau[0, hq] = np.float32((s[9] + s[10]) / 2)
        r = S.threshold_route(Q, "bf16", tree["stored"], rad["stored"], b, tau, b ** lv)
        a = S.threshold_attend(Q, K, V, "bf16", r["indices"], r["counts"], L, tau)
        np.testing.assert_allclose(a["out"], S.halfspace_attend(Q, K, V, "bf16", tau),
                                   rtol=1e-12, atol=1e-12)


def test_a_bound_or_score_at_the_threshold_survives():
    """Survival is bound >= tau and selection is q.k >= tau: a tau just below
    (by less than a float32 step) a node's bound keeps that node, and a tau
    at an exactly representable key score keeps that key."""
    b, L, lv, d = 2, 2, 3, 4
    K = np.array([[[[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0], [0, 0, 0, 1],
                    [2, 0, 0, 0], [0, 2, 0, 0], [0, 0, 2, 0], [0, 0, 0, 2],
                    [1, 1, 0, 0], [0, 1, 1, 0], [0, 0, 1, 1], [1, 0, 0, 1],
                    [3, 0, 0, 0], [0, 0, 0, 3], [1, 1, 1, 1], [0, 0, 0, 0]]]],
                 dtype=np.float32)
    V = np.arange(K.size, dtype=np.float32).reshape(K.shape) / K.size
    Q = np.array([[[1, 0, 0, 0]]], dtype=np.float32)
    tree = O.tree_build(K, "f32", b, L, lv)
    rad = S.node_radii(K, "f32", tree["stored"], b, L)
    qn = S.query_norm(Q, "f32")
    # a leaf survives when every bound on its path reaches tau: take the leaf
    # whose smallest path bound is largest and put tau at that bound (rounded
    # down to float32)
    q = Q[0, 0].astype(np.float64)
    path = np.full(b ** lv, np.inf)
    for l in range(1, lv + 1):
        c = tree["stored"][l - 1][0, 0].astype(np.float64)
        bound = c @ q + qn[0, 0] * rad["stored"][l - 1][0, 0].astype(np.float64)
        path = np.minimum(path, np.repeat(bound, b ** (lv - l)))
    top = int(np.argmax(path))
    t32 = np.float32(path[top])
    if float(t32) > path[top]:
        t32 = np.nextafter(t32, np.float32(-np.inf))
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, np.array([[t32]]), 8)
    assert top in r["indices"][0, 0, :r["counts"][0, 0]].tolist()
    # tau = 3 is the exact score of key 12 ([3, 0, 0, 0]): it alone is selected
    tau = np.array([[3.0]], dtype=np.float32)
    r = S.threshold_route(Q, "f32", tree["stored"], rad["stored"], b, tau, 8)
    a = S.threshold_attend(Q, K, V, "f32", r["indices"], r["counts"], L, tau)
    assert a["selected"][0, 0] == 1
    np.testing.assert_array_equal(a["out"][0, 0], V[0, 0, 12].astype(np.float64))
