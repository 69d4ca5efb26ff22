"""Pins of the oracles' tie measures against values worked out by hand.

The parity tests excuse an index mismatch only on a query whose oracle cut
gap (tree_route, grow_route, causal_prefill) is below 1e-5 relative, and
compare threshold survivors and outputs only where the sphere oracle's
margin is above 1e-12.  These measures therefore decide what a parity test
may forgive, so they are pinned here on hand-built trees whose scores are
small integers or dyadic fractions: every expected value below is the
fraction written out from the definition, not a re-evaluation of the
oracle's formula.

Definitions pinned (the tie band is the north-star's 1e-5 relative reading;
the sphere margin is the threshold analogue):
  * cut gap of a level that keeps W of more than W candidates:
    (s_W - s_{W+1}) / max(|s_W|, |s_{W+1}|), s_k the k-th best score in
    (score desc, node asc) order; 0 when both are 0; +inf at a level that
    keeps every candidate;
  * sphere route margin: the smallest |bound - tau| / max(|bound|, |tau|, 1)
    over every node whose bound was evaluated (pruned subtrees are not);
  * sphere attend margin: the smallest |q.k - tau| / max(|q.k|, |tau|, 1)
    over the keys of the listed leaves.

The values are chosen so that each plausible slip gives another number: the
gap taken one rank lower (s_{W+1} - s_{W+2}), without absolute values in the
denominator, over |s_W| or |s_{W+1}| alone, as an absolute difference, with
the sign flipped, or over children of nodes that were not kept; the margin
without the floor of 1, over kept nodes only, or over nodes of pruned
subtrees.
"""
from __future__ import annotations

from fractions import Fraction as F

import numpy as np
import pytest

from oracle import tis_causal_oracle as C
from oracle import tis_grow_oracle as GO
from oracle import tis_oracle as O
from oracle import tis_sphere_oracle as S


def _f(x) -> float:
    return float(x)


# ---------------------------------------------------------------- tree_route

def _two_level_tree():
    """b = 4, two levels, d = 4, one KV head; query k is the unit vector e_k,
    so its scores are coordinate k of the summaries.  Per query, (level-1
    coordinates, level-2 coordinates of the 16 leaves); entries that are not
    candidates for that query are 100, so scoring a child of a node that was
    not kept changes the result."""
    lvl1 = np.zeros((4, 4), dtype=np.float32)
    lvl2 = np.full((16, 4), 100.0, dtype=np.float32)
    # query 0: level 1 keeps {0, 2} (5, 4 | 3, 1): gap (4 - 3) / 4
    lvl1[:, 0] = [5, 3, 4, 1]
    # candidates 0..3, 8..11: 3 (7), then 0 and 10 tie at -2, lowest index 0 kept
    lvl2[[0, 1, 2, 3, 8, 9, 10, 11], 0] = [-2, -6, -6, 7, -3, -10, -2, -8]
    # query 1: level 1 keeps {1, 0} (-2, -3 | -5, -7): gap (-3 + 5) / 5
    lvl1[:, 1] = [-3, -2, -7, -5]
    # candidates 0..7: 6 (2), 0 (1) | 2 (0.5), ...: gap (1 - 0.5) / 1
    lvl2[0:8, 1] = [1, -1, 0.5, -4, 0, -1, 2, 0]
    # query 2: level 1 all zero, keeps {0, 1} by index: both scores 0, gap 0
    lvl1[:, 2] = [0, 0, 0, 0]
    # candidates 0..7: 9, 8 | 7: gap (8 - 7) / 8
    lvl2[0:8, 2] = [9, 8, 7, 6, 5, 4, 3, 2]
    # query 3: level 1 keeps {2, 0} (2, 1 | -1, -3): gap (1 + 1) / 1 = 2
    lvl1[:, 3] = [1, -1, 2, -3]
    # candidates 0..3, 8..11: 3 and 8 tie at 4 (both kept) | 2 (3): gap 1/4
    lvl2[[0, 1, 2, 3, 8, 9, 10, 11], 3] = [1, 2, 3, 4, 4, 3, 2, 1]
    stored = [lvl1[None, None], lvl2[None, None]]
    Q = np.eye(4, dtype=np.float32)[None]                 # [1, 4, 4]
    return Q, stored


TREE_GAPS = [
    [F(4 - 3, 4), F(0)],          # real tie at level 2 (-2 vs -2)
    [F(-3 + 5, 5), F(1, 2)],      # negative scores: |.| in the denominator
    [F(0), F(8 - 7, 8)],          # both scores 0 at the cut
    [F(1 + 1, 1), F(4 - 3, 4)],   # scores of opposite sign at the cut
]
TREE_LEAVES = [[0, 3], [0, 6], [0, 1], [3, 8]]


def test_tree_route_gap_closed_form():
    Q, stored = _two_level_tree()
    r = O.tree_route(Q, "f32", stored, branching=4, beam=2)
    assert r["indices"][0].tolist() == TREE_LEAVES
    want = np.array([[_f(g) for g in row] for row in TREE_GAPS])
    assert np.array_equal(r["gap"][0], want), (r["gap"][0].tolist(), want.tolist())


def test_tree_route_gap_is_inf_where_nothing_is_cut():
    """b = 2, beam 2: level 1 keeps both of its 2 candidates (no cut, +inf);
    level 2 cuts 4 candidates to 2.  Scores -1, 3 | 2, 3 -> kept {1, 3}
    (3, 3), gap (3 - 2) / 3 at level 2."""
    lvl1 = np.array([[1.0], [2.0]], dtype=np.float32)
    lvl2 = np.array([[-1.0], [3.0], [2.0], [3.0]], dtype=np.float32)
    Q = np.ones((1, 1, 1), dtype=np.float32)
    r = O.tree_route(Q, "f32", [lvl1[None, None], lvl2[None, None]], branching=2, beam=2)
    assert r["indices"][0, 0].tolist() == [1, 3]
    assert np.isposinf(r["gap"][0, 0, 0])
    assert r["gap"][0, 0, 1] == _f(F(1, 3))


def test_tree_route_gap_scale_free_and_signed():
    """The gap is relative: scaling every summary by 2^k (exact) leaves it
    unchanged; it is never negative (s_W >= s_{W+1} by the order)."""
    Q, stored = _two_level_tree()
    base = O.tree_route(Q, "f32", stored, branching=4, beam=2)["gap"]
    for k in (-20, 7):
        sc = [np.ldexp(s, k).astype(np.float32) for s in stored]
        assert np.array_equal(O.tree_route(Q, "f32", sc, branching=4, beam=2)["gap"], base)
    assert np.all(base >= 0)


# ---------------------------------------------------------------- grow_route

def test_grow_route_gap_closed_form():
    """b = 4, leaf block 1, 7 keys: depth 2, level 1 has 2 nodes (keys 0-3,
    4-6), level 2 has 7 leaves (child 7 of node 1 does not exist).  Beam 1.
    Query 0 (coordinate 0): level 1 (1 | 3) keeps node 1, gap (3 - 1) / 3;
    level 2 scores only the existing children 4, 5, 6 (9 | 8, 6), gap 1/9
    (leaves 0-3 hold 50 and must not be scored).  Query 1 (coordinate 1):
    level 1 ties at -1 (node 0 kept, gap 0); level 2 children 0-3
    (-4, -2 | -3, -8) keep leaf 1, gap (-2 + 3) / 3."""
    lvl1 = np.array([[1.0, -1.0], [3.0, -1.0]], dtype=np.float32)
    lvl2 = np.array([[50, -4], [50, -2], [50, -3], [50, -8], [6, 7], [9, 7], [8, 7]],
                    dtype=np.float32)
    Q = np.eye(2, dtype=np.float32)[None]
    r = GO.grow_route(Q, "f32", [lvl1[None, None], lvl2[None, None]], n_keys=7, branching=4,
                      leaf_block=1, beam=1)
    assert r["indices"][0].tolist() == [[5], [1]]
    want = np.array([[_f(F(2, 3)), _f(F(1, 9))], [0.0, _f(F(1, 3))]])
    assert np.array_equal(r["gap"][0], want), r["gap"][0].tolist()
    assert r["scored"][0].tolist() == [2 + 3, 2 + 4]
    # beam 2: level 1 keeps both nodes (+inf); level 2 scores all 7 leaves
    # (50, 40 | 30, 9, 8, 6, 1): gap (40 - 30) / 40, not the best score's
    lvl2b = np.array([[50], [40], [30], [1], [6], [9], [8]], dtype=np.float32)
    r = GO.grow_route(Q[:, :1, :1], "f32", [lvl1[None, None, :, :1], lvl2b[None, None]],
                      n_keys=7, branching=4, leaf_block=1, beam=2)
    assert r["indices"][0, 0].tolist() == [0, 1]
    assert np.isposinf(r["gap"][0, 0, 0])
    assert r["gap"][0, 0, 1] == _f(F(40 - 30, 40))


# ------------------------------------------------------------ causal_prefill

def test_causal_prefill_gap_closed_form():
    """b = 2, leaf block 1, keys 4, 2, 5, -1 (d = 1), query 1 at every
    position, beam 1.  Position 0: one leaf, nothing cut (+inf).  Position 1:
    leaves 4 | 2, gap 1/2.  Position 2 (depth 2): level 1 means 3 | 5 keep
    node 1, gap 2/5; its only existing child is leaf 2 (no cut).  Position 3:
    level 1 means 3 | 2 keep node 0, gap 1/3; leaves 4 | 2, gap 1/2; the
    smaller, 1/3, is the position's gap."""
    K = np.array([4.0, 2.0, 5.0, -1.0], dtype=np.float32).reshape(1, 1, 4, 1)
    V = np.zeros_like(K)
    Q = np.ones((1, 1, 4, 1), dtype=np.float32)
    r = C.causal_prefill(Q, K, V, "f32", branching=2, leaf_block=1, beam=1)
    assert r["indices"][0, 0, :, 0].tolist() == [0, 0, 2, 0]
    g = r["gap"][0, 0]
    assert np.isposinf(g[0])
    assert g[1:].tolist() == [_f(F(1, 2)), _f(F(2, 5)), _f(F(1, 3))]


# ------------------------------------------------------------ sphere margins

def _sphere_trees():
    """Two KV heads (one query each), b = 2, two levels, d = 2.
    Head 0: q = (3, 4), |q| = 5, tau = 10.  Level 1 bounds: centre (2, 1),
    r 1 -> 10 + 5 = 15 (survives, margin 5/15); centre (0, 0), r 1 -> 5
    (pruned, margin 5/10).  Level 2, children of node 0: centre (1, 1),
    r 0.5 -> 7 + 2.5 = 9.5 (pruned, margin 0.5/10); centre (4, 0), r 0 -> 12
    (survives, margin 2/12).  Children of the pruned node 1 have bound
    exactly tau (margin 0) and must not be evaluated.  Margin 1/20.
    Head 1: q = (0, 1/2), |q| = 1/2, tau = 1/4 (small values: the floor 1 of
    the denominator decides).  Level 1: centre (0, 1), r 0 -> 1/2 (survives,
    |1/2 - 1/4| / 1); centre (0, 0), r 1/4 -> 1/8 (pruned, 1/8 / 1).
    Level 2, children of node 0: centre (0, 2), r 0 -> 1 (survives, 3/4);
    centre (0, -1), r 1 -> 0 (pruned, 1/4).  Margin 1/8 (without the floor
    it would be 1/2)."""
    c1 = np.array([[[2, 1], [0, 0]], [[0, 1], [0, 0]]], dtype=np.float32)[None]
    r1 = np.array([[1, 1], [0, 0.25]], dtype=np.float32)[None]
    c2 = np.array([[[1, 1], [4, 0], [2, 1], [2, 1]],
                   [[0, 2], [0, -1], [0, 0.5], [0, 0.5]]], dtype=np.float32)[None]
    r2 = np.array([[0.5, 0, 0, 0], [0, 1, 0, 0]], dtype=np.float32)[None]
    Q = np.array([[[3, 4], [0, 0.5]]], dtype=np.float32)
    tau = np.array([[10.0, 0.25]], dtype=np.float32)
    return Q, [c1, c2], [r1, r2], tau


def test_sphere_route_margin_closed_form():
    Q, cs, rs, tau = _sphere_trees()
    r = S.threshold_route(Q, "f32", cs, rs, branching=2, tau=tau, max_nodes=4)
    assert r["counts"][0].tolist() == [1, 1]
    assert r["indices"][0, :, 0].tolist() == [1, 0]
    assert r["margin"][0].tolist() == [_f(F(1, 20)), _f(F(1, 8))]
    assert r["scored"][0].tolist() == [4, 4]


def test_sphere_route_margin_inf_for_infinite_tau():
    Q, cs, rs, _ = _sphere_trees()
    for t in (-np.inf, np.inf):
        tau = np.full((1, 2), t, dtype=np.float32)
        r = S.threshold_route(Q, "f32", cs, rs, branching=2, tau=tau, max_nodes=4)
        assert np.all(np.isposinf(r["margin"]))


def test_sphere_attend_margin_closed_form():
    """Leaves of 2 keys.  Head 0: q = (3, 4), tau = 10, leaf 1 listed with
    keys (2, 2) -> 14 (margin 4/14) and (4, 0) -> 12 (margin 2/12); leaf 0,
    not listed, holds (2, 1) -> exactly tau and must not count.  Margin 1/6.
    Head 1: q = (0, 1/2), tau = 1/4, leaf 0 listed with keys (0, 1) -> 1/2
    (|1/4| / 1) and (0, 3/4) -> 3/8 (1/8 / 1).  Margin 1/8 (without the
    floor: 1/3)."""
    Q, _, _, tau = _sphere_trees()
    K = np.array([[[2, 1], [2, 1], [2, 2], [4, 0]],
                  [[0, 1], [0, 0.75], [9, 9], [9, 9]]], dtype=np.float32)[None]
    V = np.zeros_like(K)
    idx = np.array([[[1, -1], [0, -1]]], dtype=np.int32)
    cnt = np.array([[1, 1]], dtype=np.int32)
    a = S.threshold_attend(Q, K, V, "f32", idx, cnt, leaf_block=2, tau=tau)
    assert a["margin"][0].tolist() == [_f(F(1, 6)), _f(F(1, 8))]
    assert a["selected"][0].tolist() == [2, 2]


@pytest.mark.parametrize("beam", [1, 2, 3])
def test_gap_band_splits_where_the_definition_says(beam):
    """A cut between 2 and 2(1 - 2^-20) (both exact in float32) has gap
    exactly 2^-20 and is tie-exposed (< 1e-5); at 2^-16 it is not.  Higher
    ranks hold 8, lower ones -1, so only the cut pair decides the gap."""
    for rel, exposed in ((2.0 ** -20, True), (2.0 ** -16, False)):
        vals = np.array([8.0] * (beam - 1) + [2.0, 2.0 * (1 - rel), -1.0], dtype=np.float32)
        Q = np.ones((1, 1, 1), dtype=np.float32)
        r = O.tree_route(Q, "f32", [vals.reshape(1, 1, -1, 1)], branching=len(vals), beam=beam)
        g = r["gap"][0, 0, 0]
        assert g == rel
        assert (g < 1e-5) == exposed
        assert r["indices"][0, 0].tolist() == list(range(beam))
