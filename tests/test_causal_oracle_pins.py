"""Pins of the causal prefill oracle (every position routes over the tree of
its own prefix and attends causally).

Pinned by: dense causal softmax when the beam keeps every node; causal
invariance (changing keys after a position changes nothing at it); the full
tree oracle at the last position of a whole tree; closed forms of the keys
read per position for two key patterns whose routing is known in advance
(all scores tied: the lowest leaves; scores growing with position: the
newest leaves, the partial one included).
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import tis_causal_oracle as C
from oracle import tis_oracle as O


def _rand(B, Hq, Hkv, N, d, seed, dtype="f32"):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    Q = rng.standard_normal((B, Hq, N, d)).astype(np.float32)
    return Q, K, V


def _dense_causal(Q, K, V):
    B, Hq, N, d = Q.shape
    G = Hq // K.shape[1]
    out = np.zeros((B, Hq, N, d))
    for bi in range(B):
        for h in range(Hq):
            k = K[bi, h // G].astype(np.float64)
            v = V[bi, h // G].astype(np.float64)
            s = (Q[bi, h].astype(np.float64) @ k.T) / np.sqrt(d)
            s[np.triu_indices(N, 1)] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[bi, h] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("b,L,N", [(2, 4, 37), (3, 2, 30), (2, 1, 20)])
def test_full_beam_is_dense_causal_attention(b, L, N):
    Q, K, V = _rand(1, 4, 2, N, 6, seed=N)
    leaves = -(-N // L)
    r = C.causal_prefill(Q, K, V, "f32", b, L, beam=leaves)
    np.testing.assert_allclose(r["out"], _dense_causal(Q, K, V), rtol=1e-12, atol=1e-12)
    assert np.array_equal(r["keys_read"], np.broadcast_to(np.arange(1, N + 1), r["keys_read"].shape))


def test_positions_never_see_later_keys():
    Q, K, V = _rand(1, 2, 1, 48, 8, seed=3)
    a = C.causal_prefill(Q, K, V, "f32", 2, 4, beam=2)
    for t in (0, 5, 15, 16, 31, 40):
        K2, V2 = K.copy(), V.copy()
        K2[:, :, t + 1:] = np.random.default_rng(t).standard_normal(K2[:, :, t + 1:].shape)
        V2[:, :, t + 1:] = 7.0
        b = C.causal_prefill(Q, K2, V2, "f32", 2, 4, beam=2, positions=np.arange(t + 1))
        assert np.array_equal(a["indices"][:, :, :t + 1], b["indices"])
        assert np.array_equal(a["out"][:, :, :t + 1], b["out"])


@pytest.mark.parametrize("b,L,lv,W", [(2, 4, 4, 3), (4, 8, 2, 5)])
def test_last_position_of_a_whole_tree_is_the_full_tree_decode(b, L, lv, W):
    N = b ** lv * L
    Q, K, V = _rand(1, 3, 1, N, 8, seed=b * lv)
    r = C.causal_prefill(Q, K, V, "f32", b, L, W, positions=np.array([N - 1]))
    full = O.decode(np.ascontiguousarray(Q[:, :, -1]), K, V, "f32", b, L, lv, W)
    assert np.array_equal(r["indices"][:, :, 0], full["route"]["indices"])
    np.testing.assert_allclose(r["out"][:, :, 0], full["out"], rtol=1e-12, atol=1e-12)


def test_keys_read_when_every_score_ties():
    """Identical keys: every score ties and the lowest indices win, so each
    position keeps leaves 0 .. W-1 and reads min(t + 1, W * L) keys."""
    b, L, W, N, d = 2, 16, 2, 1024, 4
    rng = np.random.default_rng(0)
    K = np.broadcast_to(rng.standard_normal(d).astype(np.float32), (1, 1, N, d)).copy()
    V = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    Q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    pos = np.array([0, 1, 15, 16, 17, 31, 32, 33, 100, 511, 1023])
    r = C.causal_prefill(Q, K, V, "f32", b, L, W, positions=pos)
    assert np.array_equal(r["keys_read"][0, 0], np.minimum(pos + 1, W * L))
    for i, t in enumerate(pos):
        want = np.arange(min(W, -(-(t + 1) // L)))
        assert np.array_equal(r["indices"][0, 0, i, :len(want)], want)


def test_keys_read_when_scores_grow_with_position():
    """K[t] = t e1 and q = e1: newer keys score higher, every node mean grows
    with the node index, so each level keeps its newest nodes and a position
    reads the newest W leaves: min(t + 1, r + (W - 1) L), r the keys in the
    partial newest leaf.  The average over 1,024 positions is a closed form."""
    b, L, W, N, d = 2, 16, 2, 1024, 4
    K = np.zeros((1, 1, N, d), dtype=np.float32)
    K[0, 0, :, 0] = np.arange(N)
    V = np.random.default_rng(1).standard_normal((1, 1, N, d)).astype(np.float32)
    Q = np.zeros((1, 1, N, d), dtype=np.float32)
    Q[..., 0] = 1.0
    pos = np.arange(0, N, 7)
    r = C.causal_prefill(Q, K, V, "f32", b, L, W, positions=pos)
    n = pos + 1
    rem = (n - 1) % L + 1
    want = np.minimum(n, rem + (W - 1) * L)
    assert np.array_equal(r["keys_read"][0, 0], want)
    newest = (n - 1) // L
    assert np.array_equal(r["indices"][0, 0].max(axis=-1), newest)
    # over all 1,024 positions: positions 1..16 read themselves (8.5 on
    # average), the other 1,008 read 16 + (1..16) (24.5 on average)
    n_all = np.arange(1, N + 1)
    avg = np.minimum(n_all, (n_all - 1) % L + 1 + (W - 1) * L).mean()
    assert avg == (16 * 8.5 + 1008 * 24.5) / 1024 == 24.25


def test_bf16_summaries_follow_the_same_definition():
    Q, K, V = _rand(1, 2, 1, 40, 8, seed=9)
    a = C.causal_prefill(Q, K, V, "f32", 2, 4, beam=40 // 4, summary_dtype="bf16")
    np.testing.assert_allclose(a["out"], _dense_causal(Q, K, V), rtol=1e-12, atol=1e-12)


def test_gap_is_the_smallest_level_gap():
    """A hand-worked prefix: d = 1, q = 1, b = 2, L = 1, beam 1, keys
    4, 0, 1, 1.  At position 3 (all 4 keys, two levels) level 1 compares the
    means 2 and 1 (relative gap (2 - 1) / 2 = 1/2) and keeps node 0; level 2
    compares its leaves 4 and 0 (gap (4 - 0) / 4 = 1).  At position 2 the
    second node holds key 2 alone (mean 1): the gaps are 1/2 and 1 again.
    At position 1 (keys 4, 0, one level) the only gap is 1, and at position 0
    nothing is cut (+inf).  The reported gap is the smallest level's."""
    K = np.array([4, 0, 1, 1], dtype=np.float32).reshape(1, 1, 4, 1)
    V = np.arange(4, dtype=np.float32).reshape(1, 1, 4, 1)
    Q = np.ones((1, 1, 4, 1), dtype=np.float32)
    r = C.causal_prefill(Q, K, V, "f32", 2, 1, 1)
    assert r["gap"][0, 0].tolist() == [np.inf, 1.0, 0.5, 0.5]
    assert r["indices"][0, 0, :, 0].tolist() == [0, 0, 0, 0]
