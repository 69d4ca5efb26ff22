"""Pins of the oracle's reduced-precision summaries (bfloat16, and fp8 e4m3
with a power-of-two scale per node, of the exact node means, rounded once).

The rounding is pinned against torch's float32 -> bfloat16 and float32 ->
float8_e4m3fn conversions (round to nearest even, library routines
independent of the oracle) on values that
are float32 numbers, where one rounding from float64 and one from float32 are
the same operation; against hand-built ties and a double-rounding witness for
values that are not; and against closed-form node means for the build.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import tis_grow_oracle as GO
from oracle import tis_oracle as O

torch = pytest.importorskip("torch")


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 by torch, returned as float32."""
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def _bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def test_bf16_equals_torch_on_float32_values():
    rng = np.random.default_rng(5)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        # every exponent of the normal range, random significands
        (rng.uniform(1, 2, 4000) * 2.0 ** rng.integers(-126, 128, 4000)).astype(np.float32),
        # float32 subnormals, which land on the bfloat16 subnormal grid or round onto it
        (rng.integers(1, 1 << 23, 2000) * 2.0 ** -149).astype(np.float32),
        # ties on the bfloat16 grid: the low 16 bits exactly 0x8000
        ((rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
    ]
    x = np.concatenate(parts)
    x = x[np.isfinite(x)]
    x = np.concatenate([x, -x])
    got = O.round_summary(x.astype(np.float64), "bf16")
    assert np.array_equal(_bits(got), _bits(_torch_bf16(x)))


def test_bf16_rounds_once_from_float64():
    """1 + 2^-8 + 2^-30 lies above the midpoint of 1 and 1 + 2^-7, so it rounds
    up; through float32 it would first become the midpoint 1 + 2^-8 exactly and
    then round to the even neighbour 1."""
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, -(1 + 2.0 ** -8 + 2.0 ** -30)])
    assert np.array_equal(O.round_summary(x, "bf16"), np.array([1 + 2.0 ** -7, -(1 + 2.0 ** -7)],
                                                               dtype=np.float32))
    via_f32 = _torch_bf16(x.astype(np.float32))
    assert np.array_equal(via_f32, np.array([1.0, -1.0], dtype=np.float32))


def test_bf16_ties_go_to_even_and_near_ties_to_the_nearer():
    v = 1 + np.arange(128) * 2.0 ** -7          # every bfloat16 in [1, 2)
    up = v + 2.0 ** -7
    mid = v + 2.0 ** -8
    even = np.where(np.arange(128) % 2 == 0, v, up)
    assert np.array_equal(O.round_summary(mid, "bf16"), even.astype(np.float32))
    assert np.array_equal(O.round_summary(mid - 2.0 ** -40, "bf16"), v.astype(np.float32))
    assert np.array_equal(O.round_summary(mid + 2.0 ** -40, "bf16"), up.astype(np.float32))
    # the same grid at another binade, scaled by a power of two
    assert np.array_equal(O.round_summary(mid * 2.0 ** -70, "bf16"),
                          (even * 2.0 ** -70).astype(np.float32))


def test_bf16_error_bound_grid_and_idempotence():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(50000) * 2.0 ** rng.integers(-60, 60, 50000)
    r = O.round_summary(x, "bf16").astype(np.float64)
    assert np.all(_bits(r) & 0xFFFF == 0), "not a bfloat16 value"
    _, e = np.frexp(x)
    assert np.all(np.abs(r - x) <= 2.0 ** (e - 9))  # half the spacing 2^(e-8)
    assert np.array_equal(O.round_summary(r, "bf16"), r.astype(np.float32))
    order = np.argsort(x)
    assert np.all(np.diff(r[order]) >= 0), "rounding must be monotone"


def test_bf16_zero_subnormal_and_overflow():
    mx = (2 - 2.0 ** -7) * 2.0 ** 127            # largest bfloat16
    half = 2.0 ** 119                            # half its spacing
    x = np.array([0.0, -0.0, mx, mx + half * 0.999, mx + half, 1e300,
                  2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -140])
    want = np.array([0.0, -0.0, mx, mx, np.inf, np.inf,
                     2.0 ** -133, 0.0, 2 * 2.0 ** -133, 0.0], dtype=np.float32)
    got = O.round_summary(x, "bf16")
    assert np.array_equal(_bits(got), _bits(want))


def test_f32_summaries_are_plain_float32_rounding():
    x = np.random.default_rng(2).standard_normal(1000)
    assert np.array_equal(O.round_summary(x, "f32"), x.astype(np.float32))
    with pytest.raises(ValueError):
        O.round_summary(x, "fp16")


@pytest.mark.parametrize("b,L,lv", [(2, 16, 6), (8, 64, 2), (3, 5, 3)])
def test_build_bf16_summaries_position_keys(b, L, lv):
    """K[t, i] = t + i (exact in float32 here): a node over keys [lo, hi) has
    mean (lo + hi - 1) / 2 + i, a float32 number, so its bfloat16 summary is
    torch's rounding of that closed form."""
    N, d = b ** lv * L, 8
    t = np.arange(N, dtype=np.float64)[:, None] + np.arange(d)[None, :]
    K = t.astype(np.float32)[None, None]
    tree = O.tree_build(K, "f32", b, L, lv, summary_dtype="bf16")
    for l in range(1, lv + 1):
        M = N // b ** l
        lo = np.arange(b ** l) * M
        closed = ((2 * lo + M - 1) / 2)[:, None] + np.arange(d)[None, :]
        assert np.array_equal(tree["mean"][l - 1][0, 0], closed)
        assert np.array_equal(tree["stored"][l - 1][0, 0],
                              _torch_bf16(closed.astype(np.float32)))


def test_build_bf16_constant_keys_and_f32_default():
    rng = np.random.default_rng(3)
    c = O.round_summary(rng.standard_normal(16), "bf16")     # bfloat16 values
    K = np.broadcast_to(c, (1, 2, 2 ** 3 * 4, 16)).astype(np.float32)
    tree = O.tree_build(K, "f32", 2, 4, 3, summary_dtype="bf16")
    for s in tree["stored"]:
        assert np.array_equal(s, np.broadcast_to(c, s.shape))
    plain = O.tree_build(K, "f32", 2, 4, 3)
    for a, m in zip(plain["stored"], plain["mean"]):
        assert np.array_equal(a, m.astype(np.float32))


def test_grow_build_bf16_partial_nodes():
    """Growing-cache nodes cut at n: the last node of each level averages only
    the keys it holds; with position keys that mean is a closed form again."""
    b, L, d = 2, 4, 4
    cap = 2 ** 4 * L
    K = (np.arange(cap, dtype=np.float64)[:, None] + np.arange(d)[None, :]).astype(
        np.float32)[None, None]
    for n in (1, 5, 37, 63, 64):
        g = GO.grow_build(K, "f32", n, b, L, summary_dtype="bf16")
        lv = g["levels"]
        for l in range(1, lv + 1):
            M = b ** (lv - l) * L
            e = -(-n // M)
            lo = np.arange(e) * M
            hi = np.minimum(lo + M, n)
            closed = ((lo + hi - 1) / 2)[:, None] + np.arange(d)[None, :]
            assert np.array_equal(g["stored"][l - 1][0, 0], _torch_bf16(closed.astype(np.float32)))


# ------------------------------------------------------------ fp8 e4m3 --

def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(
        torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_equals_torch_on_float32_values():
    rng = np.random.default_rng(21)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
        # ties on the e4m3 grid of [1, 2): k/8 + 1/16
        1 + (np.arange(8) * 2 + 1) / 16.0,
        # subnormal range and the smallest values
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 2000), [2.0 ** -10, 3 * 2.0 ** -11, 448.0, -448.0, 0.0],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = O.round_e4m3(x.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, _torch_e4m3(x))
    with pytest.raises(ValueError):
        O.round_e4m3(np.array([449.0]))


def test_e4m3_rounds_once_from_float64():
    """1 + 2^-4 + 2^-30 lies just above the midpoint of 1 and 1.125: it rounds
    up; through float32 it would become the midpoint and round to even, 1."""
    x = np.array([1 + 2.0 ** -4 + 2.0 ** -30])
    assert O.round_e4m3(x)[0] == 1.125
    assert _torch_e4m3(x.astype(np.float32))[0] == 1.0
    # and as a node summary (a row whose scale is 2^0 because of the 448)
    row = np.array([[1 + 2.0 ** -4 + 2.0 ** -30, 448.0]])
    assert np.array_equal(O.round_summary(row, "fp8"), np.array([[1.125, 448.0]], dtype=np.float32))


def test_fp8_scale_is_the_smallest_that_fits():
    rng = np.random.default_rng(22)
    amax = np.concatenate([rng.uniform(0, 1, 5000) * 2.0 ** rng.integers(-60, 60, 5000),
                           448.0 * 2.0 ** np.arange(-5, 6), [448.0 * (1 + 2.0 ** -40)]])
    e = O.fp8_scale_exponent(amax)
    assert np.all(np.ldexp(amax, -e) <= 448)
    assert np.all(np.ldexp(amax, -(e - 1)) > 448)
    assert O.fp8_scale_exponent(np.array([0.0]))[0] == 0
    assert O.fp8_scale_exponent(np.array([1e-300]))[0] == -126   # clamped: 2^e stays normal


def test_fp8_summaries_are_per_row_and_scale_equivariant():
    rng = np.random.default_rng(23)
    m = rng.standard_normal((6, 32)) * 0.1
    s = O.round_summary(m, "fp8")
    # each row: code * 2^e with the row's own e, codes on the e4m3 grid
    e = O.fp8_scale_exponent(np.abs(m).max(axis=1))
    codes = np.ldexp(s.astype(np.float64), -e[:, None])
    assert np.array_equal(O.round_e4m3(codes), codes)
    assert np.all(np.abs(codes).max(axis=1) > 224)   # the largest lands in (224, 448]
    # scaling one row by a power of two scales its stored values exactly
    m2 = m.copy()
    m2[2] *= 2.0 ** 13
    s2 = O.round_summary(m2, "fp8")
    assert np.array_equal(s2[2].astype(np.float64), s[2].astype(np.float64) * 2.0 ** 13)
    assert np.array_equal(np.delete(s2, 2, axis=0), np.delete(s, 2, axis=0))
    # half-spacing error bound: 2^(k-5) for |x| = f 2^k, at least 2^-10 before scaling back
    _, k = np.frexp(np.abs(np.ldexp(m, -e[:, None])))
    bound = np.ldexp(1.0, np.maximum(k - 5, -10) + e[:, None])
    assert np.all(np.abs(s - m) <= bound)
    assert np.array_equal(O.round_summary(np.zeros((2, 8)), "fp8"), np.zeros((2, 8)))


@pytest.mark.parametrize("b,L,lv", [(2, 16, 4), (8, 64, 2)])
def test_build_fp8_summaries_position_keys(b, L, lv):
    """Position keys: node means are the closed form (lo + hi - 1) / 2 + i,
    float32 numbers; each node's fp8 summary is torch's e4m3 rounding of the
    row scaled by its power of two."""
    N, d = b ** lv * L, 8
    t = np.arange(N, dtype=np.float64)[:, None] + np.arange(d)[None, :]
    K = t.astype(np.float32)[None, None]
    tree = O.tree_build(K, "f32", b, L, lv, summary_dtype="fp8")
    for l in range(1, lv + 1):
        M = N // b ** l
        lo = np.arange(b ** l) * M
        closed = ((2 * lo + M - 1) / 2)[:, None] + np.arange(d)[None, :]
        e = O.fp8_scale_exponent(np.abs(closed).max(axis=1))[:, None]
        want = np.ldexp(_torch_e4m3(np.ldexp(closed, -e).astype(np.float32)).astype(np.float64), e)
        assert np.array_equal(tree["stored"][l - 1][0, 0], want.astype(np.float32))
