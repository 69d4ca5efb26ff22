"""tis_probe_decode_timeline: the instrumented decode gives tis_tree_decode's
results bit for bit, and its per-wave phase stamps are complete and in
order.

The instrumented kernel is the fused decode with wall-clock stamps added, so
its output must equal the plain decode's exactly (the stamps change no
arithmetic).  Every workgroup's 16 waves pass entry, descent done, the
merge barrier and the end; the waves that gather pass the load phases; the
8 walking waves pass every scored level.  Stamps of one wave never go back
in time.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SLOTS, WAVES = 24, 16


def _say(*a):
    print("[timeline]", *a, flush=True)


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()  # raises if libtis.so is missing
    return t


def _w(name, b, L, lv, W, B, Hkv, G, seed, dtype="bf16", d=128):
    return workloads.Workload(name, dtype, B, Hkv * G, Hkv, d, b, L, lv, W, "normal", seed=seed)


CASES = [
    # unsplit: 128 queries over 32,768-key heads, two scored levels
    (_w("tl_unsplit", 8, 64, 3, 8, B=4, Hkv=8, G=4, seed=71), "f32"),
    # split queries (2 queries, 64 parts each), two scored levels
    (_w("tl_split", 4, 64, 5, 64, B=1, Hkv=2, G=2, seed=72), "f32"),
    # float32 inputs, d = 64, bfloat16 summaries, three scored levels
    (_w("tl_f32_d64", 4, 16, 4, 8, B=2, Hkv=2, G=3, seed=73, dtype="f32", d=64), "bf16"),
]


@pytest.mark.parametrize("w,sd", CASES, ids=[c[0].name for c in CASES])
def test_timeline_decode_matches_decode(tis, w, sd):
    _say(w.name, "summaries", sd)
    x = workloads.generate(w)
    Q, K, V = (tis.from_storage(x[k], w.dtype, "cuda") for k in ("Q", "K", "V"))
    plan = tis.DecodePlan(Q, K, V, w.branching, w.leaf_block, w.levels, w.beam,
                          summary_dtype=sd)
    plan.build()
    plan.decode()
    torch.cuda.synchronize()
    ref = plan.out.clone()
    nbytes = plan.timeline_bytes()
    assert nbytes > 0 and nbytes % (SLOTS * WAVES * 8) == 0
    tl = torch.zeros(nbytes // 8, dtype=torch.int64, device="cuda")
    plan.out.fill_(float("nan"))
    plan.decode_timeline(tl)
    torch.cuda.synchronize()
    assert torch.equal(plan.out, ref), "instrumented decode differs from tis_tree_decode"

    st = tl.cpu().numpy().reshape(-1, WAVES, SLOTS)
    groups = st.shape[0]
    first_cut = next((l for l in range(1, w.levels + 1)
                      if w.branching ** l > w.beam), w.levels + 1)
    scored = w.levels - first_cut + 1
    _say(w.name, "workgroups", groups, "scored levels", scored)
    # every wave of every workgroup: entry, descent done, merge barrier, end
    for k in (0, 1, 6, 7):
        assert (st[:, :, k] > 0).all(), k
    # the 8 walking waves stamp every scored level (scored, then ranked)
    for j in range(min(scored, 8)):
        assert (st[:, :8, 8 + 2 * j] > 0).all(), j
        assert (st[:, :8, 9 + 2 * j] > 0).all(), j
    # each wave's stamps go forward in phase order (slots it passed only)
    order = [0] + [s for j in range(min(scored, 8)) for s in (8 + 2 * j, 9 + 2 * j)] + \
        [1, 2, 3, 4, 5, 6, 7]
    seq = st[:, :, order].reshape(-1, len(order)).astype(np.int64)
    for row in seq:
        v = row[row > 0]
        assert (np.diff(v) >= 0).all(), row
    # at least one wave per workgroup gathered (first K load, keys, values)
    for k in (2, 3, 4):
        assert (st[:, :, k] > 0).any(axis=1).all(), k
    khz = tis.ops.lib().tis_wall_clock_khz(0)
    assert khz > 0
    span_us = (st[:, :, 7].max() - st[:, :, 0].min()) / khz * 1e3
    _say(w.name, f"clock {khz} kHz, launch span {span_us:.2f} us")
    assert 0 < span_us < 1e5
