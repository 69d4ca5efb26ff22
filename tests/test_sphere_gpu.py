"""Parity of threshold retrieval with bounding spheres (tis_tree_radii,
tis_tree_route_threshold, tis_tree_decode_threshold through the C-ABI) with
the CPU oracle in oracle/tis_sphere_oracle.py.

Radii: within one float32 step of the oracle's (both round up the fp64
largest squared distance; a different rounding needs that maximum to sit
within fp64 summation-order noise of a float32 square).  Survivors: exactly
the oracle's for every query whose closest bound-to-tau margin is above
1e-12 relative (the rest are counted and reported).  Output: within the input
type's tolerance of the oracle's attention over the GPU's survivors, for every
query whose closest key-score-to-tau margin is above 1e-12 relative, and equal
to dense halfspace attention there too.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import workloads
from oracle import tis_oracle as O
from oracle import tis_sphere_oracle as S
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MARGIN = 1e-12


def _say(*a):
    print("[sphere]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()
    return t


def _taus(x, w, k_rank):
    """Per query, halfway between its k-th and (k+1)-th best key score."""
    q = O.widen(x["Q"], w.dtype)
    tau = np.empty((w.batch, w.q_heads), dtype=np.float32)
    for bi in range(w.batch):
        for h in range(w.kv_heads):
            k = O.widen(x["K"][bi, h], w.dtype)
            s = -np.sort(-(q[bi, h * w.group:(h + 1) * w.group] @ k.T), axis=1)
            tau[bi, h * w.group:(h + 1) * w.group] = ((s[:, k_rank - 1] + s[:, k_rank]) / 2)
    return tau


def _radii_levels(tis, tree, radii):
    return [tis.radii_level(tree, radii, l).cpu().numpy() for l in range(1, tree.levels + 1)]


def check_case(tis, w, k_ranks, sd="f32", max_nodes=None, label=None):
    t0 = time.time()
    label = label or w.name
    x = workloads.generate(w)
    dev = "cuda"
    K = tis.from_storage(x["K"], w.dtype, dev)
    V = tis.from_storage(x["V"], w.dtype, dev)
    Q = tis.from_storage(x["Q"], w.dtype, dev)
    tree = tis.tree_build(K, w.branching, w.leaf_block, w.levels, summary_dtype=sd)
    radii = tis.tree_radii(K, tree)
    torch.cuda.synchronize()
    ob = O.tree_build(x["K"], w.dtype, w.branching, w.leaf_block, w.levels, summary_dtype=sd)
    orad = S.node_radii(x["K"], w.dtype, ob["stored"], w.branching, w.leaf_block)
    g_rad = _radii_levels(tis, tree, radii)
    eq, tot, worst = parity.compare_summaries(g_rad, orad["stored"])
    _say(f"{label} ({sd} summaries): radii bit-equal {eq}/{tot} (worst {worst} ulp), "
         f"{time.time() - t0:.1f}s")
    nodes = max_nodes or w.branching ** w.levels
    for k_rank in k_ranks:
        tau = _taus(x, w, k_rank)
        tau_d = torch.from_numpy(tau).to(dev)
        orr = S.threshold_route(x["Q"], w.dtype, ob["stored"], orad["stored"], w.branching, tau,
                                nodes)
        idx, cnt = tis.tree_route_threshold(Q, tree, radii, tau_d, nodes)
        out, didx, dcnt = tis.tree_decode_threshold(Q, K, V, tree, radii, tau_d, nodes,
                                                    return_indices=True)
        torch.cuda.synchronize()
        idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        out, didx, dcnt = out.cpu().numpy(), didx.cpu().numpy(), dcnt.cpu().numpy()
        assert np.array_equal(didx, idx) and np.array_equal(dcnt, cnt), "decode kept others"
        safe = orr["margin"] > MARGIN
        same = np.all(idx == orr["indices"], axis=-1) & (cnt == orr["counts"])
        assert np.all(same[safe]), f"{np.count_nonzero(~same & safe)} queries differ"
        parity.check_excused(int((~same & ~safe).sum()), same.size)
        oa = S.threshold_attend(x["Q"], x["K"], x["V"], w.dtype, idx, cnt, w.leaf_block, tau)
        ok = safe & (oa["margin"] > MARGIN)
        # queries left out of the output check: near-tie routes or key scores
        parity.check_excused(int((~ok & (cnt >= 0)).sum()), ok.size)
        err = parity.compare_outputs(out[ok], oa["out"][ok], w.dtype) if ok.any() else 0.0
        over = cnt < 0
        assert np.all(np.isnan(out[over]))
        kept = cnt[cnt >= 0]
        _say(f"{label} k={k_rank}: survivors exact {int(same.sum())}/{same.size} "
             f"(tie-exposed {int((~safe).sum())}); leaves kept mean "
             f"{float(kept.mean()) if kept.size else 0:.1f} max {int(kept.max()) if kept.size else 0}"
             f" of {w.branching ** w.levels}; overflow {int(over.sum())}; keys attended mean "
             f"{float(oa['selected'][~over].mean()) if (~over).any() else 0:.1f}; bounds scored "
             f"mean {float(orr['scored'].mean()):.0f}; max-abs {err:.2e}; "
             f"{time.time() - t0:.1f}s")
    return x, tree, radii


def _custom(name, dtype, b, L, lv, d=128, B=1, Hkv=2, G=3, gen="normal", seed=11, clusters=0):
    return workloads.Workload(name, dtype, B, Hkv * G, Hkv, d, b, L, lv, 4, gen,
                              clusters=clusters, seed=seed)


CASES = [
    # (workload, k_ranks, summary type)
    (_custom("sph_f32_d64", "f32", 2, 8, 4, d=64), (1, 9, 40), "f32"),
    (_custom("sph_bf16_d128", "bf16", 4, 16, 3), (1, 17, 100), "f32"),
    (_custom("sph_bf16_d128_bf16s", "bf16", 4, 16, 3), (1, 17, 100), "bf16"),
    (_custom("sph_f32_d128_bf16s", "f32", 3, 5, 3, G=2), (2, 30), "bf16"),
    (_custom("sph_ragged_bf16_d64", "bf16", 3, 7, 3, d=64), (3, 50), "f32"),
    (_custom("sph_deep_binary", "bf16", 2, 4, 9, d=64, Hkv=3, G=1), (1, 8, 64), "f32"),
    (_custom("sph_single_level", "bf16", 16, 8, 1), (4, 60), "f32"),
    (_custom("sph_clustered", "bf16", 8, 64, 2, B=2, Hkv=2, G=4, gen="mixture",
             clusters=32), (32, 100, 200), "f32"),
    # whole-wave leaf blocks (32, 64 and 96 keys: several row batches a
    # leaf), 1 to 8 levels, both head dims and summary types
    (_custom("sph_l32_d64", "bf16", 4, 32, 4, d=64), (1, 17, 90), "f32"),
    (_custom("sph_l64_lv6_bf16s", "bf16", 2, 64, 6), (1, 33), "bf16"),
    (_custom("sph_l96_lv8", "bf16", 2, 96, 8, d=64, Hkv=1, G=2), (2, 40), "f32"),
    (_custom("sph_l32_lv1", "bf16", 16, 32, 1, B=2), (3, 50), "f32"),
    # float32 keys in leaf blocks of 64 keys or more (4 lanes a key, 4 keys a lane)
    (_custom("sph_f32_l64_d128", "f32", 4, 64, 3), (1, 20, 100), "f32"),
    (_custom("sph_f32_l128_d64_bf16s", "f32", 2, 128, 4, d=64), (2, 70), "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_threshold_matches_oracle(tis, case):
    w, k_ranks, sd = case
    check_case(tis, w, k_ranks, sd=sd)


def test_dense_halfspace_equality_and_extremes(tis):
    """Away from ties the tree's answer is dense halfspace attention; tau =
    -inf keeps every leaf (dense attention), +inf none (zero rows); too small
    a max_nodes overflows (counts -1, NaN rows)."""
    w = _custom("sph_extremes", "f32", 2, 4, 4, d=64, G=2, seed=5)
    x, tree, radii = check_case(tis, w, (5,))
    dev = "cuda"
    K = tis.from_storage(x["K"], w.dtype, dev)
    V = tis.from_storage(x["V"], w.dtype, dev)
    Q = tis.from_storage(x["Q"], w.dtype, dev)
    tau = _taus(x, w, 5)
    out = tis.tree_decode_threshold(Q, K, V, tree, radii, torch.from_numpy(tau).to(dev), 16)
    dense = S.halfspace_attend(x["Q"], x["K"], x["V"], w.dtype, tau)
    parity.compare_outputs(out.cpu().numpy(), dense, w.dtype)
    n_leaves = w.branching ** w.levels
    for t, want in ((-np.inf, n_leaves), (np.inf, 0)):
        tt = torch.full((w.batch, w.q_heads), t, dtype=torch.float32, device=dev)
        out, idx, cnt = tis.tree_decode_threshold(Q, K, V, tree, radii, tt, n_leaves,
                                                  return_indices=True)
        torch.cuda.synchronize()
        assert np.all(cnt.cpu().numpy() == want)
        if want == 0:
            assert np.all(out.cpu().numpy() == 0)
        else:
            all_idx = np.tile(np.arange(n_leaves), (w.batch, w.q_heads, 1))
            parity.compare_outputs(out.cpu().numpy(), O.tree_attend(
                x["Q"], x["K"], x["V"], w.dtype, all_idx, w.leaf_block), w.dtype)
    tt = torch.full((w.batch, w.q_heads), -np.inf, dtype=torch.float32, device=dev)
    out, idx, cnt = tis.tree_decode_threshold(Q, K, V, tree, radii, tt, n_leaves - 1,
                                              return_indices=True)
    torch.cuda.synchronize()
    assert np.all(cnt.cpu().numpy() == -1) and np.all(idx.cpu().numpy() == -1)
    assert np.all(np.isnan(out.cpu().numpy()))


@pytest.mark.timeout(900)
def test_full_size_gqa_32k(tis):
    """The 32K-key GQA workload at full size: radii of every node, survivors
    and output of every query, at a threshold that keeps each query's own
    cluster (its 64 best keys)."""
    w = workloads.get("gqa_32k")
    check_case(tis, w, (64,), max_nodes=512, label="gqa_32k (full size)")
