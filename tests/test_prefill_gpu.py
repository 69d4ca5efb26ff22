"""Parity of causal prefill routing (tis_causal_prefill through the C-ABI)
with the CPU oracle in oracle/tis_causal_oracle.py: every position's kept
leaves exactly (positions whose oracle cut gap is below 1e-5 are counted
instead), every position's output within the input type's tolerance of the
oracle's attention over the GPU's leaves.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import workloads
from oracle import tis_causal_oracle as C
from oracle import tis_grow_oracle as GO
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[prefill]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()
    return t


def _inputs(dtype, B, Hkv, G, N, d, gen, seed, b=2, L=16):
    lv = GO.depth_for(N, b, L)
    clusters = b ** lv * L // 64 if gen == "mixture" else 0
    w = workloads.Workload("prefill", dtype, B, Hkv * G, Hkv, d, b, L, lv, 1, gen,
                           clusters=clusters, seed=seed)
    x = workloads.generate(w)
    rng = np.random.default_rng(seed + 1000)
    K = np.ascontiguousarray(x["K"][:, :, :N])
    V = np.ascontiguousarray(x["V"][:, :, :N])
    # one query per position: the workload's queries plus per-position noise
    q = workloads.generate(workloads.Workload("prefill_q", dtype, B, Hkv * G, Hkv, d, b, L, lv,
                                              1, "normal", seed=seed + 7))
    qf = O_widen(q["Q"], dtype)[:, :, None, :] + rng.standard_normal((B, Hkv * G, N, d))
    Q = to_storage(qf, dtype)
    return Q, K, V


def O_widen(x, dtype):
    return workloads.bf16_bits_to_f32(x).astype(np.float64) if dtype == "bf16" else \
        np.asarray(x, dtype=np.float64)


def to_storage(x, dtype):
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return x32 if dtype == "f32" else workloads.f32_to_bf16_bits(x32)


CASES = [
    # (label, dtype, summary type, B, Hkv, G, N, d, b, L, beam, generator)
    ("alhr_shape", "f32", "f32", 1, 1, 8, 1024, 64, 2, 16, 2, "normal"),
    ("ragged_bf16_d128", "bf16", "f32", 1, 2, 2, 301, 128, 3, 5, 4, "normal"),
    ("clustered_bf16", "bf16", "f32", 2, 1, 4, 640, 128, 4, 16, 3, "mixture"),
    ("bf16_summaries", "bf16", "bf16", 1, 2, 2, 200, 64, 2, 8, 3, "normal"),
    ("wide_beam", "f32", "f32", 1, 1, 2, 129, 64, 2, 4, 40, "normal"),
    ("leaf_1", "f32", "f32", 1, 1, 2, 50, 64, 2, 1, 3, "normal"),
    # workgroup sizes by candidates a level (beam * b): one wave up to 32
    # (most cases above), two waves up to 64, four up to 128, else eight
    ("cand_48", "bf16", "f32", 1, 2, 2, 500, 128, 4, 8, 12, "normal"),
    ("cand_48_f32_d64", "f32", "f32", 1, 1, 3, 333, 64, 6, 5, 8, "normal"),
    # more than 128 candidates a level (8-wave workgroups)
    ("cand_160", "bf16", "f32", 1, 2, 2, 700, 128, 8, 4, 20, "normal"),
    # leaf blocks of a multiple of 16 keys, 32 or more: attention 16
    # positions at a time on the matrix cores, a wave per query head, 4, 2
    # or 1 heads of a KV group a workgroup (group 3: one); positions not a
    # multiple of 16, leaves of 2, 3 and 4 key tiles
    ("tiles_L32_ragged_g3", "bf16", "f32", 1, 2, 3, 333, 128, 3, 32, 5, "normal"),
    ("tiles_L48_f32_bf16s_g2", "f32", "bf16", 2, 1, 2, 250, 64, 2, 48, 3, "normal"),
    # a wide beam: up to 64 * 12 leaves in a workgroup's union
    ("tiles_L32_beam_12_g4", "f32", "f32", 1, 1, 4, 400, 128, 2, 32, 12, "mixture"),
    ("tiles_L64_bf16_d64_g8", "bf16", "f32", 1, 2, 8, 300, 64, 4, 64, 2, "normal"),
    ("tiles_L32_bf16_g1", "bf16", "bf16", 2, 3, 1, 129, 64, 4, 32, 3, "normal"),
    # a beam whose union table does not fit 4 heads' LDS: 2 heads a workgroup
    ("tiles_L32_beam_48_g4", "bf16", "f32", 1, 1, 4, 200, 64, 2, 32, 48, "normal"),
    # fewer positions than a tile: one workgroup row block, 7 rows
    ("tiles_7_positions", "f32", "f32", 1, 2, 4, 7, 128, 2, 32, 2, "normal"),
    ("tiles_1_position", "bf16", "f32", 1, 1, 2, 1, 64, 2, 32, 1, "normal"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_causal_prefill_matches_oracle(tis, case):
    _check_case(tis, *case)


# Values far from zero: an output is then a weighted mean of values near the
# offset, so any mismatch between the weights the numerator uses and those
# the denominator sums shows at the offset's scale.  The tile path keeps the
# weights at fp32 precision (bf16 high and low parts), so its error stays at
# the fp32 accumulation level, far inside the bf16 bar.
V_OFFSET_CASES = [
    ("tiles_L32_v_offset_64", "bf16", "f32", 1, 2, 3, 333, 128, 3, 32, 5, "normal"),
    ("tiles_L64_v_offset_64_g4", "bf16", "f32", 1, 1, 4, 700, 128, 4, 64, 6, "mixture"),
    ("fused_L16_v_offset_64", "bf16", "f32", 1, 1, 2, 300, 64, 2, 16, 3, "normal"),
]


@pytest.mark.parametrize("case", V_OFFSET_CASES, ids=[c[0] for c in V_OFFSET_CASES])
def test_causal_prefill_values_with_offset(tis, case):
    err = _check_case(tis, *case, v_offset=64.0)
    assert err <= 2e-3, f"max-abs {err:.3g} with values near 64"


def _check_case(tis, label, dtype, sd, B, Hkv, G, N, d, b, L, beam, gen, v_offset=0.0):
    t0 = time.time()
    Q, K, V = _inputs(dtype, B, Hkv, G, N, d, gen, seed=N, b=b, L=L)
    if v_offset:
        V = to_storage(O_widen(V, dtype) + v_offset, dtype)
    cap = N + 37  # the cache has room past the prefilled keys
    Kc = np.zeros((B, Hkv, cap, d), dtype=K.dtype)
    Vc = np.zeros_like(Kc)
    Kc[:, :, :N], Vc[:, :, :N] = K, V
    Kd = tis.from_storage(Kc, dtype, "cuda")
    Vd = tis.from_storage(Vc, dtype, "cuda")
    Qd = tis.from_storage(Q, dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L, summary_dtype=sd)
    ct.append(N)
    out, idx = ct.causal_prefill(Qd, beam, return_indices=True)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    orc = C.causal_prefill(Q, K, V, dtype, b, L, beam, summary_dtype=sd)
    _say(f"{label}: oracle done in {time.time() - t0:.1f}s")
    tie = orc["gap"] < parity.TIE_GAP
    same = np.all(idx == orc["indices"], axis=-1)
    assert np.all(same | tie), f"{np.count_nonzero(~same & ~tie)} positions keep other leaves"
    parity.check_excused(int((~same & tie).sum()), same.size, what="positions")
    # outputs: the oracle's attention over the GPU's leaves, position by position
    err = 0.0
    Bq, Hq = Q.shape[:2]
    for t in range(N):
        o_g = GO.grow_attend(np.ascontiguousarray(Q[:, :, t]), K, V, dtype, idx[:, :, t], t + 1, L)
        err = max(err, parity.compare_outputs(out[:, :, t], o_g, dtype))
    reads = np.array([[[C.keys_read(idx[bi, h, t], t + 1, L) for t in range(N)]
                       for h in range(Hq)] for bi in range(Bq)])
    _say(f"{label}: positions exact {int(same.sum())}/{same.size} (tie-exposed mismatches "
         f"{int((~same & tie).sum())}); keys read per query {reads.mean():.2f} on average over "
         f"{N} positions (dense causal: {(N + 1) / 2:.1f}); max-abs {err:.2e}; "
         f"{time.time() - t0:.1f}s")
    return err


@pytest.mark.timeout(900)
def test_prefill_gqa_4096_positions_sampled(tis):
    """The benchmark's prefill launch (the GQA workload's first 4,096 keys,
    all 128 query heads, one query per position), checked at sampled
    positions: the first, leaf and node boundaries, depth changes, the last."""
    w = workloads.get("gqa_32k")
    x = workloads.generate(w)
    P = 4096
    rng = np.random.default_rng(99)
    q = O_widen(x["Q"], w.dtype)[:, :, None, :] + rng.standard_normal(
        (w.batch, w.q_heads, P, w.head_dim))
    Q = to_storage(q, w.dtype)
    Kd = tis.from_storage(x["K"], w.dtype, "cuda")
    Vd = tis.from_storage(x["V"], w.dtype, "cuda")
    Qd = tis.from_storage(Q, w.dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, w.branching, w.leaf_block)
    ct.append(P)
    out, idx = ct.causal_prefill(Qd, w.beam, return_indices=True)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    L = w.leaf_block
    pos = np.unique(np.array([0, 1, L - 1, L, 8 * L - 1, 8 * L, 8 * L + 1, 64 * L - 1, 64 * L,
                              1000, 2047, 2048, P - 2, P - 1]))
    pos = pos[pos < P]
    K = np.ascontiguousarray(x["K"][:, :, :P])
    V = np.ascontiguousarray(x["V"][:, :, :P])
    orc = C.causal_prefill(Q, K, V, w.dtype, w.branching, L, w.beam, positions=pos)
    tie = orc["gap"] < parity.TIE_GAP
    same = np.all(idx[:, :, pos] == orc["indices"], axis=-1)
    assert np.all(same | tie), f"{np.count_nonzero(~same & ~tie)} sampled positions differ"
    parity.check_excused(int((~same & tie).sum()), same.size, what="positions")
    err = 0.0
    for i, t in enumerate(pos):
        o_g = GO.grow_attend(np.ascontiguousarray(Q[:, :, t]), K, V, w.dtype, idx[:, :, t],
                             int(t) + 1, L)
        err = max(err, parity.compare_outputs(out[:, :, t], o_g, w.dtype))
    _say(f"gqa_32k prefill of {P} positions: {len(pos)} sampled positions x "
         f"{w.batch * w.q_heads} queries exact {int(same.sum())}/{same.size} (tie-exposed "
         f"{int((~same & tie).sum())}); max-abs {err:.2e}")


LONG = [
    # (label, dtype, b, L, d, G, positions, beam, sampled positions)
    # spans of 5 * 3^h, not multiples of 64: node starts fall inside the
    # 64-key runs; 9,000 keys take the runs of 4,096 as well as those of 64
    ("span_ragged_9000", "f32", 3, 5, 64, 2, 9000, 4,
     [0, 63, 64, 3644, 3645, 3646, 3708, 3709, 4095, 4096, 4097, 7289, 7290, 7291, 8191, 8192,
      8959, 8960, 8999]),
    # past 64^3 keys: runs of 262,144 keys too
    ("runs_262144", "bf16", 4, 16, 64, 2, 270_000, 4,
     [0, 4095, 4096, 65535, 65536, 131071, 200_000, 262_143, 262_144, 262_207, 262_208, 269_999]),
    # the 16-position attention over a long prefill (leaves of 32 keys, 4
    # heads a workgroup): unions of many leaves per tile, the last tile
    # partial
    ("tiles_20000", "bf16", 4, 32, 64, 4, 20_000, 6,
     [0, 15, 16, 31, 32, 1000, 4095, 4096, 8191, 8192, 12_345, 16_383, 16_384, 19_983, 19_984,
      19_999]),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", LONG, ids=[c[0] for c in LONG])
def test_prefill_long_sampled(tis, case):
    """Long prefills, where a position's open node starts tens of thousands
    of keys back: the partial means come from fp64 sums over runs of 64,
    4,096, 262,144 keys.  Checked at sampled positions (node and run
    boundaries on both sides) against the oracle."""
    label, dtype, b, L, d, G, P, beam, pos = case
    t0 = time.time()
    rng = np.random.default_rng(P)
    K = to_storage(rng.standard_normal((1, 1, P, d)), dtype)
    V = to_storage(rng.standard_normal((1, 1, P, d)), dtype)
    Q = to_storage(rng.standard_normal((1, G, P, d)), dtype)
    Kd = tis.from_storage(K, dtype, "cuda")
    Vd = tis.from_storage(V, dtype, "cuda")
    Qd = tis.from_storage(Q, dtype, "cuda")
    ct = tis.CacheTree(Kd, Vd, b, L)
    ct.append(P)
    out, idx = ct.causal_prefill(Qd, beam, return_indices=True)
    torch.cuda.synchronize()
    pos = np.array(pos)
    out, idx = out[:, :, pos].cpu().numpy(), idx[:, :, pos].cpu().numpy()
    _say(f"{label}: GPU prefill of {P} positions done, {time.time() - t0:.1f}s")
    orc = C.causal_prefill(Q, K, V, dtype, b, L, beam, positions=pos)
    tie = orc["gap"] < parity.TIE_GAP
    same = np.all(idx == orc["indices"], axis=-1)
    assert np.all(same | tie), f"{np.count_nonzero(~same & ~tie)} sampled positions differ"
    parity.check_excused(int((~same & tie).sum()), same.size, what="positions")
    err = 0.0
    for i, t in enumerate(pos):
        o_g = GO.grow_attend(np.ascontiguousarray(Q[:, :, t]), K, V, dtype, idx[:, :, i],
                             int(t) + 1, L)
        err = max(err, parity.compare_outputs(out[:, :, i], o_g, dtype))
    _say(f"{label}: {len(pos)} sampled positions x {G} queries exact {int(same.sum())}/"
         f"{same.size} (tie-exposed {int((~same & tie).sum())}); max-abs {err:.2e}; "
         f"{time.time() - t0:.1f}s")
