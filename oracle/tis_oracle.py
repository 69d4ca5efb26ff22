"""CPU oracle for tree-indexed sparse attention decode (fp64 numpy).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference the GPU
path is checked against. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does, and
it shares no code with the HIP library or its Python binding.

What is computed, and where it comes from
-----------------------------------------
"Subquadratic Attention with a Hierarchical Tree-Structured Indexer" (ZHA),
Abstract: every node of an index tree over the KV cache holds a compressed
summary of the keys below it, each level built on the one beneath; a later
query descends the tree level by level and ends with a small set of keys; a
query costs its descent plus the attention over that set.  "Vdev-Ctrl Releases ALHR", Technical Breakthrough and Core Features:
the tree is static and keys/values are routed hierarchically.  Progressive
Sparse Attention related-papers page (the NSA / InfLLMv2 abstract): blocks are
chosen by coarse scores and fine softmax attention runs on the selected tokens.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * summary of a node = arithmetic mean of the keys under it, computed exactly
    and rounded once to float32 (the stored summary), or, for reduced-precision
    summaries, rounded once, straight from the exact mean, to bfloat16 (round
    to nearest, ties to even; never through float32, which would round twice),
    or to fp8 e4m3 with a power-of-two scale per node (round_summary);
  * levels = branchings below the root; leaves = branching**levels contiguous
    blocks of leaf_block keys; the root is implicit and never scored;
  * node score = plain dot product q . summary (fp64, no scale);
  * beam = global top-`beam` over all children of all kept nodes at a level,
    ordered by (score descending, node index ascending);
  * selection is per query head; GQA maps q head h to KV head h // (Hq/Hkv);
  * final attention = exact softmax over the union of the selected leaf
    blocks with scale 1/sqrt(d), no mask; output float64 here.

Every function below is written from those definitions, not from any listing.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = ["widen", "round_summary", "round_e4m3", "fp8_scale_exponent", "tree_build",
           "tree_route", "tree_attend", "decode"]


# ---------------------------------------------------------------------------
# exact widening of the stored inputs
# ---------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored inputs to float64.

    dtype "f32": float32 values; "bf16": uint16 arrays of bf16 bit patterns
    (the bf16 value is the float32 whose high half is the pattern)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        hi = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# rounding of the exact means to the stored summary type
# ---------------------------------------------------------------------------

_E4M3_SIG_BITS = 4            # significant bits of an fp8 e4m3 value (3 stored + 1)
_E4M3_MIN_QUANTUM_EXP = -9    # spacing of e4m3 subnormals: 2^-9
_E4M3_MAX = 448.0             # largest finite e4m3 value (1.75 * 2^8)
_FP8_SCALE_EXP_RANGE = (-126, 127)   # the scale 2^e is a normal float32
_BF16_SIG_BITS = 8            # significant bits of a bfloat16 (7 stored + 1)
_BF16_MIN_QUANTUM_EXP = -133  # spacing of bfloat16 subnormals: 2^-133
_BF16_OVERFLOW = 2.0 ** 128   # the first power of two past the largest bfloat16


def fp8_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Per row, the smallest integer e with amax * 2^-e <= 448 (the largest
    e4m3 value), so the row's largest magnitude lands in (224, 448]; 0 for an
    all-zero row; clamped to [-126, 127] so that 2^e is a normal float32.
    With amax = f * 2^k, 0.5 <= f < 1, and 448 = 0.875 * 2^9: e = k - 9 when
    f <= 0.875, else k - 8."""
    amax = np.asarray(amax, dtype=np.float64)
    f, k = np.frexp(amax)
    e = np.where(f <= 0.875, k - 9, k - 8)
    e = np.where(amax == 0, 0, e)
    return np.clip(e, *_FP8_SCALE_EXP_RANGE).astype(np.int64)


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round to nearest even on the fp8 e4m3 grid (4 significant bits; below
    2^-6 the fixed subnormal spacing 2^-9), for |x| <= 448, from float64."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > _E4M3_MAX):
        raise ValueError("e4m3 rounding needs |x| <= 448")
    ax = np.abs(x)
    _, e = np.frexp(ax)
    q = np.maximum(e - _E4M3_SIG_BITS, _E4M3_MIN_QUANTUM_EXP)
    return np.copysign(np.ldexp(np.rint(np.ldexp(ax, -q)), q), x)


def round_summary(x: np.ndarray, summary_dtype: str) -> np.ndarray:
    """Exact float64 values rounded once to the stored summary type, returned
    as float32 (every bfloat16 value is a float32 value).

    "f32": IEEE round to nearest even.  "fp8": each row (the last axis, one
    node's summary) is scaled by 2^-e, e = fp8_scale_exponent(its largest
    magnitude), rounded once to e4m3 (round_e4m3) and scaled back: the stored
    value code * 2^e, exact in float32.  "bf16": round to nearest even on the
    bfloat16 grid (8 significant bits; below 2^-126 the fixed subnormal spacing
    2^-133), taken directly from the float64 value: x = m * 2^e with
    0.5 <= |m| < 1 lies on a grid of spacing 2^(e-8), so x / spacing is rounded
    to an integer (numpy's rint rounds halves to even) and scaled back; both
    scalings are by powers of two and exact.  Results of magnitude 2^128 or more
    overflow to infinity, as round to nearest gives."""
    x = np.asarray(x, dtype=np.float64)
    if summary_dtype == "f32":
        return x.astype(np.float32)
    if summary_dtype == "fp8":
        e = fp8_scale_exponent(np.abs(x).max(axis=-1))[..., None]
        return np.ldexp(round_e4m3(np.ldexp(x, -e)), e).astype(np.float32)
    if summary_dtype != "bf16":
        raise ValueError(f"unknown summary dtype {summary_dtype!r}")
    ax = np.abs(x)
    _, e = np.frexp(ax)
    q = np.maximum(e - _BF16_SIG_BITS, _BF16_MIN_QUANTUM_EXP)
    y = np.ldexp(np.rint(np.ldexp(ax, -q)), q)
    y = np.where(y >= _BF16_OVERFLOW, np.inf, y)
    return np.copysign(y, x).astype(np.float32)


def _check_geometry(n_keys: int, branching: int, leaf_block: int, levels: int) -> None:
    if branching < 2 or leaf_block < 1 or levels < 1:
        raise ValueError("need branching >= 2, leaf_block >= 1, levels >= 1")
    if n_keys != branching ** levels * leaf_block:
        raise ValueError("n_keys must equal branching**levels * leaf_block")


# ---------------------------------------------------------------------------
# build: node summary = mean of the keys under the node
# ---------------------------------------------------------------------------

def tree_build(K: np.ndarray, dtype: str, branching: int, leaf_block: int,
               levels: int, summary_dtype: str = "f32") -> Dict[str, List[np.ndarray]]:
    """Summaries of every node at levels 1..levels (ZHA Abstract: each tree
    node holds a compressed summary of the cached keys below it).

    K: [B, Hkv, N, d] stored keys. Level l has n_l = branching**l nodes; node
    n of level l covers the M_l = N / n_l contiguous keys [n*M_l, (n+1)*M_l).
    Its summary is the mean of those keys. Because all children of a node are
    equal-sized, this equals the recursive mean of child means.

    Returns {"mean": [fp64 [B,Hkv,n_l,d] for l=1..levels],
             "stored": [the same rounded once to summary_dtype ("f32" or
                        "bf16"), as float32 arrays]}.
    """
    B, H, N, d = K.shape
    _check_geometry(N, branching, leaf_block, levels)
    means = [np.empty((B, H, branching ** l, d), dtype=np.float64)
             for l in range(1, levels + 1)]
    for bi in range(B):
        for h in range(H):
            k64 = widen(K[bi, h], dtype)                      # [N, d]
            for l in range(1, levels + 1):
                n_l = branching ** l
                M_l = N // n_l
                node_sums = k64.reshape(n_l, M_l, d).sum(axis=1)
                means[l - 1][bi, h] = node_sums / M_l
            del k64
    stored = [round_summary(m, summary_dtype) for m in means]
    return {"mean": means, "stored": stored}


# ---------------------------------------------------------------------------
# route: top-down beam traversal
# ---------------------------------------------------------------------------

def tree_route(Q: np.ndarray, dtype: str, stored: Sequence[np.ndarray],
               branching: int, beam: int) -> Dict[str, np.ndarray]:
    """Top-down traversal that keeps a fixed beam of nodes per level (ZHA
    Abstract: a query descends the tree level by level to a small set of
    keys; ALHR post: the static tree routes keys level by level).

    Q: [B, Hq, d] stored queries; stored[l-1]: float32 [B, Hkv, n_l, d].
    Level 1 candidates are the `branching` children of the implicit root; at
    level l the candidates are all children of the nodes kept at level l-1.
    Each candidate is scored q . summary in fp64, candidates are ordered by
    (score desc, node index asc) and the first min(beam, #candidates) kept.

    Returns
      indices : int32 [B, Hq, min(beam, n_leaves)] selected leaves, ascending
      trace   : int32 [B, Hq, levels, beam] kept nodes per level, ascending,
                padded with -1
      gap     : fp64 [B, Hq, levels] relative score gap at the cut
                (sigma_W - sigma_W+1) / max(|sigma_W|, |sigma_W+1|),
                0 if both are 0, +inf where nothing was cut
      scored  : int64 [B, Hq] number of candidate summaries scored
    """
    B, Hq, d = Q.shape
    levels = len(stored)
    Hkv = stored[0].shape[1]
    if Hq % Hkv != 0:
        raise ValueError("q_heads must be a multiple of kv_heads")
    G = Hq // Hkv
    n_leaves = branching ** levels
    if not 1 <= beam <= n_leaves:
        raise ValueError("beam must lie in [1, branching**levels]")
    q64 = widen(Q, dtype)
    W_out = min(beam, n_leaves)
    indices = np.empty((B, Hq, W_out), dtype=np.int32)
    trace = np.full((B, Hq, levels, beam), -1, dtype=np.int32)
    gap = np.full((B, Hq, levels), np.inf, dtype=np.float64)
    scored = np.zeros((B, Hq), dtype=np.int64)
    children = np.arange(branching, dtype=np.int64)
    for bi in range(B):
        for hq in range(Hq):
            hk = hq // G
            q = q64[bi, hq]
            kept = None
            for l in range(1, levels + 1):
                if kept is None:
                    cand = children.copy()
                else:
                    cand = (kept[:, None] * branching + children[None, :]).ravel()
                summ = stored[l - 1][bi, hk][cand].astype(np.float64)
                sigma = summ @ q
                scored[bi, hq] += len(cand)
                order = np.lexsort((cand, -sigma))
                n_keep = min(beam, len(cand))
                if len(cand) > n_keep:
                    a, c = sigma[order[n_keep - 1]], sigma[order[n_keep]]
                    den = max(abs(a), abs(c))
                    gap[bi, hq, l - 1] = 0.0 if den == 0.0 else (a - c) / den
                kept = cand[order[:n_keep]]
                trace[bi, hq, l - 1, :n_keep] = np.sort(kept)
            indices[bi, hq] = np.sort(kept)
    return {"indices": indices, "trace": trace, "gap": gap, "scored": scored}


# ---------------------------------------------------------------------------
# attend: exact softmax over the keys of the selected leaf blocks
# ---------------------------------------------------------------------------

def tree_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str,
                indices: np.ndarray, leaf_block: int,
                scale: Optional[float] = None) -> np.ndarray:
    """Final attention restricted to the retrieved keys (ZHA Abstract: the
    attention after the descent; NSA/InfLLMv2 abstract on the Progressive
    Sparse Attention page: exact softmax over the tokens of the chosen blocks).

    The key set of a query is the union of the leaf blocks named in its row of
    `indices` ([B, Hq, W], any order; negative entries are empty slots;
    repeated entries count once). Scores s_t = scale * q . k_t, scale defaults
    to 1/sqrt(d); o = sum_t softmax(s)_t v_t, in fp64. A query whose set is
    empty gets a zero row. An entry >= N / leaf_block raises ValueError.
    Returns fp64 [B, Hq, d].
    """
    B, Hq, d = Q.shape
    _, Hkv, N, _ = K.shape
    G = Hq // Hkv
    n_blocks = N // leaf_block
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q64 = widen(Q, dtype)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for bi in range(B):
        for hq in range(Hq):
            hk = hq // G
            sel = np.asarray(indices[bi, hq], dtype=np.int64)
            if np.any(sel >= n_blocks):
                raise ValueError("leaf index out of range")
            blocks = np.unique(sel[sel >= 0])
            if blocks.size == 0:
                continue
            rows = (blocks[:, None] * leaf_block
                    + np.arange(leaf_block)[None, :]).ravel()
            k = widen(K[bi, hk, rows], dtype)
            v = widen(V[bi, hk, rows], dtype)
            s = scale * (k @ q64[bi, hq])
            p = np.exp(s - s.max())
            out[bi, hq] = (p @ v) / p.sum()
    return out


def decode(Q, K, V, dtype: str, branching: int, leaf_block: int, levels: int,
           beam: int, scale: Optional[float] = None) -> Dict[str, object]:
    """Build, route and attend in sequence (one decode step after a build)."""
    tree = tree_build(K, dtype, branching, leaf_block, levels)
    r = tree_route(Q, dtype, tree["stored"], branching, beam)
    o = tree_attend(Q, K, V, dtype, r["indices"], leaf_block, scale)
    return {"tree": tree, "route": r, "out": o}

