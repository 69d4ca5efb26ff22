"""CPU oracle for a tree over a growing KV cache (fp64 numpy).

TEST INFRASTRUCTURE ONLY, like tis_oracle: the slow, plain reference that the
GPU's incrementally maintained tree is checked against.  Only the test suite,
the smoke check and the CPU baseline leg of the benchmark may import it; it
shares no code with the HIP library or its Python binding.

What is computed, and where it comes from
-----------------------------------------
"Subquadratic Attention with a Hierarchical Tree-Structured Indexer" (ZHA),
Abstract: the summary tree sits over the KV cache and its depth grows step by
step as the context gets longer.  "Vdev-Ctrl Releases ALHR": keys arrive one
decode step at a time.  The pages define no tree for a cache whose length is
not a whole number of full subtrees, so this module takes the plainest
reading that keeps every other definition of tis_oracle unchanged:

  * depth: the tree over N keys has the fewest levels lv >= 1 for which
    branching**lv * leaf_block >= N (it gains a level exactly when N first
    exceeds branching**lv * leaf_block);
  * node n of level l covers keys [n * M_l, (n + 1) * M_l) cut at N, with
    M_l = branching**(lv - l) * leaf_block; a node exists when it covers at
    least one key (n * M_l < N);
  * summary = exact mean of the keys the node covers, rounded once to float32
    (or bfloat16, as tis_oracle.round_summary does);
  * route: as in tis_oracle, but the candidates of a level are only the
    children that exist; the beam is min(beam, number of candidates);
  * attend: as in tis_oracle, with leaf block j holding keys
    [j * leaf_block, (j + 1) * leaf_block) cut at N.

With N = branching**levels * leaf_block every function here gives exactly what
the tis_oracle function of the same role gives (the tests pin that).  How the
tree reached N (one build, or a build and any sequence of appends) does not
enter the definition: the oracle always describes the tree of the first N keys.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle.tis_oracle import round_summary, widen

__all__ = ["depth_for", "grow_build", "grow_route", "grow_attend"]


def depth_for(n_keys: int, branching: int, leaf_block: int) -> int:
    """Fewest levels lv >= 1 with branching**lv * leaf_block >= n_keys."""
    if n_keys < 1 or branching < 2 or leaf_block < 1:
        raise ValueError("need n_keys >= 1, branching >= 2, leaf_block >= 1")
    lv = 1
    while branching ** lv * leaf_block < n_keys:
        lv += 1
    return lv


def _existing(n_keys: int, branching: int, leaf_block: int, lv: int, level: int) -> int:
    """Number of level-`level` nodes that cover at least one of the N keys."""
    M = branching ** (lv - level) * leaf_block
    return -(-n_keys // M)


def grow_build(K: np.ndarray, dtype: str, n_keys: int, branching: int,
               leaf_block: int, summary_dtype: str = "f32") -> Dict[str, object]:
    """Summaries of every existing node of the tree over the first n_keys keys.

    K: [B, Hkv, C, d] stored keys of a cache with room for C >= n_keys keys
    (rows past n_keys are ignored).  Returns
      levels : lv = depth_for(n_keys, ...)
      mean   : [fp64 [B, Hkv, e_l, d] for l = 1..lv], e_l existing nodes
      stored : the same rounded once to summary_dtype ("f32" or "bf16",
               tis_oracle.round_summary), as float32 arrays
    """
    B, H, C, d = K.shape
    if not 1 <= n_keys <= C:
        raise ValueError("need 1 <= n_keys <= cache capacity")
    lv = depth_for(n_keys, branching, leaf_block)
    means = []
    for l in range(1, lv + 1):
        M = branching ** (lv - l) * leaf_block
        e = _existing(n_keys, branching, leaf_block, lv, l)
        means.append(np.empty((B, H, e, d), dtype=np.float64))
    for bi in range(B):
        for h in range(H):
            k64 = widen(K[bi, h, :n_keys], dtype)             # [N, d]
            for l in range(1, lv + 1):
                M = branching ** (lv - l) * leaf_block
                for n in range(means[l - 1].shape[2]):
                    lo, hi = n * M, min((n + 1) * M, n_keys)
                    means[l - 1][bi, h, n] = k64[lo:hi].sum(axis=0) / (hi - lo)
            del k64
    stored = [round_summary(m, summary_dtype) for m in means]
    return {"levels": lv, "mean": means, "stored": stored}


def grow_route(Q: np.ndarray, dtype: str, stored: Sequence[np.ndarray], n_keys: int,
               branching: int, leaf_block: int, beam: int) -> Dict[str, np.ndarray]:
    """Top-down beam traversal over the existing nodes (tis_oracle.tree_route
    with each level's candidates cut to the children that exist).

    Returns indices (int32 [B, Hq, min(beam, e_lv)], ascending), trace
    (int32 [B, Hq, lv, beam], -1 padded), gap (fp64 [B, Hq, lv], +inf where
    nothing was cut) and scored (int64 [B, Hq]), with the meanings of
    tis_oracle.tree_route."""
    B, Hq, d = Q.shape
    lv = len(stored)
    if lv != depth_for(n_keys, branching, leaf_block):
        raise ValueError("stored levels do not match n_keys")
    Hkv = stored[0].shape[1]
    G = Hq // Hkv
    e = [stored[l].shape[2] for l in range(lv)]   # existing nodes per level
    if beam < 1:
        raise ValueError("beam must be >= 1")
    q64 = widen(Q, dtype)
    W_out = min(beam, e[-1])
    indices = np.empty((B, Hq, W_out), dtype=np.int32)
    trace = np.full((B, Hq, lv, beam), -1, dtype=np.int32)
    gap = np.full((B, Hq, lv), np.inf, dtype=np.float64)
    scored = np.zeros((B, Hq), dtype=np.int64)
    children = np.arange(branching, dtype=np.int64)
    for bi in range(B):
        for hq in range(Hq):
            hk = hq // G
            q = q64[bi, hq]
            kept = None
            for l in range(1, lv + 1):
                if kept is None:
                    cand = children.copy()
                else:
                    cand = (kept[:, None] * branching + children[None, :]).ravel()
                cand = cand[cand < e[l - 1]]
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


def grow_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str,
                indices: np.ndarray, n_keys: int, leaf_block: int,
                scale: Optional[float] = None) -> np.ndarray:
    """Exact softmax over the keys of the selected leaf blocks, each block cut
    at n_keys (tis_oracle.tree_attend with a last block that may be short).

    K, V: [B, Hkv, C, d] with C >= n_keys.  Negative entries are empty slots,
    repeats count once, an entry >= ceil(n_keys / leaf_block) raises
    ValueError; an empty set gives a zero row.  Returns fp64 [B, Hq, d]."""
    B, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    n_blocks = -(-n_keys // leaf_block)
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
            rows = np.concatenate([np.arange(j * leaf_block, min((j + 1) * leaf_block, n_keys))
                                   for j in blocks])
            k = widen(K[bi, hk, rows], dtype)
            v = widen(V[bi, hk, rows], dtype)
            s = scale * (k @ q64[bi, hq])
            p = np.exp(s - s.max())
            out[bi, hq] = (p @ v) / p.sum()
    return out
