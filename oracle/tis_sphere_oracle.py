"""CPU oracle for threshold retrieval over the summary tree with bounding
spheres (fp64 numpy).

TEST INFRASTRUCTURE ONLY, like tis_oracle: the slow, plain reference the GPU
path is checked against.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; it shares no code with the HIP
library or its Python binding.

What is computed, and where it comes from
-----------------------------------------
"Sparse Attention as a Range Searching Problem" (gist.science explainer of
Louver), Methodologie: sparse attention as exact retrieval of every key whose
score q.k reaches a threshold tau (a halfspace range query); keys are grouped
in clusters, each enclosed by a bounding sphere (centre c, radius rho); a
cluster whose sphere does not meet the halfspace is pruned, which can never
drop a key that reaches tau; the surviving keys are checked exactly.  Here
the clusters are the nodes of the summary tree of tis_oracle ("Subquadratic
Attention with a Hierarchical Tree-Structured Indexer", Abstract), so the
pruning runs level by level down the tree.  Readings (the pages give no
formulas for this combination):

  * centre of a node = its stored summary (the mean, rounded once, as
    tis_oracle.tree_build stores it); radius = the smallest float32 r >= 0
    with r^2 >= D, where D is the largest squared distance from the stored
    centre to a key under the node, evaluated in float64.  Rounding up keeps
    every key inside the stored sphere;
  * the largest score any point of the sphere can reach is
    q.c + |q| r (Cauchy-Schwarz); a node survives when that bound is >= tau,
    evaluated in float64 (|q| = sqrt of the float64 sum of squares);
  * traversal: the candidates of level 1 are the root's children, those of
    level l the children of the level-(l-1) survivors; a level may keep at
    most `max_nodes` survivors, more is an overflow (count -1, no leaves);
  * attention: exact softmax, scale 1/sqrt(d) by default, over the keys of the
    surviving leaves whose float64 score q.k is >= tau; no such key: a zero
    row; overflow: a NaN row.

Because no key with q.k >= tau is ever pruned, the result equals softmax over
every key of the cache with q.k >= tau (halfspace_attend), which the tests
check.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle.tis_oracle import widen

__all__ = ["round_up_radius", "node_radii", "threshold_route", "threshold_attend",
           "halfspace_attend", "query_norm"]


def round_up_radius(D: np.ndarray) -> np.ndarray:
    """Smallest float32 r >= 0 with r * r >= D (float64 D >= 0).  r * r is
    exact in float64 for a float32 r, so each comparison is exact; the
    float32 nearest sqrt(D) is moved up or down a step until it is the
    smallest one that qualifies."""
    D = np.asarray(D, dtype=np.float64)
    if np.any(D < 0) or not np.all(np.isfinite(D)):
        raise ValueError("squared distances must be finite and >= 0")
    r = np.sqrt(D).astype(np.float32)
    for _ in range(4):
        low = r.astype(np.float64) ** 2 < D
        r = np.where(low, np.nextafter(r, np.float32(np.inf)), r)
    for _ in range(4):
        down = np.nextafter(r, np.float32(0))
        ok = (r > 0) & (down.astype(np.float64) ** 2 >= D)
        r = np.where(ok, down, r)
    assert np.all(r.astype(np.float64) ** 2 >= D)
    return r.astype(np.float32)


def node_radii(K: np.ndarray, dtype: str, stored: Sequence[np.ndarray], branching: int,
               leaf_block: int) -> Dict[str, List[np.ndarray]]:
    """Radius of every node about its stored summary.

    K: [B, Hkv, N, d] stored keys; stored[l-1]: [B, Hkv, b^l, d] summaries (as
    float32 arrays).  Returns {"D": [float64 [B, Hkv, b^l]] largest squared
    distances, "stored": [float32 radii, round_up_radius(D)]}."""
    B, H, N, d = K.shape
    lv = len(stored)
    if N != branching ** lv * leaf_block:
        raise ValueError("n_keys must equal branching**levels * leaf_block")
    Ds = [np.empty((B, H, branching ** l), dtype=np.float64) for l in range(1, lv + 1)]
    for bi in range(B):
        for h in range(H):
            k64 = widen(K[bi, h], dtype)
            for l in range(1, lv + 1):
                n_l = branching ** l
                M = N // n_l
                c = stored[l - 1][bi, h].astype(np.float64)          # [n_l, d]
                diff = k64.reshape(n_l, M, d) - c[:, None, :]
                Ds[l - 1][bi, h] = (diff * diff).sum(axis=2).max(axis=1)
    return {"D": Ds, "stored": [round_up_radius(x) for x in Ds]}


def query_norm(Q: np.ndarray, dtype: str) -> np.ndarray:
    """|q| in float64, [B, Hq]."""
    q = widen(Q, dtype)
    return np.sqrt((q * q).sum(axis=-1))


def threshold_route(Q: np.ndarray, dtype: str, stored: Sequence[np.ndarray],
                    radii: Sequence[np.ndarray], branching: int, tau: np.ndarray,
                    max_nodes: int) -> Dict[str, np.ndarray]:
    """Level-by-level pruning with the sphere bound.

    Q [B, Hq, d]; tau [B, Hq] (float32 values, widened); stored / radii as
    from tis_oracle.tree_build / node_radii.  Returns
      indices int32 [B, Hq, max_nodes]: surviving leaves ascending, -1 padded
              (all -1 on overflow);
      counts  int32 [B, Hq]: number of surviving leaves, -1 on overflow;
      margin  float64 [B, Hq]: smallest |bound - tau| / max(|bound|, |tau|, 1)
              over every node whose bound was evaluated (how close a decision
              came to flipping; +inf for an infinite tau);
      scored  int64 [B, Hq]: bounds evaluated."""
    B, Hq, d = Q.shape
    lv = len(stored)
    Hkv = stored[0].shape[1]
    G = Hq // Hkv
    if max_nodes < 1:
        raise ValueError("max_nodes must be >= 1")
    q64 = widen(Q, dtype)
    qn = query_norm(Q, dtype)
    tau64 = np.asarray(tau, dtype=np.float32).astype(np.float64)
    indices = np.full((B, Hq, max_nodes), -1, dtype=np.int32)
    counts = np.zeros((B, Hq), dtype=np.int32)
    margin = np.full((B, Hq), np.inf)
    scored = np.zeros((B, Hq), dtype=np.int64)
    children = np.arange(branching, dtype=np.int64)
    for bi in range(B):
        for hq in range(Hq):
            hk = hq // G
            t = tau64[bi, hq]
            kept = np.zeros(1, dtype=np.int64)      # the root
            overflow = False
            for l in range(1, lv + 1):
                cand = (kept[:, None] * branching + children[None, :]).ravel()
                c = stored[l - 1][bi, hk][cand].astype(np.float64)
                r = radii[l - 1][bi, hk][cand].astype(np.float64)
                bound = c @ q64[bi, hq] + qn[bi, hq] * r
                scored[bi, hq] += len(cand)
                den = np.maximum(np.maximum(np.abs(bound), abs(t)), 1.0)
                if len(cand) and np.isfinite(t):
                    margin[bi, hq] = min(margin[bi, hq], float(np.min(np.abs(bound - t) / den)))
                kept = np.sort(cand[bound >= t])
                if len(kept) > max_nodes:
                    overflow = True
                    break
            if overflow:
                counts[bi, hq] = -1
            else:
                counts[bi, hq] = len(kept)
                indices[bi, hq, :len(kept)] = kept
    return {"indices": indices, "counts": counts, "margin": margin, "scored": scored}


def threshold_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str,
                     indices: np.ndarray, counts: np.ndarray, leaf_block: int,
                     tau: np.ndarray, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Softmax over the keys of the listed leaves whose float64 score reaches
    tau.  Returns {"out": float64 [B, Hq, d], "margin": smallest
    |q.k - tau| / max(|q.k|, |tau|, 1) over the keys of the listed leaves,
    "selected": number of keys attended}."""
    B, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q64 = widen(Q, dtype)
    tau64 = np.asarray(tau, dtype=np.float32).astype(np.float64)
    out = np.zeros((B, Hq, d))
    margin = np.full((B, Hq), np.inf)
    selected = np.zeros((B, Hq), dtype=np.int64)
    for bi in range(B):
        for hq in range(Hq):
            if counts[bi, hq] < 0:
                out[bi, hq] = np.nan
                continue
            leaves = np.asarray(indices[bi, hq, :counts[bi, hq]], dtype=np.int64)
            if leaves.size == 0:
                continue
            rows = (leaves[:, None] * leaf_block + np.arange(leaf_block)[None, :]).ravel()
            k = widen(K[bi, hq // G, rows], dtype)
            s = k @ q64[bi, hq]
            t = tau64[bi, hq]
            if np.isfinite(t):
                den = np.maximum(np.maximum(np.abs(s), abs(t)), 1.0)
                margin[bi, hq] = float(np.min(np.abs(s - t) / den))
            sel = s >= t
            selected[bi, hq] = int(sel.sum())
            if not sel.any():
                continue
            v = widen(V[bi, hq // G, rows[sel]], dtype)
            x = scale * s[sel]
            p = np.exp(x - x.max())
            out[bi, hq] = (p @ v) / p.sum()
    return {"out": out, "margin": margin, "selected": selected}


def halfspace_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str, tau: np.ndarray,
                     scale: Optional[float] = None) -> np.ndarray:
    """Dense reference: softmax over every key of the cache with q.k >= tau
    (zero row when there is none), float64 [B, Hq, d]."""
    B, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q64 = widen(Q, dtype)
    tau64 = np.asarray(tau, dtype=np.float32).astype(np.float64)
    out = np.zeros((B, Hq, d))
    for bi in range(B):
        for hq in range(Hq):
            k = widen(K[bi, hq // G], dtype)
            s = k @ q64[bi, hq]
            sel = s >= tau64[bi, hq]
            if not sel.any():
                continue
            v = widen(V[bi, hq // G][sel], dtype)
            x = scale * s[sel]
            p = np.exp(x - x.max())
            out[bi, hq] = (p @ v) / p.sum()
    return out
