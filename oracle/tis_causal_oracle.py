"""CPU oracle for causal prefill routing over the summary tree (fp64 numpy).

TEST INFRASTRUCTURE ONLY, like tis_oracle: the slow, plain reference the GPU
path is checked against.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; it shares no code with the HIP
library or its Python binding.

What is computed, and where it comes from
-----------------------------------------
"Vdev-Ctrl Releases ALHR" (Summary; Technical Breakthrough and Core
Features): in a 1,024-token test a query reads about 30 keys on average where
dense attention reads 512 -- 512 being the average causal prefix of 1,024
positions, so every position is a query over the keys up to it.  "Subquadratic
Attention with a Hierarchical Tree-Structured Indexer" (Abstract): the tree
over the KV cache grows deeper as the context grows.  Reading: the query at
position t routes over the tree of the first t + 1 keys, exactly as defined
for a growing cache (tis_grow_oracle: depth, nodes cut at t + 1, exact means
rounded once, candidates only among existing children), and attends over the
keys of its kept leaf blocks cut at t + 1 (so never past itself).  Each
position is therefore the growing-cache decode step at n = t + 1, and this
module is that step run for every position.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from oracle import tis_grow_oracle as GO

__all__ = ["causal_prefill", "keys_read"]


def keys_read(indices: np.ndarray, n_keys: int, leaf_block: int) -> int:
    """Keys a query reads: the sizes of its kept leaf blocks cut at n_keys."""
    sel = np.unique(np.asarray(indices)[np.asarray(indices) >= 0])
    return int(sum(min(leaf_block, n_keys - j * leaf_block) for j in sel))


def causal_prefill(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dtype: str, branching: int,
                   leaf_block: int, beam: int, summary_dtype: str = "f32",
                   scale: Optional[float] = None,
                   positions: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Q: [B, Hq, N, d], one query per position; K, V: [B, Hkv, N, d].

    Returns (for the positions asked, all by default)
      indices   int32 [B, Hq, P, beam]: kept leaves ascending, -1 padded
      out       float64 [B, Hq, P, d]
      keys_read int64 [B, Hq, P]
      gap       float64 [B, Hq, P]: smallest relative cut gap over the levels
                (tis_oracle's tie measure; +inf where nothing was cut)
      positions int64 [P]."""
    B, Hq, N, d = Q.shape
    if K.shape[2] != N or V.shape != K.shape:
        raise ValueError("Q, K and V must cover the same positions")
    pos = np.arange(N) if positions is None else np.asarray(positions, dtype=np.int64)
    P = len(pos)
    indices = np.full((B, Hq, P, beam), -1, dtype=np.int32)
    out = np.zeros((B, Hq, P, d))
    nread = np.zeros((B, Hq, P), dtype=np.int64)
    gap = np.full((B, Hq, P), np.inf)
    for i, t in enumerate(pos):
        n = int(t) + 1
        ob = GO.grow_build(K, dtype, n, branching, leaf_block, summary_dtype=summary_dtype)
        q = np.ascontiguousarray(Q[:, :, t])
        r = GO.grow_route(q, dtype, ob["stored"], n, branching, leaf_block, beam)
        w = r["indices"].shape[-1]
        indices[:, :, i, :w] = r["indices"]
        out[:, :, i] = GO.grow_attend(q, K, V, dtype, r["indices"], n, leaf_block, scale)
        g = np.where(np.isfinite(r["gap"]), r["gap"], np.inf)
        gap[:, :, i] = g.min(axis=-1)
        for bi in range(B):
            for h in range(Hq):
                nread[bi, h, i] = keys_read(r["indices"][bi, h], n, leaf_block)
    return {"indices": indices, "out": out, "keys_read": nread, "gap": gap, "positions": pos}
