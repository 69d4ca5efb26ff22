"""Seeded synthetic inputs for tree-indexed sparse attention decode.

This module is shared by the CPU oracle tests and the GPU path. It only draws
random numbers and rounds them to the storage dtype; it holds none of the
method's arithmetic (no summaries, scores, selection or softmax).

The five workloads stand in for the page workloads:
  * "alhr_1k"      -- the 1,024-token test of the ALHR post (Vdev-Ctrl Releases
                      ALHR, "Technical Breakthrough and Core Features"):
                      one fp32 head, binary tree, 64 leaves of 16 keys.
  * "gqa_32k"      -- a ~40k-token decode like the contexts of the Louver
                      explainer (Sparse Attention as a Range Searching Problem,
                      "Experimentele Resultaten"), as a clustered GQA cache.
  * "gqa_256k"     -- long-context decode toward the >1M-token regime of the ZHA
                      abstract (Subquadratic Attention with a Hierarchical
                      Tree-Structured Indexer, Abstract).
  * "long_1m"      -- 1,048,576 keys per KV head, build then one decode step
                      (same abstract: contexts beyond one million tokens).
  * "deep_planted" -- a six-level tree (same abstract: trees up to 6 levels)
                      with one planted key block per query, a synthetic
                      retrieval check.

Storage: fp32 inputs are float32 arrays; bf16 inputs are uint16 arrays holding
bf16 bit patterns produced by round-to-nearest-even from float32.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "generate", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "small"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    branching: int
    leaf_block: int
    levels: int
    beam: int
    generator: str        # "normal", "mixture", "planted"
    clusters: int = 0     # mixture only
    seed: int = 0

    @property
    def n_keys(self) -> int:
        return self.branching ** self.levels * self.leaf_block

    @property
    def n_leaves(self) -> int:
        return self.branching ** self.levels

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def queries(self) -> int:
        return self.batch * self.q_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "alhr_1k": Workload("alhr_1k", "f32", 1, 64, 1, 64, 2, 16, 6, 2, "normal", seed=1),
    "gqa_32k": Workload("gqa_32k", "bf16", 4, 32, 8, 128, 8, 64, 3, 8, "mixture",
                        clusters=256, seed=2),
    "gqa_256k": Workload("gqa_256k", "bf16", 2, 32, 8, 128, 8, 64, 4, 16, "mixture",
                         clusters=1024, seed=3),
    "long_1m": Workload("long_1m", "bf16", 1, 32, 8, 128, 8, 32, 5, 16, "mixture",
                        clusters=4096, seed=4),
    "deep_planted": Workload("deep_planted", "bf16", 1, 128, 8, 128, 4, 64, 6, 8,
                             "planted", seed=5),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def small(name: str, levels: Optional[int] = None, batch: int = 1,
          kv_heads: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """A reduced copy of a workload (fewer levels / heads) with the same
    generator, for parity cases the oracle finishes in seconds."""
    w = WORKLOADS[name]
    lv = w.levels if levels is None else levels
    kvh = w.kv_heads if kv_heads is None else kv_heads
    qh = kvh * w.group
    beam = min(w.beam, w.branching ** lv)
    clusters = w.clusters
    if w.generator == "mixture":
        # keep the keys-per-cluster of the full workload
        keys_per_cluster = w.n_keys // w.clusters
        clusters = max(1, (w.branching ** lv * w.leaf_block) // keys_per_cluster)
    return dataclasses.replace(w, name=f"{name}_lv{lv}", levels=lv, batch=batch,
                               kv_heads=kvh, q_heads=qh, beam=beam,
                               clusters=clusters,
                               seed=w.seed if seed is None else seed)


# ----------------------------------------------------------------------------
# bf16 storage helpers (data preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.
    Inputs are finite by construction."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(w: Workload, stream: int, extra: int = 0) -> np.random.Generator:
    names = list(WORKLOADS)
    wid = names.index(w.name) if w.name in WORKLOADS else 1000 + len(w.name)
    return np.random.default_rng(np.random.SeedSequence([w.seed, wid, stream, extra]))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x)


def _head(w: Workload, b: int, h: int):
    """Keys, values (storage dtype), queries (float32) and planted blocks of
    the G query heads of (batch b, KV head h): one head's own random streams,
    so heads can be drawn in any order or in parallel with the same result."""
    N, d, G = w.n_keys, w.head_dim, w.group
    planted = np.full(G, -1, dtype=np.int64)
    rk = _rng(w, 1, b * w.kv_heads + h)
    rv = _rng(w, 2, b * w.kv_heads + h)
    rq = _rng(w, 3, b * w.kv_heads + h)
    if w.generator == "normal":
        k = rk.standard_normal((N, d), dtype=np.float32)
        q = rq.standard_normal((G, d), dtype=np.float32)
    elif w.generator == "mixture":
        C = w.clusters
        assert N % C == 0, "mixture needs equal contiguous segments"
        seg = N // C
        mu = rk.standard_normal((C, d), dtype=np.float32)
        k = rk.standard_normal((N, d), dtype=np.float32)
        k *= np.float32(0.3)
        k += np.repeat(mu, seg, axis=0)
        cq = rq.integers(0, C, size=G)
        q = mu[cq] + np.float32(0.3) * rq.standard_normal((G, d), dtype=np.float32)
    elif w.generator == "planted":
        k = rk.standard_normal((N, d), dtype=np.float32)
        q = rq.standard_normal((G, d), dtype=np.float32)
        rp = _rng(w, 4, b * w.kv_heads + h)
        L = w.leaf_block
        blocks = rp.choice(N // L, size=G, replace=False)
        for g in range(G):
            qh = q[g].astype(np.float64)
            qh /= np.linalg.norm(qh)
            c = rp.uniform(0.9, 1.0, size=L)
            u = rp.standard_normal((L, d))
            u -= np.outer(u @ qh, qh)
            u /= np.linalg.norm(u, axis=1, keepdims=True)
            kk = np.sqrt(d) * (c[:, None] * qh[None, :]
                               + np.sqrt(1.0 - c * c)[:, None] * u)
            k[blocks[g] * L:(blocks[g] + 1) * L] = kk.astype(np.float32)
            planted[g] = blocks[g]
    else:
        raise ValueError(w.generator)
    ks = _store(k, w.dtype)
    del k
    vs = _store(rv.standard_normal((N, d), dtype=np.float32), w.dtype)
    return ks, vs, q, planted


def generate(w: Workload, workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Return {"K","V": [B,Hkv,N,d], "Q": [B,Hq,d]} in the storage dtype, plus
    "planted": int64 [B,Hq] planted leaf block per query (-1 if none).

    Recipes:
      normal  : K, V, Q ~ N(0, 1) i.i.d.
      mixture : per (batch, KV head) `clusters` centres mu_c ~ N(0, I_d); the
                keys are laid out in equal contiguous segments, segment c drawn
                as mu_c + 0.3*eps; each query is mu_c + 0.3*eps for a cluster c
                drawn uniformly from its KV head's centres; V ~ N(0, 1).
      planted : K, V, Q ~ N(0, 1); for each query a distinct leaf block of its
                KV head is overwritten with keys sqrt(d)*(c*qhat + sqrt(1-c^2)*u),
                c ~ U[0.9, 1], u a random unit vector orthogonal to qhat, so
                every planted key has cosine >= 0.9 with its query.

    Every (batch, KV head) draws from its own seeded streams, so the heads
    are generated by `workers` threads (default: up to 8) with the same
    result as one at a time.
    """
    B, Hq, Hkv, d, N = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.n_keys
    G = w.group
    K = np.empty((B, Hkv, N, d), dtype=np.float32 if w.dtype == "f32" else np.uint16)
    V = np.empty_like(K)
    Qf = np.empty((B, Hq, d), dtype=np.float32)
    planted = np.full((B, Hq), -1, dtype=np.int64)

    def one(bh):
        b, h = bh
        ks, vs, q, pl = _head(w, b, h)
        K[b, h] = ks
        V[b, h] = vs
        Qf[b, h * G:(h + 1) * G] = q
        planted[b, h * G:(h + 1) * G] = pl

    heads = [(b, h) for b in range(B) for h in range(Hkv)]
    if workers is None:
        workers = min(8, os.cpu_count() or 1)
    if workers <= 1 or len(heads) == 1:
        for bh in heads:
            one(bh)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(workers, len(heads))) as ex:
            list(ex.map(one, heads))
    Q = _store(Qf, w.dtype)
    return {"K": K, "V": V, "Q": Q, "planted": planted}
