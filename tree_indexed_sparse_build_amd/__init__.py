"""Tree-indexed sparse attention decode on AMD Instinct MI355X (gfx950).

A tree of mean key summaries is built over each KV head's cache; each decode
query walks it top-down keeping a fixed beam of nodes per level, then runs
exact softmax attention over the keys of its selected leaf blocks
("Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
Abstract).  The three calls run as hand-written HIP kernels in libtis.so.
"""
from .ops import (Tree, tree_build, tree_route, tree_attend, tree_attend_grouped,  # noqa: F401
                  tree_decode, decode,
                  tree_decode_noalloc, version, from_storage, DecodePlan, CacheTree, tree_radii, radii_level,
                  tree_route_threshold, tree_decode_threshold)
from ._lib import TisError, TIS_MAX_SURVIVORS, TIS_NOALLOC_SCRATCH_BYTES  # noqa: F401
