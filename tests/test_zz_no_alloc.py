"""tis_tree_decode_noalloc (the decode for callers that cannot allocate)
against tis_tree_decode, through the C-ABI.

Both entry points run the same kernels with the same split of each query;
only where the split partial states live differs (the caller's workspace, or
the library's per-GPU scratch).  So the kept leaves and the outputs must be
equal bit for bit, and both must meet the oracle's bar (indices exact away
from near ties, max-abs 2e-2 for bf16 inputs).  Two calls run in a row, the
second on a smaller input, so the second finds the first's partial states
in the scratch; a third call needs no scratch at all.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from oracle import tis_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[no-alloc]", *a, flush=True)


@pytest.fixture(scope="module")
def tis():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_indexed_sparse_build_amd as t
    t.version()  # raises if libtis.so is missing
    return t


def _w(name, b, L, lv, W, B, Hkv, G, seed):
    return workloads.Workload(name, "bf16", B, Hkv * G, Hkv, 128, b, L, lv, W, "normal",
                              seed=seed)


# (workload, whether its queries are split, so that the scratch is used)
CALLS = [
    (_w("noalloc_split_big", 4, 64, 4, 64, B=2, Hkv=2, G=3, seed=41), True),    # 12 queries
    (_w("noalloc_split_small", 4, 64, 3, 64, B=1, Hkv=1, G=2, seed=42), True),  # 2 queries
    (_w("noalloc_unsplit", 8, 64, 2, 4, B=2, Hkv=2, G=4, seed=43), False),
]


def test_noalloc_decode_matches_workspace_decode(tis):
    lib = tis.ops.lib()
    for w, split in CALLS:
        wsb = lib.tis_decode_workspace_bytes(w.batch, w.q_heads, w.head_dim, w.beam,
                                             w.leaf_block)
        assert (wsb > 0) == split and wsb <= tis.TIS_NOALLOC_SCRATCH_BYTES, (w.name, wsb)
        x = workloads.generate(w)
        Q, K, V = (tis.from_storage(x[k], w.dtype, "cuda") for k in ("Q", "K", "V"))
        tree = tis.tree_build(K, w.branching, w.leaf_block, w.levels)
        _say(f"{w.name}: {w.queries} queries, {w.beam * w.leaf_block} keys each, "
             f"workspace of tis_tree_decode {wsb} bytes")
        o_ref, i_ref = tis.tree_decode(Q, K, V, tree, w.beam, return_indices=True)
        out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), device="cuda")
        idx = torch.full((w.batch, w.q_heads, w.beam), -7, dtype=torch.int32, device="cuda")
        tis.tree_decode_noalloc(Q, K, V, tree, w.beam, out=out, indices=idx)
        torch.cuda.synchronize()
        assert torch.equal(idx, i_ref), f"{w.name}: other leaves than tis_tree_decode"
        assert torch.equal(out.view(torch.int32), o_ref.view(torch.int32)), \
            f"{w.name}: output differs from tis_tree_decode"
        ob = O.tree_build(x["K"], w.dtype, w.branching, w.leaf_block, w.levels)
        orr = O.tree_route(x["Q"], w.dtype, ob["stored"], w.branching, w.beam)
        gi = idx.cpu().numpy()
        exact, tie, nq = parity.compare_indices(gi, orr, max_excused=0)
        want = O.tree_attend(x["Q"], x["K"], x["V"], w.dtype, gi, w.leaf_block)
        err = parity.compare_outputs(out.cpu().numpy(), want, w.dtype)
        _say(f"{w.name}: bit-equal to tis_tree_decode; indices exact {exact}/{nq}; "
             f"max-abs {err:.2e} against the oracle")
