"""The C-ABI library: it loads, exports every entry point include/tis.h
declares, and its host-side checks reject bad arguments before anything is
enqueued.  No compute call is made: every call below fails a check first,
and the pointers passed are never dereferenced."""
import ctypes
import os
import re

import pytest

from tree_indexed_sparse_build_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tis.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tis_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"tis_tree_build", "tis_tree_route", "tis_tree_attend", "tis_tree_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_version(lib):
    assert lib.tis_version().decode().startswith("tis ")


def test_summary_bytes_by_type(lib):
    assert lib.tis_tree_summary_bytes_as(4, 8, 128, 8, 3, _lib.TIS_F32) == 4 * 128 * 32 * 584
    assert lib.tis_tree_summary_bytes_as(4, 8, 128, 8, 3, _lib.TIS_BF16) == 2 * 128 * 32 * 584
    # fp8: a byte an element (16-byte aligned), then a float32 scale a node
    nodes = 32 * 584
    assert lib.tis_tree_summary_bytes_as(4, 8, 128, 8, 3, _lib.TIS_FP8_E4M3) == (
        -(-nodes * 128 // 16) * 16 + 4 * nodes)
    assert lib.tis_tree_summary_bytes_as(4, 8, 128, 8, 3, 3) == 0
    # growing caches take float32 or bfloat16 summaries only
    assert lib.tis_cache_tree_summary_bytes_as(4, 8, 128, 8, 64, 40000, _lib.TIS_FP8_E4M3) == 0
    assert lib.tis_cache_tree_summary_bytes_as(4, 8, 128, 8, 64, 40000, _lib.TIS_BF16) == (
        2 * 128 * 32 * (625 + 79 + 10 + 2))
    assert lib.tis_cache_tree_summary_bytes_as(4, 8, 128, 8, 64, 40000, 9) == 0


def test_summary_bytes(lib):
    # 4 * d * B * Hkv * (8 + 64 + 512) for the 32K-key GQA workload
    assert lib.tis_tree_summary_bytes(4, 8, 128, 8, 3) == 4 * 128 * 32 * 584
    assert lib.tis_tree_summary_bytes(1, 1, 64, 2, 6) == 4 * 64 * 126
    assert lib.tis_tree_summary_bytes(1, 1, 64, 1, 6) == 0
    assert lib.tis_tree_summary_bytes(1, 1, 64, 2, 0) == 0
    assert lib.tis_tree_summary_bytes(1, 1, 64, 2, 17) == 0


def test_workspace_bytes(lib):
    # the build keeps fp64 sums of levels 2..r, r = the level of its chunk roots
    # 32K keys, 4 x 8 heads: chunks are level-1 nodes (8 leaves per wave, 8 waves)
    assert lib.tis_build_workspace_bytes(4, 8, 32768, 128, 8, 64, 3) == 0
    # 256K keys, 2 x 8 heads: chunks at level 2 (16 KiB of arrival counters
    # come first)
    assert lib.tis_build_workspace_bytes(2, 8, 262144, 128, 8, 64, 4) == 16384 + 16 * 64 * 128 * 8
    # 1M keys, 8 heads: chunks at level 3 (8 leaves per wave, 8 waves per workgroup:
    # the deepest plan whose wave-level rows fit the LDS staging), sums of levels 2, 3
    assert lib.tis_build_workspace_bytes(1, 8, 1 << 20, 128, 8, 32, 5) == 16384 + 8 * (64 + 512) * 128 * 8
    # a single-level tree needs none
    assert lib.tis_build_workspace_bytes(1, 1, 64, 128, 16, 4, 1) == 0
    # invalid geometry -> 0
    assert lib.tis_build_workspace_bytes(4, 8, 1000, 128, 8, 64, 3) == 0
    # attend and decode: 128 queries run one workgroup each, no workspace
    assert lib.tis_attend_workspace_bytes(4, 32, 128, 8, 64) == 0
    assert lib.tis_decode_workspace_bytes(4, 32, 128, 8, 64) == 0
    # 32 queries with 512 keys each: 8 workgroups per query
    assert lib.tis_attend_workspace_bytes(1, 32, 128, 16, 32) == 1024 + 32 * 8 * (128 + 4) * 4
    # 32 queries with 256 keys each: one workgroup per query
    assert lib.tis_attend_workspace_bytes(1, 32, 128, 8, 32) == 0
    # 32 queries with 64 x 64 keys each: 8 workgroups per query keep partial
    # states after the 1 KiB of arrival counters
    assert lib.tis_attend_workspace_bytes(1, 32, 128, 64, 64) == 1024 + 32 * 8 * (128 + 4) * 4
    assert lib.tis_decode_workspace_bytes(1, 32, 128, 64, 64) == 1024 + 32 * 8 * (128 + 4) * 4
    # a short key set is never split
    assert lib.tis_attend_workspace_bytes(1, 4, 64, 2, 16) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: each call fails a check first


@pytest.fixture(autouse=True)
def _no_device_visible():
    # Every call below must fail a host check; on a machine with a GPU a
    # mistake here would launch on fake pointers, so these run without one.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-check tests run where no GPU is visible")


def _tree(summ=FAKE, b=2, L=16, lv=3, d=64, B=1, H=1, sd=_lib.TIS_F32):
    return _lib.TisTree(B, H, b ** lv * L, d, b, L, lv, sd, summ)


def _build(lib, **kw):
    # b=2, lv=6: the build needs a workspace (two kernels), so ws / wsb are checked
    a = dict(K=FAKE, dt=_lib.TIS_BF16, B=1, H=1, N=1024, d=64, b=2, L=16, lv=6,
             tree=_lib.TisTree(0, 0, 0, 0, 0, 0, 0, 0, FAKE), ws=FAKE, wsb=0)
    a.update(kw)
    return lib.tis_tree_build(a["K"], a["dt"], a["B"], a["H"], a["N"], a["d"], a["b"], a["L"],
                              a["lv"], ctypes.byref(a["tree"]), a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), _lib.TIS_E_NULL),
    (dict(ws=None), _lib.TIS_E_NULL),
    (dict(tree=_lib.TisTree(0, 0, 0, 0, 0, 0, 0, 0, None)), _lib.TIS_E_NULL),
    (dict(dt=7), _lib.TIS_E_DTYPE),
    (dict(tree=_lib.TisTree(0, 0, 0, 0, 0, 0, 0, 3, FAKE)), _lib.TIS_E_DTYPE),
    (dict(N=96), _lib.TIS_E_SHAPE),
    (dict(b=1), _lib.TIS_E_SHAPE),
    (dict(b=65, N=65 ** 3 * 16, lv=3), _lib.TIS_E_UNSUPPORTED),
    (dict(lv=0), _lib.TIS_E_SHAPE),
    (dict(lv=17), _lib.TIS_E_UNSUPPORTED),
    (dict(L=0), _lib.TIS_E_SHAPE),
    (dict(d=96), _lib.TIS_E_UNSUPPORTED),
    (dict(d=0), _lib.TIS_E_SHAPE),
    (dict(B=0), _lib.TIS_E_SHAPE),
    (dict(K=FAKE + 2, wsb=1 << 20), _lib.TIS_E_ALIGN),
    (dict(ws=FAKE + 8, wsb=1 << 20), _lib.TIS_E_ALIGN),
    (dict(wsb=255), _lib.TIS_E_WORKSPACE),
    (dict(wsb=1 << 20, d=96), _lib.TIS_E_UNSUPPORTED),
])
def test_build_rejects(lib, kw, status):
    assert _build(lib, **kw) == status
    assert lib.tis_last_error().decode()


def test_build_rejects_overflowing_geometry(lib):
    assert _build(lib, b=64, lv=16, N=0) == _lib.TIS_E_SHAPE


def _route(lib, Q=FAKE, dt=_lib.TIS_F32, Hq=2, tree=None, beam=2, idx=FAKE, trace=None):
    t = tree if tree is not None else _tree(H=1)
    return lib.tis_tree_route(Q, dt, Hq, ctypes.byref(t), beam, idx, trace, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), _lib.TIS_E_NULL),
    (dict(idx=None), _lib.TIS_E_NULL),
    (dict(tree=_tree(summ=None)), _lib.TIS_E_NULL),
    (dict(dt=3), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(H=2), Hq=3), _lib.TIS_E_SHAPE),
    (dict(Hq=0), _lib.TIS_E_SHAPE),
    (dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(beam=9), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(b=64, lv=2, L=1), beam=5), _lib.TIS_E_UNSUPPORTED),
    (dict(tree=_lib.TisTree(1, 1, 100, 64, 2, 16, 3, 0, FAKE)), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(sd=-1)), _lib.TIS_E_DTYPE),
    (dict(Q=FAKE + 4), _lib.TIS_E_ALIGN),
    (dict(idx=FAKE + 2), _lib.TIS_E_ALIGN),
    (dict(trace=FAKE + 1), _lib.TIS_E_ALIGN),
])
def test_route_rejects(lib, kw, status):
    assert _route(lib, **kw) == status
    assert lib.tis_last_error().decode()


def _attend(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, B=1, Hq=4, Hkv=2, N=256, d=128, L=16,
             idx=FAKE, beam=4, scale=0.0, O=FAKE, ws=FAKE, wsb=0)
    a.update(kw)
    return lib.tis_tree_attend(a["Q"], a["K"], a["V"], a["dt"], a["B"], a["Hq"], a["Hkv"], a["N"],
                               a["d"], a["L"], a["idx"], a["beam"], a["scale"], a["O"], a["ws"],
                               a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(V=None), _lib.TIS_E_NULL),
    (dict(O=None), _lib.TIS_E_NULL),
    (dict(dt=-1), _lib.TIS_E_DTYPE),
    (dict(Hq=3), _lib.TIS_E_SHAPE),
    (dict(N=250), _lib.TIS_E_SHAPE),
    (dict(L=0), _lib.TIS_E_SHAPE),
    (dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(beam=257), _lib.TIS_E_UNSUPPORTED),
    (dict(d=32), _lib.TIS_E_UNSUPPORTED),
    (dict(scale=float("nan")), _lib.TIS_E_SHAPE),
    (dict(scale=float("inf")), _lib.TIS_E_SHAPE),
    (dict(K=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(O=FAKE + 4), _lib.TIS_E_ALIGN),
    (dict(idx=FAKE + 2), _lib.TIS_E_ALIGN),
    # 4 queries with 64 x 64 keys each: split, so a workspace is needed
    (dict(B=1, Hq=4, Hkv=2, N=4096, L=64, beam=64, ws=None), _lib.TIS_E_NULL),
    (dict(B=1, Hq=4, Hkv=2, N=4096, L=64, beam=64, ws=FAKE, wsb=100), _lib.TIS_E_WORKSPACE),
])
def test_attend_rejects(lib, kw, status):
    assert _attend(lib, **kw) == status
    assert lib.tis_last_error().decode()


def _attend_grouped(lib, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, B=1, Hq=4, Hkv=2, N=256, d=128, L=16,
             idx=FAKE, beam=4, scale=0.0, O=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib.tis_tree_attend_grouped(a["Q"], a["K"], a["V"], a["dt"], a["B"], a["Hq"], a["Hkv"],
                                       a["N"], a["d"], a["L"], a["idx"], a["beam"], a["scale"],
                                       a["O"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(V=None), _lib.TIS_E_NULL),
    (dict(idx=None), _lib.TIS_E_NULL),
    (dict(dt=-1), _lib.TIS_E_DTYPE),
    (dict(Hq=3), _lib.TIS_E_SHAPE),
    (dict(N=250), _lib.TIS_E_SHAPE),
    (dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(d=32), _lib.TIS_E_UNSUPPORTED),
    (dict(scale=float("nan")), _lib.TIS_E_SHAPE),
    (dict(K=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(idx=FAKE + 2), _lib.TIS_E_ALIGN),
    # 65 query heads per KV head, or 576 slots in a group
    (dict(Hq=130, Hkv=2), _lib.TIS_E_UNSUPPORTED),
    (dict(Hq=64, Hkv=1, beam=9), _lib.TIS_E_UNSUPPORTED),
    # 2 groups: split, so a workspace is needed
    (dict(ws=None), _lib.TIS_E_NULL),
    (dict(wsb=100), _lib.TIS_E_WORKSPACE),
    (dict(ws=FAKE + 8), _lib.TIS_E_ALIGN),
])
def test_attend_grouped_rejects(lib, kw, status):
    assert _attend_grouped(lib, **kw) == status
    assert lib.tis_last_error().decode()


def test_attend_grouped_workspace_bytes(lib):
    part = (128 + 4) * 4
    # 32 groups of 4 heads, beam 8: 8 parts per group
    assert lib.tis_attend_grouped_workspace_bytes(4, 32, 8, 128, 8) == 1024 + 32 * 8 * 4 * part
    # 8 groups of 16 heads: 16 parts (16 x 16 states for the last part to merge)
    assert lib.tis_attend_grouped_workspace_bytes(1, 128, 8, 128, 8) == 1024 + 8 * 16 * 16 * part
    # no more parts than the group has slots
    assert lib.tis_attend_grouped_workspace_bytes(1, 2, 2, 128, 1) == 0
    assert lib.tis_attend_grouped_workspace_bytes(1, 2, 1, 128, 1) == 1024 + 2 * 2 * part
    # 256 groups: one workgroup each, no workspace
    assert lib.tis_attend_grouped_workspace_bytes(64, 8, 4, 128, 2) == 0
    assert lib.tis_attend_grouped_workspace_bytes(1, 3, 2, 128, 8) == 0  # 3 heads over 2


def _decode(lib, Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, tree=None, beam=2, scale=0.0,
            O=FAKE, idx=None, ws=None, wsb=0):
    t = tree if tree is not None else _tree(H=1)
    return lib.tis_tree_decode(Q, K, V, dt, Hq, ctypes.byref(t), beam, scale, O, idx, ws, wsb,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), _lib.TIS_E_NULL),
    (dict(O=None), _lib.TIS_E_NULL),
    (dict(tree=_tree(summ=None)), _lib.TIS_E_NULL),
    (dict(dt=9), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(H=2), Hq=3), _lib.TIS_E_SHAPE),
    (dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(beam=9), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(b=64, lv=2, L=1), beam=5), _lib.TIS_E_UNSUPPORTED),
    (dict(scale=float("nan")), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(sd=5)), _lib.TIS_E_DTYPE),
    (dict(V=FAKE + 4), _lib.TIS_E_ALIGN),
    (dict(idx=FAKE + 2), _lib.TIS_E_ALIGN),
    # 2 queries, beam 64 over leaves of 64 keys: split, so a workspace is needed
    (dict(tree=_tree(b=4, lv=4, L=64, d=128), beam=64, Hq=2), _lib.TIS_E_NULL),
    (dict(tree=_tree(b=4, lv=4, L=64, d=128), beam=64, Hq=2, ws=FAKE, wsb=16), _lib.TIS_E_WORKSPACE),
    (dict(tree=_tree(b=4, lv=4, L=64, d=128), beam=64, Hq=2, ws=FAKE + 8, wsb=1 << 20),
     _lib.TIS_E_ALIGN),
])
def test_decode_rejects(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.tis_last_error().decode()


def _decode_timeline(lib, Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, tree=None, beam=2,
                     scale=0.0, O=FAKE, ws=None, wsb=0, tl=FAKE, tlb=1 << 20):
    t = tree if tree is not None else _tree(H=1)
    return lib.tis_probe_decode_timeline(Q, K, V, dt, Hq, ctypes.byref(t), beam, scale, O, ws,
                                         wsb, tl, tlb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(tl=None), _lib.TIS_E_NULL),
    (dict(K=None), _lib.TIS_E_NULL),
    (dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(tl=FAKE + 4), _lib.TIS_E_ALIGN),
    (dict(tlb=2 * 16 * 24 * 8 - 8), _lib.TIS_E_WORKSPACE),
    (dict(tree=_tree(H=1, sd=_lib.TIS_FP8_E4M3)), _lib.TIS_E_UNSUPPORTED),
    # a split decode still needs its workspace
    (dict(tree=_tree(b=4, lv=4, L=64, d=128), beam=64, Hq=2), _lib.TIS_E_NULL),
])
def test_decode_timeline_rejects(lib, kw, status):
    assert _decode_timeline(lib, **kw) == status
    assert lib.tis_last_error().decode()


def test_decode_timeline_bytes(lib):
    # one record of 24 eight-byte slots per wave, 16 waves per workgroup
    assert lib.tis_probe_decode_timeline_bytes(1, 2, 2, 16) == 2 * 16 * 24 * 8
    # 2 queries with beam 64 over 64-key leaves split into 64 parts each
    assert lib.tis_probe_decode_timeline_bytes(1, 2, 64, 64) == 2 * 64 * 16 * 24 * 8
    assert lib.tis_probe_decode_timeline_bytes(4, 32, 8, 64) == 128 * 16 * 24 * 8
    assert lib.tis_probe_decode_timeline_bytes(0, 2, 2, 16) == 0
    assert lib.tis_probe_decode_timeline_bytes(1, 2, 0, 16) == 0


def _decode_noalloc(lib, Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, tree=None, beam=2,
                    scale=0.0, O=FAKE, idx=None):
    t = tree if tree is not None else _tree(H=1)
    return lib.tis_tree_decode_noalloc(Q, K, V, dt, Hq, ctypes.byref(t), beam, scale, O, idx,
                                       None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), _lib.TIS_E_NULL),
    (dict(O=None), _lib.TIS_E_NULL),
    (dict(tree=_tree(summ=None)), _lib.TIS_E_NULL),
    (dict(dt=9), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(H=2), Hq=3), _lib.TIS_E_SHAPE),
    (dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(beam=9), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(b=64, lv=2, L=1), beam=5), _lib.TIS_E_UNSUPPORTED),
    (dict(scale=float("inf")), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(sd=5)), _lib.TIS_E_DTYPE),
    (dict(Q=FAKE + 4), _lib.TIS_E_ALIGN),
    (dict(idx=FAKE + 2), _lib.TIS_E_ALIGN),
])
def test_decode_noalloc_rejects(lib, kw, status):
    """The same host checks as tis_tree_decode, before anything is looked up
    or enqueued."""
    assert _decode_noalloc(lib, **kw) == status
    assert lib.tis_last_error().decode()


def test_noalloc_scratch_covers_every_split_geometry(lib):
    """The split rule gives a query at most 256 / queries parts and splits
    only below 128 queries, so the largest workspace any geometry asks for
    fits the library's scratch (no valid decode is turned away)."""
    worst = 0
    for queries in range(1, 129):
        for beam in (16, 64, 256):
            for d in (64, 128):
                worst = max(worst, lib.tis_decode_workspace_bytes(1, queries, d, beam, 4096))
    assert 0 < worst <= _lib.TIS_NOALLOC_SCRATCH_BYTES


# ------------------------------------------------------- growing cache --

def test_cache_tree_bytes(lib):
    # capacity 40000, b 8, L 64: heights 0..3 (8^4 * 64 >= 40000), rows
    # ceil(40000 / 64) = 625, 79, 10, 2 per head
    heads, d = 4 * 8, 128
    assert lib.tis_cache_tree_summary_bytes(4, 8, d, 8, 64, 40000) == 4 * d * heads * (625 + 79 + 10 + 2)
    # two halves of fp64 open-node sums, one row per height, then a row per
    # chunk for long appends (chunks of 512 keys: ceil(40000 / 512) = 79)
    assert lib.tis_cache_tree_state_bytes(4, 8, d, 8, 64, 40000) == 8 * d * heads * (2 * 4 + 79)
    # a cache of one leaf: one height with one row
    assert lib.tis_cache_tree_summary_bytes(1, 1, 64, 2, 16, 10) == 4 * 64
    assert lib.tis_cache_tree_state_bytes(1, 1, 64, 2, 16, 10) == (2 + 1) * 8 * 64
    # invalid geometry -> 0
    assert lib.tis_cache_tree_summary_bytes(1, 1, 64, 1, 16, 100) == 0
    assert lib.tis_cache_tree_summary_bytes(1, 1, 96, 2, 16, 100) == 0
    assert lib.tis_cache_tree_state_bytes(1, 1, 64, 2, 16, 0) == 0
    # a full cache deeper than 16 levels
    assert lib.tis_cache_tree_state_bytes(1, 1, 64, 2, 1, 1 << 20) == 0


def _ctree(summ=FAKE, state=FAKE, B=1, H=1, d=64, b=2, L=16, C=1000, n=0, lv=0,
           sd=_lib.TIS_F32, half=0):
    return _lib.TisCacheTree(batch=B, kv_heads=H, head_dim=d, branching=b, leaf_block=L,
                             capacity=C, n_keys=n, levels=lv, summary_dtype=sd, state_half=half,
                             summaries=summ, state=state)


@pytest.mark.parametrize("kw,status", [
    (dict(summ=None), _lib.TIS_E_NULL),
    (dict(state=None), _lib.TIS_E_NULL),
    (dict(b=1), _lib.TIS_E_SHAPE),
    (dict(d=32), _lib.TIS_E_UNSUPPORTED),
    (dict(C=0), _lib.TIS_E_SHAPE),
    (dict(state=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(sd=3), _lib.TIS_E_DTYPE),
    (dict(sd=_lib.TIS_FP8_E4M3), _lib.TIS_E_UNSUPPORTED),
])
def test_cache_reset_rejects(lib, kw, status):
    t = _ctree(**kw)
    assert lib.tis_cache_tree_reset(ctypes.byref(t), None) == status
    assert lib.tis_last_error().decode()


@pytest.mark.parametrize("tree_kw,call_kw,status", [
    (dict(), dict(K=None), _lib.TIS_E_NULL),
    (dict(summ=None), dict(), _lib.TIS_E_NULL),
    (dict(), dict(dt=5), _lib.TIS_E_DTYPE),
    (dict(), dict(n_new=-1), _lib.TIS_E_SHAPE),
    (dict(), dict(n_new=1001), _lib.TIS_E_SHAPE),
    (dict(n=990, lv=6), dict(n_new=11), _lib.TIS_E_SHAPE),   # past the capacity
    (dict(n=100, lv=2), dict(n_new=1), _lib.TIS_E_SHAPE),    # 100 keys need 3 levels
    (dict(n=-1), dict(n_new=1), _lib.TIS_E_SHAPE),
    (dict(), dict(K=FAKE + 4, n_new=1), _lib.TIS_E_ALIGN),
])
def test_cache_append_rejects(lib, tree_kw, call_kw, status):
    t = _ctree(**tree_kw)
    a = dict(K=FAKE, dt=_lib.TIS_BF16, n_new=1)
    a.update(call_kw)
    assert lib.tis_cache_tree_append(a["K"], a["dt"], a["n_new"], ctypes.byref(t), None) == status
    assert lib.tis_last_error().decode()
    assert t.n_keys == tree_kw.get("n", 0)  # a rejected append changes nothing


def test_cache_append_of_nothing_is_a_no_op(lib):
    t = _ctree(n=100, lv=3)
    assert lib.tis_cache_tree_append(FAKE, _lib.TIS_BF16, 0, ctypes.byref(t), None) == _lib.TIS_OK
    assert (t.n_keys, t.levels) == (100, 3)


@pytest.mark.parametrize("tree_kw,call_kw,status", [
    (dict(), dict(), _lib.TIS_E_SHAPE),                      # empty tree
    (dict(n=100, lv=3), dict(Q=None), _lib.TIS_E_NULL),
    (dict(n=100, lv=3), dict(idx=None), _lib.TIS_E_NULL),
    (dict(n=100, lv=3, state=None), dict(), _lib.TIS_E_NULL),
    (dict(n=100, lv=3), dict(dt=2), _lib.TIS_E_DTYPE),
    (dict(n=100, lv=4), dict(), _lib.TIS_E_SHAPE),           # levels do not match n_keys
    (dict(n=100, lv=3), dict(Hq=0), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3, H=2), dict(Hq=3), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3), dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3), dict(beam=129), _lib.TIS_E_UNSUPPORTED),
    (dict(n=100, lv=3), dict(Q=FAKE + 2), _lib.TIS_E_ALIGN),
    (dict(n=100, lv=3), dict(idx=FAKE + 2), _lib.TIS_E_ALIGN),
])
def test_cache_route_rejects(lib, tree_kw, call_kw, status):
    t = _ctree(**tree_kw)
    a = dict(Q=FAKE, dt=_lib.TIS_BF16, Hq=2, beam=4, idx=FAKE, trace=None)
    a.update(call_kw)
    assert lib.tis_cache_tree_route(a["Q"], a["dt"], a["Hq"], ctypes.byref(t), a["beam"], a["idx"],
                                    a["trace"], None) == status
    assert lib.tis_last_error().decode()


@pytest.mark.parametrize("tree_kw,call_kw,status", [
    (dict(), dict(), _lib.TIS_E_SHAPE),                      # empty tree
    (dict(n=100, lv=3), dict(V=None), _lib.TIS_E_NULL),
    (dict(n=100, lv=3), dict(O=None), _lib.TIS_E_NULL),
    (dict(n=100, lv=3), dict(scale=float("nan")), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3), dict(K=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(n=100, lv=3), dict(beam=200), _lib.TIS_E_UNSUPPORTED),
    # 2 queries, beam 64 over leaves of 128 keys: split, so a workspace is needed
    (dict(n=30000, lv=4, d=128, b=4, L=128, C=30000), dict(beam=64, Hq=2), _lib.TIS_E_NULL),
    (dict(n=30000, lv=4, d=128, b=4, L=128, C=30000), dict(beam=64, Hq=2, ws=FAKE, wsb=8),
     _lib.TIS_E_WORKSPACE),
])
def test_cache_decode_rejects(lib, tree_kw, call_kw, status):
    t = _ctree(**tree_kw)
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, beam=4, scale=0.0, O=FAKE, idx=None,
             ws=None, wsb=0)
    a.update(call_kw)
    assert lib.tis_cache_tree_decode(a["Q"], a["K"], a["V"], a["dt"], a["Hq"], ctypes.byref(t),
                                     a["beam"], a["scale"], a["O"], a["idx"], a["ws"], a["wsb"],
                                     None) == status
    assert lib.tis_last_error().decode()


@pytest.mark.parametrize("tree_kw,call_kw,status", [
    (dict(n=100, lv=3), dict(Q=None), _lib.TIS_E_NULL),
    (dict(n=100, lv=3), dict(K=None), _lib.TIS_E_NULL),
    (dict(n=100, lv=3, state=None), dict(), _lib.TIS_E_NULL),
    (dict(n=1000, lv=6), dict(), _lib.TIS_E_SHAPE),            # the cache is full
    (dict(n=100, lv=4), dict(), _lib.TIS_E_SHAPE),             # levels do not match n_keys
    (dict(n=100, lv=3, half=2), dict(), _lib.TIS_E_SHAPE),     # no such state half
    (dict(n=100, lv=3, sd=_lib.TIS_FP8_E4M3), dict(), _lib.TIS_E_UNSUPPORTED),
    (dict(n=100, lv=3), dict(dt=2), _lib.TIS_E_DTYPE),
    (dict(n=100, lv=3, H=2), dict(Hq=3), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3), dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3), dict(beam=200), _lib.TIS_E_UNSUPPORTED),
    (dict(n=100, lv=3), dict(scale=float("inf")), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3), dict(V=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(n=30000, lv=4, d=128, b=4, L=128, C=30001), dict(beam=64, Hq=2), _lib.TIS_E_NULL),
])
def test_cache_append_decode_rejects(lib, tree_kw, call_kw, status):
    """A rejected step launches nothing and leaves the tree as it was."""
    t = _ctree(**tree_kw)
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, beam=4, scale=0.0, O=FAKE, idx=None,
             ws=None, wsb=0)
    a.update(call_kw)
    assert lib.tis_cache_tree_append_decode(a["Q"], a["K"], a["V"], a["dt"], a["Hq"],
                                            ctypes.byref(t), a["beam"], a["scale"], a["O"],
                                            a["idx"], a["ws"], a["wsb"], None) == status
    assert lib.tis_last_error().decode()
    assert (t.n_keys, t.levels, t.state_half) == (tree_kw.get("n", 0), tree_kw.get("lv", 0),
                                                  tree_kw.get("half", 0))


def test_caller_buffers_must_match():
    """An output buffer handed to the binding is checked before any launch."""
    torch = pytest.importorskip("torch")
    from tree_indexed_sparse_build_amd import ops
    with pytest.raises(ValueError, match="shape"):
        ops._check_buffer(torch.empty(2, 3, 4), (2, 3, 8), torch.float32, "out")
    with pytest.raises(ValueError, match="int32"):
        ops._check_buffer(torch.empty(2, 3, 4), (2, 3, 4), torch.int32, "indices")


# ----------------------------------------------------- bounding spheres --

def test_radius_bytes(lib):
    # 4 x 8 heads, b 8, 3 levels: 8 + 64 + 512 nodes each
    assert lib.tis_tree_radius_bytes(4, 8, 8, 3) == 4 * 32 * 584
    assert lib.tis_radius_workspace_bytes(4, 8, 8, 3) == 8 * 32 * 584
    assert lib.tis_tree_radius_bytes(1, 1, 1, 3) == 0
    assert lib.tis_radius_workspace_bytes(1, 1, 2, 17) == 0
    assert lib.tis_decode_threshold_workspace_bytes(4, 32, 128, 8, 64) == 0


def _radii(lib, **kw):
    a = dict(K=FAKE, dt=_lib.TIS_BF16, tree=_tree(), radii=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib.tis_tree_radii(a["K"], a["dt"], ctypes.byref(a["tree"]), a["radii"], a["ws"],
                              a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), _lib.TIS_E_NULL),
    (dict(radii=None), _lib.TIS_E_NULL),
    (dict(ws=None), _lib.TIS_E_NULL),
    (dict(tree=_tree(summ=None)), _lib.TIS_E_NULL),
    (dict(dt=4), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(sd=7)), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(sd=_lib.TIS_FP8_E4M3)), _lib.TIS_E_UNSUPPORTED),
    (dict(tree=_lib.TisTree(1, 1, 100, 64, 2, 16, 3, 0, FAKE)), _lib.TIS_E_SHAPE),
    (dict(wsb=8 * 14 - 1), _lib.TIS_E_WORKSPACE),      # 2 + 4 + 8 nodes need 112 bytes
    (dict(radii=FAKE + 2), _lib.TIS_E_ALIGN),
    (dict(ws=FAKE + 8), _lib.TIS_E_ALIGN),
])
def test_radii_rejects(lib, kw, status):
    assert _radii(lib, **kw) == status
    assert lib.tis_last_error().decode()


def _threshold(lib, fused, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, tree=_tree(H=1), radii=FAKE,
             tau=FAKE, nodes=8, idx=FAKE, cnt=FAKE, O=FAKE, scale=0.0, ws=None, wsb=0)
    a.update(kw)
    if not fused:
        return lib.tis_tree_route_threshold(a["Q"], a["dt"], a["Hq"], ctypes.byref(a["tree"]),
                                            a["radii"], a["tau"], a["nodes"], a["idx"], a["cnt"],
                                            None)
    return lib.tis_tree_decode_threshold(a["Q"], a["K"], a["V"], a["dt"], a["Hq"],
                                         ctypes.byref(a["tree"]), a["radii"], a["tau"],
                                         a["nodes"], a["scale"], a["O"], a["idx"], a["cnt"],
                                         a["ws"], a["wsb"], None)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), _lib.TIS_E_NULL),
    (dict(radii=None), _lib.TIS_E_NULL),
    (dict(tau=None), _lib.TIS_E_NULL),
    (dict(tree=_tree(summ=None)), _lib.TIS_E_NULL),
    (dict(dt=3), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(sd=9)), _lib.TIS_E_DTYPE),
    (dict(tree=_tree(sd=_lib.TIS_FP8_E4M3)), _lib.TIS_E_UNSUPPORTED),
    (dict(Hq=0), _lib.TIS_E_SHAPE),
    (dict(tree=_tree(H=2), Hq=3), _lib.TIS_E_SHAPE),
    (dict(nodes=0), _lib.TIS_E_SHAPE),
    (dict(nodes=_lib.TIS_MAX_SURVIVORS + 1), _lib.TIS_E_UNSUPPORTED),
    (dict(tau=FAKE + 2), _lib.TIS_E_ALIGN),
    (dict(radii=FAKE + 1), _lib.TIS_E_ALIGN),
    (dict(Q=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(cnt=FAKE + 2), _lib.TIS_E_ALIGN),
])
def test_threshold_rejects(lib, fused, kw, status):
    assert _threshold(lib, fused, **kw) == status
    assert lib.tis_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(K=None), _lib.TIS_E_NULL),
    (dict(O=None), _lib.TIS_E_NULL),
    (dict(scale=float("inf")), _lib.TIS_E_SHAPE),
    (dict(V=FAKE + 4), _lib.TIS_E_ALIGN),
])
def test_decode_threshold_rejects(lib, kw, status):
    assert _threshold(lib, True, **kw) == status


# -------------------------------------------------------- causal prefill --

def test_prefill_workspace_bytes(lib):
    f = lib.tis_causal_prefill_workspace_bytes
    F32, BF16 = _lib.TIS_F32, _lib.TIS_BF16

    def up(x):
        return -(-x // 256) * 256

    # 1,024 keys, b 2, L 32: depth 5; one fp32 row per (head, position,
    # height), an fp64 row per (head, run of 64 keys); L a multiple of 16 and
    # 32 or more, so also the kept leaves (2 query heads, beam 3) and V per 16
    # keys (fp32)
    means, sums = 1024 * 5 * 64 * 4, 16 * 64 * 8
    idx = up(means + sums)
    vt = up(idx + 2 * 1024 * 3 * 4)
    assert f(1, 1, 2, 64, 2, 32, 1024, 3, F32, F32) == vt + 64 * 16 * 64 * 4
    # bf16 keys: V's copy is half as large
    assert f(1, 1, 2, 64, 2, 32, 1024, 3, BF16, F32) == vt + 64 * 16 * 64 * 2
    # L 16 and L 5: no 16-position attention, so no leaves or V copy
    assert f(1, 1, 2, 64, 2, 16, 1024, 3, F32, F32) == 1024 * 6 * 64 * 4 + sums
    assert f(2, 3, 6, 128, 4, 5, 100, 2, BF16, BF16) == (
        6 * 100 * 3 * 128 * 2 + 6 * 2 * 128 * 8)   # 100 keys: 4^3 * 5 = 320 >= 100, depth 3
    # past 64^2 keys the sums get a second level (runs of 4,096 keys), past
    # 64^3 a third: 300,000 keys, b 4, L 32: 4^7 * 32 >= 300,000, depth 7
    n = 300_000
    runs = -(-n // 64) + -(-n // 64 ** 2) + -(-n // 64 ** 3)
    idx = up(2 * n * 7 * 64 * 4 + 2 * runs * 64 * 8)
    vt = up(idx + 2 * n * 1 * 4)
    assert f(1, 2, 2, 64, 4, 32, n, 1, F32, F32) == vt + 2 * (-(-n // 16)) * 16 * 64 * 4
    # a beam whose union table fits no workgroup (f32, d 128, beam 88, even
    # one head a workgroup): the fused kernel, no leaves or V copy
    assert f(1, 1, 1, 128, 2, 32, 1024, 88, F32, F32) == 1024 * 5 * 128 * 4 + 16 * 128 * 8
    # invalid: no keys, head_dim 96, summary type 5, fp8 keys, q_heads not a
    # multiple of kv_heads, beam 0
    assert f(1, 1, 1, 64, 2, 16, 0, 1, F32, F32) == 0
    assert f(1, 1, 1, 96, 2, 16, 10, 1, F32, F32) == 0
    assert f(1, 1, 1, 64, 2, 16, 10, 1, F32, 5) == 0
    assert f(1, 1, 1, 64, 2, 16, 10, 1, _lib.TIS_FP8_E4M3, F32) == 0
    assert f(1, 2, 3, 64, 2, 16, 10, 1, F32, F32) == 0
    assert f(1, 1, 1, 64, 2, 16, 10, 0, F32, F32) == 0


def _prefill(lib, tree_kw=None, **kw):
    t = _ctree(**(tree_kw or dict(n=100, lv=3)))
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=_lib.TIS_BF16, Hq=2, beam=2, scale=0.0, O=FAKE,
             idx=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.tis_causal_prefill(a["Q"], a["K"], a["V"], a["dt"], a["Hq"], ctypes.byref(t),
                                  a["beam"], a["scale"], a["O"], a["idx"], a["ws"], a["wsb"],
                                  None)


@pytest.mark.parametrize("tree_kw,kw,status", [
    (None, dict(Q=None), _lib.TIS_E_NULL),
    (None, dict(ws=None), _lib.TIS_E_NULL),
    (None, dict(O=None), _lib.TIS_E_NULL),
    (dict(n=0, lv=0), dict(), _lib.TIS_E_SHAPE),            # empty tree
    (dict(n=100, lv=2), dict(), _lib.TIS_E_SHAPE),          # wrong depth
    (None, dict(dt=6), _lib.TIS_E_DTYPE),
    (dict(n=100, lv=3, sd=4), dict(), _lib.TIS_E_DTYPE),
    (dict(n=100, lv=3, sd=_lib.TIS_FP8_E4M3), dict(), _lib.TIS_E_UNSUPPORTED),
    (None, dict(beam=0), _lib.TIS_E_SHAPE),
    (dict(n=100, lv=3, H=2), dict(Hq=3), _lib.TIS_E_SHAPE),
    (None, dict(scale=float("nan")), _lib.TIS_E_SHAPE),
    (None, dict(wsb=100 * 3 * 64 * 4 - 1), _lib.TIS_E_WORKSPACE),
    (None, dict(ws=FAKE + 4), _lib.TIS_E_ALIGN),
    (None, dict(O=FAKE + 4), _lib.TIS_E_ALIGN),
    (None, dict(Hq=1 << 25), _lib.TIS_E_UNSUPPORTED),       # 2^25 heads x 100 positions
])
def test_prefill_rejects(lib, tree_kw, kw, status):
    assert _prefill(lib, tree_kw, **kw) == status
    assert lib.tis_last_error().decode()


def test_struct_layout_matches_the_header(tmp_path):
    """The binding's ctypes structs have the C header's layout: every field's
    offset and each struct's size, from a C program compiled against
    include/tis.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"tis_tree": _lib.TisTree, "tis_cache_tree": _lib.TisCacheTree}
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "tis.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c99", "-I", inc, "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {}
    for line in out.splitlines():
        cname, field, value = line.split()
        got[(cname, field)] = int(value)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


# ------------------------------------------------- measurement probes --
@pytest.mark.parametrize("kw,status", [
    (dict(buf=None), _lib.TIS_E_NULL),
    (dict(sink=None), _lib.TIS_E_NULL),
    (dict(buf=FAKE + 8), _lib.TIS_E_ALIGN),
    (dict(nbytes=0), _lib.TIS_E_SHAPE),
    (dict(nbytes=24), _lib.TIS_E_SHAPE),
])
def test_probe_read_rejects(lib, kw, status):
    a = dict(buf=FAKE, nbytes=1 << 20, nt=0, sink=FAKE)
    a.update(kw)
    assert lib.tis_probe_read(a["buf"], a["nbytes"], a["nt"], a["sink"], None) == status
    assert lib.tis_last_error().decode().startswith("tis_probe_read")


@pytest.mark.parametrize("kw,status", [
    (dict(nxt=None), _lib.TIS_E_NULL),
    (dict(out=None), _lib.TIS_E_NULL),
    (dict(nxt=FAKE + 2), _lib.TIS_E_ALIGN),
    (dict(n=0), _lib.TIS_E_SHAPE),
    (dict(n=1 << 32), _lib.TIS_E_SHAPE),
    (dict(hops=-1), _lib.TIS_E_SHAPE),
])
def test_probe_chase_rejects(lib, kw, status):
    a = dict(nxt=FAKE, n=1024, start=0, hops=10, out=FAKE)
    a.update(kw)
    assert lib.tis_probe_chase(a["nxt"], a["n"], a["start"], a["hops"], a["out"], None) == status
    assert lib.tis_last_error().decode().startswith("tis_probe_chase")
