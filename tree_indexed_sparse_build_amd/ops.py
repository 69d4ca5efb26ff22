"""Python binding of the three calls: tree_build, tree_route, tree_attend.

Torch supplies device memory and the stream; every step of the computation
runs in libtis's HIP kernels.  Tensors must live on a ROCm device; float32
and bfloat16 are the accepted element types.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Dict, Optional, Tuple

import torch

from . import _lib
from ._lib import TisCacheTree, TisTree, check, lib

_DTYPES = {torch.float32: _lib.TIS_F32, torch.bfloat16: _lib.TIS_BF16}

__all__ = ["Tree", "DecodePlan", "CacheTree", "tree_build", "tree_route", "tree_attend",
           "tree_decode", "tree_decode_noalloc", "decode", "version", "from_storage",
           "summary_offsets"]


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _need_device(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a ROCm device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# stored summary types: name -> (tis_dtype code, torch dtype of the buffer);
# "fp8" (full tree only): e4m3 codes, then a float32 power-of-two scale per node
SUMMARY_DTYPES = {"f32": (0, torch.float32), "bf16": (1, torch.bfloat16),
                  "fp8": (2, torch.uint8)}


def _summary_dtype(name: str):
    try:
        return SUMMARY_DTYPES[name]
    except KeyError:
        raise ValueError(f"summary_dtype must be one of {sorted(SUMMARY_DTYPES)}") from None


def _check_buffer(t: torch.Tensor, shape, dtype: torch.dtype, name: str) -> None:
    """A caller-supplied output must be exactly what the kernel writes."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}")
    _need_device(t)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# Workspaces, one per (device, kind), grown on demand and reused: calls are
# ordered on the caller's stream.  They start zeroed: the arrival counters at
# the start of a build, attend or decode workspace must be zero on first
# use, and every call leaves them so.
_workspaces: Dict[Tuple[int, str], torch.Tensor] = {}


def _workspace(device: torch.device, kind: str, nbytes: int) -> torch.Tensor:
    key = (device.index if device.index is not None else torch.cuda.current_device(), kind)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


@dataclasses.dataclass
class Tree:
    """A built tree: summaries (float32, or bfloat16 with summary_dtype
    "bf16"), level-major ([B, Hkv, n_l, d] blocks for l = 1..levels,
    concatenated), plus its geometry."""
    summaries: torch.Tensor
    batch: int
    kv_heads: int
    n_keys: int
    head_dim: int
    branching: int
    leaf_block: int
    levels: int
    summary_dtype: str = "f32"

    def c_struct(self) -> TisTree:
        return TisTree(self.batch, self.kv_heads, self.n_keys, self.head_dim, self.branching,
                       self.leaf_block, self.levels, _summary_dtype(self.summary_dtype)[0],
                       self.summaries.data_ptr())

    def level(self, l: int) -> torch.Tensor:
        """Summaries of level l (1..levels) as a [B, Hkv, b**l, d] view; for
        fp8 summaries a float32 copy of the values they stand for (each code
        times its node's scale)."""
        off = summary_offsets(self.batch, self.kv_heads, self.head_dim, self.branching,
                              self.levels)
        n = self.branching ** l
        rows = self.summaries[off[l - 1]:off[l - 1] + self.batch * self.kv_heads * n *
                              self.head_dim].view(self.batch, self.kv_heads, n, self.head_dim)
        if self.summary_dtype != "fp8":
            return rows
        total = off[-1]
        sc_off = -(-total // 16) * 16
        scales = self.summaries[sc_off:sc_off + 4 * (total // self.head_dim)].view(torch.float32)
        first = off[l - 1] // self.head_dim
        sc = scales[first:first + self.batch * self.kv_heads * n].view(
            self.batch, self.kv_heads, n, 1)
        return _e4m3_values(rows) * sc


def _e4m3_values(codes: torch.Tensor) -> torch.Tensor:
    """float32 values of e4m3 codes (torch's own float8_e4m3fn decoding)."""
    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    return table.to(codes.device)[codes.long()]


def summary_offsets(batch, kv_heads, head_dim, branching, levels):
    off, out = 0, []
    for l in range(1, levels + 1):
        out.append(off)
        off += batch * kv_heads * branching ** l * head_dim
    out.append(off)
    return out


def tree_build(K: torch.Tensor, branching: int, leaf_block: int, levels: int,
               summary_dtype: str = "f32") -> Tree:
    """Summaries of every node: K [B, Hkv, N, d] with N = branching**levels * leaf_block;
    summary_dtype "f32" or "bf16" (each mean rounded once to that type)."""
    _need_device(K)
    if K.dim() != 4:
        raise ValueError("K must be [B, Hkv, N, d]")
    B, H, N, d = K.shape
    code, tdt = _summary_dtype(summary_dtype)
    L = lib()
    nbytes = L.tis_tree_summary_bytes_as(B, H, d, branching, levels, code)
    if nbytes == 0:
        raise _lib.TisError(_lib.TIS_E_SHAPE, "invalid tree geometry")
    summ = torch.empty(nbytes // tdt.itemsize, dtype=tdt, device=K.device)
    wsb = L.tis_build_workspace_bytes(B, H, N, d, branching, leaf_block, levels)
    ws = _workspace(K.device, "build", wsb) if wsb else None
    t = TisTree(0, 0, 0, 0, 0, 0, 0, code, summ.data_ptr())
    check(L.tis_tree_build(K.data_ptr(), _dtype_code(K), B, H, N, d, branching, leaf_block,
                           levels, ctypes.byref(t), ws.data_ptr() if ws is not None else None,
                           ws.numel() if ws is not None else 0, _stream(K.device)))
    return Tree(summ, t.batch, t.kv_heads, t.n_keys, t.head_dim, t.branching, t.leaf_block,
                t.levels, summary_dtype)


def tree_route(Q: torch.Tensor, tree: Tree, beam: int, trace: bool = False):
    """Leaf blocks each query keeps: int32 [B, Hq, beam], ascending.  With
    trace=True also returns the kept nodes of every level, int32
    [B, Hq, levels, beam] padded with -1."""
    _need_device(Q, tree.summaries)
    if Q.dim() != 3:
        raise ValueError("Q must be [B, Hq, d]")
    B, Hq, d = Q.shape
    if B != tree.batch or d != tree.head_dim:
        raise ValueError("Q does not match the tree's batch / head_dim")
    idx = torch.empty((B, Hq, beam), dtype=torch.int32, device=Q.device)
    tr = (torch.empty((B, Hq, tree.levels, beam), dtype=torch.int32, device=Q.device)
          if trace else None)
    t = tree.c_struct()
    check(lib().tis_tree_route(Q.data_ptr(), _dtype_code(Q), Hq, ctypes.byref(t), beam,
                               idx.data_ptr(), tr.data_ptr() if tr is not None else None,
                               _stream(Q.device)))
    return (idx, tr) if trace else idx


def tree_attend(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, indices: torch.Tensor,
                leaf_block: int, scale: Optional[float] = None) -> torch.Tensor:
    """Softmax attention of each query over the keys of its selected leaf
    blocks.  Q [B, Hq, d]; K, V [B, Hkv, N, d]; indices int32 [B, Hq, W].
    Returns float32 [B, Hq, d]."""
    _need_device(Q, K, V, indices)
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    B, Hq, d = Q.shape
    _, Hkv, N, _ = K.shape
    if tuple(V.shape) != tuple(K.shape) or K.shape[0] != B or K.shape[3] != d:
        raise ValueError("shape mismatch between Q, K and V")
    if indices.dim() != 3 or indices.shape[0] != B or indices.shape[1] != Hq:
        raise ValueError("indices must be [B, Hq, W]")
    W = indices.shape[2]
    O = torch.empty((B, Hq, d), dtype=torch.float32, device=Q.device)
    L = lib()
    wsb = L.tis_attend_workspace_bytes(B, Hq, d, W, leaf_block)
    ws = _workspace(Q.device, "attend", wsb) if wsb else None
    check(L.tis_tree_attend(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, Hq,
                            Hkv, N, d, leaf_block, indices.data_ptr(), W,
                            0.0 if scale is None else float(scale), O.data_ptr(),
                            ws.data_ptr() if ws is not None else None,
                            ws.numel() if ws is not None else 0, _stream(Q.device)))
    return O


def tree_attend_grouped(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                        indices: torch.Tensor, leaf_block: int,
                        scale: Optional[float] = None) -> torch.Tensor:
    """tree_attend with the query heads that share a KV head attended
    together (each shared leaf read once per group, scores and P V on the
    matrix cores).  Same arguments and result as tree_attend, to fp32
    rounding."""
    _need_device(Q, K, V, indices)
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    B, Hq, d = Q.shape
    _, Hkv, N, _ = K.shape
    if tuple(V.shape) != tuple(K.shape) or K.shape[0] != B or K.shape[3] != d:
        raise ValueError("shape mismatch between Q, K and V")
    if indices.dim() != 3 or indices.shape[0] != B or indices.shape[1] != Hq:
        raise ValueError("indices must be [B, Hq, W]")
    W = indices.shape[2]
    O = torch.empty((B, Hq, d), dtype=torch.float32, device=Q.device)
    L = lib()
    wsb = L.tis_attend_grouped_workspace_bytes(B, Hq, Hkv, d, W)
    ws = _workspace(Q.device, "attend", wsb) if wsb else None
    check(L.tis_tree_attend_grouped(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B,
                                    Hq, Hkv, N, d, leaf_block, indices.data_ptr(), W,
                                    0.0 if scale is None else float(scale), O.data_ptr(),
                                    ws.data_ptr() if ws is not None else None,
                                    ws.numel() if ws is not None else 0, _stream(Q.device)))
    return O


def tree_decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, tree: Tree, beam: int,
                scale: Optional[float] = None, return_indices: bool = False):
    """Route and attend every query in one launch.  Returns O (float32
    [B, Hq, d]), and with return_indices=True also the kept leaves (int32
    [B, Hq, beam], ascending, the same as tree_route's)."""
    _need_device(Q, K, V, tree.summaries)
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    B, Hq, d = Q.shape
    if (B, d) != (tree.batch, tree.head_dim) or tuple(K.shape) != (
            tree.batch, tree.kv_heads, tree.n_keys, tree.head_dim) or V.shape != K.shape:
        raise ValueError("Q, K, V do not match the tree")
    O = torch.empty((B, Hq, d), dtype=torch.float32, device=Q.device)
    idx = (torch.empty((B, Hq, beam), dtype=torch.int32, device=Q.device)
           if return_indices else None)
    t = tree.c_struct()
    L = lib()
    wsb = L.tis_decode_workspace_bytes(B, Hq, d, beam, tree.leaf_block)
    ws = _workspace(Q.device, "decode", wsb) if wsb else None
    check(L.tis_tree_decode(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), Hq,
                            ctypes.byref(t), beam, 0.0 if scale is None else float(scale),
                            O.data_ptr(), idx.data_ptr() if idx is not None else None,
                            ws.data_ptr() if ws is not None else None,
                            ws.numel() if ws is not None else 0, _stream(Q.device)))
    return (O, idx) if return_indices else O


def tree_decode_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, tree: Tree,
                        beam: int, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                        indices: Optional[torch.Tensor] = None) -> torch.Tensor:
    """tree_decode through tis_tree_decode_noalloc: no workspace, the library
    keeps the split partial states in its own per-GPU scratch.  With `out`
    (float32 [B, Hq, d]) and, optionally, `indices` (int32 [B, Hq, beam])
    given, nothing is allocated on this path either.  Calls that may overlap
    on one GPU race (they share the scratch).  Returns O."""
    _need_device(Q, K, V, tree.summaries)
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    B, Hq, d = Q.shape
    if (B, d) != (tree.batch, tree.head_dim) or tuple(K.shape) != (
            tree.batch, tree.kv_heads, tree.n_keys, tree.head_dim) or V.shape != K.shape:
        raise ValueError("Q, K, V do not match the tree")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=Q.device)
    else:
        _check_buffer(out, (B, Hq, d), torch.float32, "out")
    if indices is not None:
        _check_buffer(indices, (B, Hq, beam), torch.int32, "indices")
    t = tree.c_struct()
    check(lib().tis_tree_decode_noalloc(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                                        Hq, ctypes.byref(t), beam,
                                        0.0 if scale is None else float(scale), out.data_ptr(),
                                        indices.data_ptr() if indices is not None else None,
                                        _stream(Q.device)))
    return out


def tree_radii(K: torch.Tensor, tree: Tree) -> torch.Tensor:
    """Radius of every node about its stored summary (the smallest float32
    whose square covers the largest squared key distance): float32, level-
    major, one element per node (level l a [B, Hkv, b**l] block)."""
    _need_device(K, tree.summaries)
    L = lib()
    nb = L.tis_tree_radius_bytes(tree.batch, tree.kv_heads, tree.branching, tree.levels)
    wsb = L.tis_radius_workspace_bytes(tree.batch, tree.kv_heads, tree.branching, tree.levels)
    if nb == 0:
        raise _lib.TisError(_lib.TIS_E_SHAPE, "invalid tree geometry")
    radii = torch.empty(nb // 4, dtype=torch.float32, device=K.device)
    ws = _workspace(K.device, "radii", wsb)
    t = tree.c_struct()
    check(L.tis_tree_radii(K.data_ptr(), _dtype_code(K), ctypes.byref(t), radii.data_ptr(),
                           ws.data_ptr(), ws.numel(), _stream(K.device)))
    return radii


def radii_level(tree: Tree, radii: torch.Tensor, l: int) -> torch.Tensor:
    """Radii of level l as a [B, Hkv, b**l] view."""
    heads = tree.batch * tree.kv_heads
    off = heads * sum(tree.branching ** k for k in range(1, l))
    n = tree.branching ** l
    return radii[off:off + heads * n].view(tree.batch, tree.kv_heads, n)


def _check_tau(tau: torch.Tensor, B: int, Hq: int) -> None:
    _check_buffer(tau, (B, Hq), torch.float32, "tau")


def tree_route_threshold(Q: torch.Tensor, tree: Tree, radii: torch.Tensor, tau: torch.Tensor,
                         max_nodes: int):
    """Leaves whose every ancestor's sphere bound q.c + |q| r reaches tau:
    (indices int32 [B, Hq, max_nodes] ascending, -1 padded; counts int32
    [B, Hq], -1 where a level had more than max_nodes survivors)."""
    _need_device(Q, tree.summaries, radii)
    B, Hq, d = Q.shape
    _check_tau(tau, B, Hq)
    idx = torch.empty((B, Hq, max_nodes), dtype=torch.int32, device=Q.device)
    cnt = torch.empty((B, Hq), dtype=torch.int32, device=Q.device)
    t = tree.c_struct()
    check(lib().tis_tree_route_threshold(Q.data_ptr(), _dtype_code(Q), Hq, ctypes.byref(t),
                                         radii.data_ptr(), tau.data_ptr(), int(max_nodes),
                                         idx.data_ptr(), cnt.data_ptr(), _stream(Q.device)))
    return idx, cnt


def tree_decode_threshold(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, tree: Tree,
                          radii: torch.Tensor, tau: torch.Tensor, max_nodes: int,
                          scale: Optional[float] = None, return_indices: bool = False,
                          out: Optional[torch.Tensor] = None):
    """Softmax over the keys with q.k >= tau, found through the sphere bound,
    in one launch.  Returns O (float32 [B, Hq, d]; zero rows where no key
    reaches tau, NaN after an overflow) and, with return_indices=True, also
    (indices, counts) as tree_route_threshold gives them."""
    _need_device(Q, K, V, tree.summaries, radii)
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    B, Hq, d = Q.shape
    _check_tau(tau, B, Hq)
    O = out if out is not None else torch.empty((B, Hq, d), dtype=torch.float32,
                                                 device=Q.device)
    _check_buffer(O, (B, Hq, d), torch.float32, "out")
    idx = cnt = None
    if return_indices:
        idx = torch.empty((B, Hq, max_nodes), dtype=torch.int32, device=Q.device)
        cnt = torch.empty((B, Hq), dtype=torch.int32, device=Q.device)
    L = lib()
    wsb = L.tis_decode_threshold_workspace_bytes(B, Hq, d, max_nodes, tree.leaf_block)
    ws = _workspace(Q.device, "decode", wsb) if wsb else None
    t = tree.c_struct()
    check(L.tis_tree_decode_threshold(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q),
                                      Hq, ctypes.byref(t), radii.data_ptr(), tau.data_ptr(),
                                      int(max_nodes), 0.0 if scale is None else float(scale),
                                      O.data_ptr(), idx.data_ptr() if idx is not None else None,
                                      cnt.data_ptr() if cnt is not None else None,
                                      ws.data_ptr() if ws is not None else None,
                                      ws.numel() if ws is not None else 0, _stream(Q.device)))
    return (O, idx, cnt) if return_indices else O


def decode(Q, K, V, branching: int, leaf_block: int, levels: int, beam: int,
           scale: Optional[float] = None):
    """Build, then one fused decode step, on the current stream (no host sync
    between).  Returns (tree, indices, O)."""
    tree = tree_build(K, branching, leaf_block, levels)
    out, idx = tree_decode(Q, K, V, tree, beam, scale, return_indices=True)
    return tree, idx, out


def version() -> str:
    return lib().tis_version().decode()


def from_storage(arr, dtype: str, device="cuda") -> torch.Tensor:
    """Device tensor from a host storage array: float32 values ("f32") or
    uint16 bf16 bit patterns ("bf16"), bits unchanged."""
    import numpy as np
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    elif dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)).view(
            torch.bfloat16)
    else:
        raise ValueError(f"unknown storage dtype {dtype!r}")
    return t.to(device)


class DecodePlan:
    """Pre-allocated buffers and C-ABI arguments for repeated build / route /
    attend over fixed device tensors, so a call costs one C-ABI call and no
    allocation (used by timing loops).  Each call goes to the current stream,
    so a step can be captured into a graph and replayed."""

    def __init__(self, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, branching: int,
                 leaf_block: int, levels: int, beam: int, scale: Optional[float] = None,
                 summary_dtype: str = "f32"):
        _need_device(Q, K, V)
        L = lib()
        self._lib = L
        B, H, N, d = K.shape
        Hq = Q.shape[1]
        self.Q, self.K, self.V = Q, K, V
        self.dt = _dtype_code(K)
        self.geom = (B, H, N, d, branching, leaf_block, levels)
        self.q_heads, self.beam, self.scale = Hq, beam, 0.0 if scale is None else float(scale)
        code, tdt = _summary_dtype(summary_dtype)
        self.summary_dtype = summary_dtype
        nbytes = L.tis_tree_summary_bytes_as(B, H, d, branching, levels, code)
        if nbytes == 0:
            raise _lib.TisError(_lib.TIS_E_SHAPE, "invalid tree geometry")
        self.summaries = torch.empty(nbytes // tdt.itemsize, dtype=tdt, device=K.device)
        wsb = L.tis_build_workspace_bytes(*self.geom)
        self.ws_build = (torch.zeros(wsb, dtype=torch.uint8, device=K.device) if wsb
                         else None)
        wsa = L.tis_attend_workspace_bytes(B, Hq, d, beam, leaf_block)
        self.ws_attend = (torch.zeros(wsa, dtype=torch.uint8, device=K.device) if wsa
                          else None)
        wsd = L.tis_decode_workspace_bytes(B, Hq, d, beam, leaf_block)
        self.ws_decode = (torch.zeros(wsd, dtype=torch.uint8, device=K.device) if wsd
                          else None)
        G = Hq // H
        wsg = L.tis_attend_grouped_workspace_bytes(B, Hq, H, d, beam)
        self.ws_grouped = (torch.zeros(max(wsg, 256), dtype=torch.uint8, device=K.device)
                           if G <= 64 and G * beam <= 512 else None)
        self.indices = torch.empty((B, Hq, beam), dtype=torch.int32, device=K.device)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=K.device)
        self.tree_c = TisTree(0, 0, 0, 0, 0, 0, 0, code, self.summaries.data_ptr())
        self.device = K.device

    def build(self) -> None:
        B, H, N, d, b, Lb, lv = self.geom
        ws = self.ws_build
        check(self._lib.tis_tree_build(self.K.data_ptr(), self.dt, B, H, N, d, b, Lb, lv,
                                       ctypes.byref(self.tree_c),
                                       None if ws is None else ws.data_ptr(),
                                       0 if ws is None else ws.numel(), _stream(self.device)))

    def route(self) -> None:
        check(self._lib.tis_tree_route(self.Q.data_ptr(), self.dt, self.q_heads,
                                       ctypes.byref(self.tree_c), self.beam,
                                       self.indices.data_ptr(), None, _stream(self.device)))

    def attend(self) -> None:
        B, H, N, d, b, Lb, lv = self.geom
        check(self._lib.tis_tree_attend(self.Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(),
                                        self.dt, B, self.q_heads, H, N, d, Lb,
                                        self.indices.data_ptr(), self.beam, self.scale,
                                        self.out.data_ptr(),
                                        None if self.ws_attend is None
                                        else self.ws_attend.data_ptr(),
                                        0 if self.ws_attend is None
                                        else self.ws_attend.numel(), _stream(self.device)))

    def attend_grouped(self) -> None:
        """attend() with the query heads of each KV head attended together
        (tree_attend_grouped) over the routed indices, into self.out."""
        B, H, N, d, b, Lb, lv = self.geom
        if self.ws_grouped is None:
            raise RuntimeError("this geometry has no grouped attend (G > 64 or G * beam > 512)")
        check(self._lib.tis_tree_attend_grouped(
            self.Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(), self.dt, B, self.q_heads, H,
            N, d, Lb, self.indices.data_ptr(), self.beam, self.scale, self.out.data_ptr(),
            self.ws_grouped.data_ptr(), self.ws_grouped.numel(), _stream(self.device)))

    def decode(self) -> None:
        """Route and attend in one launch (indices not written)."""
        B, H, N, d, b, Lb, lv = self.geom
        ws = self.ws_decode
        check(self._lib.tis_tree_decode(self.Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(),
                                        self.dt, self.q_heads, ctypes.byref(self.tree_c),
                                        self.beam, self.scale, self.out.data_ptr(), None,
                                        None if ws is None else ws.data_ptr(),
                                        0 if ws is None else ws.numel(), _stream(self.device)))

    def timeline_bytes(self) -> int:
        """Bytes of the buffer decode_timeline() fills."""
        B, H, N, d, b, Lb, lv = self.geom
        return int(self._lib.tis_probe_decode_timeline_bytes(B, self.q_heads, self.beam, Lb))

    def decode_timeline(self, timeline: torch.Tensor) -> None:
        """decode() by the instrumented kernel (tis_probe_decode_timeline):
        the same output in self.out, plus a wall-clock stamp per wave and
        phase in `timeline` (int64, timeline_bytes() bytes, cleared by the
        caller)."""
        B, H, N, d, b, Lb, lv = self.geom
        ws = self.ws_decode
        check(self._lib.tis_probe_decode_timeline(
            self.Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(), self.dt, self.q_heads,
            ctypes.byref(self.tree_c), self.beam, self.scale, self.out.data_ptr(),
            None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
            timeline.data_ptr(), timeline.numel() * timeline.element_size(),
            _stream(self.device)))

    def tree(self) -> Tree:
        B, H, N, d, b, Lb, lv = self.geom
        return Tree(self.summaries, B, H, N, d, b, Lb, lv)


class CacheTree:
    """The tree over a growing KV cache (tis_cache_tree_* calls).

    K and V are the cache: [B, Hkv, capacity, d] device tensors whose first
    n_keys rows are in use.  Write new rows into K (and V) first, then call
    append(n) to add them to the tree.  Summaries are height-major: height h
    (0 = leaves) is a [B, Hkv, ceil(capacity / (L b^h)), d] block; level l of
    the current tree is height levels - l.
    """

    def __init__(self, K: torch.Tensor, V: torch.Tensor, branching: int, leaf_block: int,
                 summary_dtype: str = "f32"):
        _need_device(K, V)
        if V.shape != K.shape or V.dtype != K.dtype:
            raise ValueError("K and V must match")
        B, H, C, d = K.shape
        L = lib()
        self.K, self.V = K, V
        self.dt = _dtype_code(K)
        code, tdt = _summary_dtype(summary_dtype)
        self.summary_dtype = summary_dtype
        sb = L.tis_cache_tree_summary_bytes_as(B, H, d, branching, leaf_block, C, code)
        stb = L.tis_cache_tree_state_bytes(B, H, d, branching, leaf_block, C)
        if sb == 0 or stb == 0:
            raise _lib.TisError(_lib.TIS_E_SHAPE, "invalid cache geometry")
        self.summaries = torch.empty(sb // tdt.itemsize, dtype=tdt, device=K.device)
        self.state = torch.empty(stb // 8, dtype=torch.float64, device=K.device)
        self.c = TisCacheTree(B, H, d, branching, leaf_block, C, 0, 0, code, 0,
                              self.summaries.data_ptr(), self.state.data_ptr())
        self._cref = ctypes.byref(self.c)
        self._kptr = K.data_ptr()
        self._append = L.tis_cache_tree_append
        self.reset()

    @property
    def n_keys(self) -> int:
        return self.c.n_keys

    @property
    def levels(self) -> int:
        return self.c.levels

    def reset(self) -> None:
        check(lib().tis_cache_tree_reset(ctypes.byref(self.c), _stream(self.K.device)))

    def append(self, n_new: int) -> None:
        check(self._append(self._kptr, self.dt, int(n_new), self._cref, _stream(self.K.device)))

    def height_block(self, h: int) -> torch.Tensor:
        """Summaries of height h as [B, Hkv, rows, d] (a view)."""
        c = self.c
        heads = c.batch * c.kv_heads
        off, span = 0, c.leaf_block
        for _ in range(h):
            off += heads * -(-c.capacity // span) * c.head_dim
            span *= c.branching
        rows = -(-c.capacity // span)
        return self.summaries[off:off + heads * rows * c.head_dim].view(
            c.batch, c.kv_heads, rows, c.head_dim)

    def level(self, l: int) -> torch.Tensor:
        """The existing nodes of level l (1 = below the root) of the current
        tree, [B, Hkv, e_l, d] (a view)."""
        c = self.c
        if not 1 <= l <= c.levels:
            raise ValueError(f"level {l} outside 1..{c.levels}")
        span = c.leaf_block * c.branching ** (c.levels - l)
        return self.height_block(c.levels - l)[:, :, :-(-c.n_keys // span)]

    def route(self, Q: torch.Tensor, beam: int, trace: bool = False):
        """Kept leaves ([B, Hq, beam] int32, ascending, -1 padded) and, with
        trace=True, the kept nodes per level ([B, Hq, levels, beam])."""
        _need_device(Q)
        if Q.dtype != self.K.dtype:
            raise TypeError("Q must have the cache's dtype")
        B, Hq, d = Q.shape
        idx = torch.empty((B, Hq, beam), dtype=torch.int32, device=Q.device)
        tr = (torch.empty((B, Hq, max(self.levels, 1), beam), dtype=torch.int32,
                          device=Q.device) if trace else None)
        check(lib().tis_cache_tree_route(Q.data_ptr(), self.dt, Hq, ctypes.byref(self.c), beam,
                                         idx.data_ptr(), tr.data_ptr() if tr is not None else None,
                                         _stream(Q.device)))
        return (idx, tr) if trace else idx

    def causal_prefill(self, Q: torch.Tensor, beam: int, scale: Optional[float] = None,
                       return_indices: bool = False, out: Optional[torch.Tensor] = None):
        """Every position t < n_keys as a query over the tree of the first
        t + 1 keys, attending causally.  Q: [B, Hq, n_keys, d], the query of
        each position.  Returns O (float32 [B, Hq, n_keys, d]) and, with
        return_indices=True, the kept leaves (int32 [B, Hq, n_keys, beam],
        ascending, -1 padded)."""
        _need_device(Q)
        if Q.dtype != self.K.dtype:
            raise TypeError("Q must have the cache's dtype")
        if Q.dim() != 4 or Q.shape[2] != self.n_keys:
            raise ValueError("Q must be [B, Hq, n_keys, d]")
        B, Hq, n, d = Q.shape
        O = out if out is not None else torch.empty((B, Hq, n, d), dtype=torch.float32,
                                                     device=Q.device)
        _check_buffer(O, (B, Hq, n, d), torch.float32, "out")
        idx = (torch.empty((B, Hq, n, beam), dtype=torch.int32, device=Q.device)
               if return_indices else None)
        c = self.c
        L = lib()
        wsb = L.tis_causal_prefill_workspace_bytes(c.batch, c.kv_heads, Hq, c.head_dim,
                                                   c.branching, c.leaf_block, c.n_keys, beam,
                                                   self.dt, c.summary_dtype)
        ws = _workspace(Q.device, "prefill", wsb)
        check(L.tis_causal_prefill(Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(), self.dt,
                                   Hq, ctypes.byref(c), beam,
                                   0.0 if scale is None else float(scale), O.data_ptr(),
                                   idx.data_ptr() if idx is not None else None, ws.data_ptr(),
                                   ws.numel(), _stream(Q.device)))
        return (O, idx) if return_indices else O

    def bind_decode(self, Q: torch.Tensor, beam: int, out: torch.Tensor,
                    scale: Optional[float] = None, append: bool = False):
        """A zero-argument callable that decodes Q into `out` on the current
        stream with every argument prepared once (for decode loops, where the
        host cost of a call would otherwise exceed the kernel's).  With
        append=True each call is append_decode: it first adds key n_keys
        (already written into K and V) to the tree."""
        _need_device(Q)
        if Q.dtype != self.K.dtype:
            raise TypeError("Q must have the cache's dtype")
        B, Hq, d = Q.shape
        _check_buffer(out, (B, Hq, d), torch.float32, "out")
        L = lib()
        wsb = L.tis_decode_workspace_bytes(B, Hq, d, beam, self.c.leaf_block)
        ws = _workspace(Q.device, "decode", wsb) if wsb else None
        f = L.tis_cache_tree_append_decode if append else L.tis_cache_tree_decode
        args = (Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(), self.dt, Hq,
                ctypes.byref(self.c), beam, 0.0 if scale is None else float(scale),
                out.data_ptr(), None, ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0)
        dev = Q.device
        keep = (Q, out, ws)  # the buffers must outlive the callable

        def run() -> None:
            _ = keep
            check(f(*args, _stream(dev)))
        return run

    def append_decode(self, Q: torch.Tensor, beam: int, scale: Optional[float] = None,
                      return_indices: bool = False, out: Optional[torch.Tensor] = None,
                      indices: Optional[torch.Tensor] = None):
        """One decode step: add key n_keys (already written into K and V) to
        the tree and decode Q over the tree with it, in one launch.  Same
        results and tree as append(1) followed by decode(...)."""
        return self._decode(lib().tis_cache_tree_append_decode, Q, beam, scale, return_indices,
                            out, indices)

    def decode(self, Q: torch.Tensor, beam: int, scale: Optional[float] = None,
               return_indices: bool = False, out: Optional[torch.Tensor] = None,
               indices: Optional[torch.Tensor] = None):
        """Route and attend every query over the cache in one launch."""
        return self._decode(lib().tis_cache_tree_decode, Q, beam, scale, return_indices, out,
                            indices)

    def _decode(self, f, Q, beam, scale, return_indices, out, indices):
        _need_device(Q)
        if Q.dtype != self.K.dtype:
            raise TypeError("Q must have the cache's dtype")
        B, Hq, d = Q.shape
        O = out if out is not None else torch.empty((B, Hq, d), dtype=torch.float32,
                                                     device=Q.device)
        _check_buffer(O, (B, Hq, d), torch.float32, "out")
        idx = indices
        if idx is None and return_indices:
            idx = torch.empty((B, Hq, beam), dtype=torch.int32, device=Q.device)
        if idx is not None:
            _check_buffer(idx, (B, Hq, beam), torch.int32, "indices")
        L = lib()
        wsb = L.tis_decode_workspace_bytes(B, Hq, d, beam, self.c.leaf_block)
        ws = _workspace(Q.device, "decode", wsb) if wsb else None
        check(f(Q.data_ptr(), self.K.data_ptr(), self.V.data_ptr(), self.dt, Hq,
                ctypes.byref(self.c), beam, 0.0 if scale is None else float(scale), O.data_ptr(),
                idx.data_ptr() if idx is not None else None,
                ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0, _stream(Q.device)))
        return (O, idx) if return_indices else O
