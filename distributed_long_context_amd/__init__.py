"""MI355X (gfx950) attention tiles for one GPU's share of distributed attention.

Thin Python binding over libmesh_attn.so (include/mesh_attn.h).  The functions
keep the C names; they only marshal torch tensors (device memory) and the
current HIP stream into the C structs.  Every step of the computation runs in
the library's HIP kernels; there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes as C
from typing import Iterable, Optional, Sequence

from . import _abi
from ._abi import (MA_OK, MA_ERR_INVALID, MA_ERR_UNSUPPORTED, MA_ERR_LAUNCH, MA_F32, MA_BF16, MA_MASK_NONE,
                   MA_MASK_CAUSAL, MA_MASK_STRIPED_ZIGZAG, MA_TILE_EMPTY, MA_TILE_PARTIAL, MA_TILE_FULL,
                   MA_MAX_MERGE, MeshAttnError, lib)

__all__ = [
    "mesh_attn_tile_fwd", "mesh_attn_merge", "mesh_attn_reduce_add", "mesh_attn_tile_bwd", "mesh_attn_tile_bwd_workspace_size",
    "mesh_attn_tile_bwd_noalloc",
    "mesh_attn_map_mesh_tile", "mesh_attn_map_groups", "mesh_attn_map_zigzag", "mesh_attn_pos_contiguous",
    "mesh_attn_pos_zigzag", "mesh_attn_pos_striped", "mesh_attn_pos_at", "mesh_attn_classify",
    "mesh_attn_count_allowed", "mesh_attn_build_worklist", "mesh_attn_goo_plan", "mesh_attn_version", "Pos", "Tile", "BwdTile",
    "MA_F32", "MA_BF16", "MA_MASK_NONE", "MA_MASK_CAUSAL", "MA_MASK_STRIPED_ZIGZAG", "MA_TILE_EMPTY",
    "MA_TILE_PARTIAL", "MA_TILE_FULL", "MeshAttnError", "lib",
]


# ---------------------------------------------------------------- positions --

class Pos:
    """Token positions of a partition: segments (local_begin, global_begin, stride)."""

    def __init__(self, segments: Sequence[Sequence[int]]):
        self.segments = [tuple(int(x) for x in s) for s in segments]

    @classmethod
    def from_c(cls, p: _abi.ma_pos) -> "Pos":
        return cls([(p.seg[i].local_begin, p.seg[i].global_begin, p.seg[i].stride) for i in range(p.nseg)])

    def to_c(self) -> _abi.ma_pos:
        p = _abi.ma_pos()
        p.nseg = len(self.segments)
        for i, (lb, gb, st) in enumerate(self.segments[:_abi.MA_MAX_SEGMENTS]):
            p.seg[i].local_begin, p.seg[i].global_begin, p.seg[i].stride = lb, gb, st
        return p

    def __repr__(self):
        return f"Pos({self.segments})"


_CONTIGUOUS_FROM_0 = None  # the ma_pos of a tile without positions (one segment from 0), built once


def _pos_c(pos: Optional[Pos]) -> _abi.ma_pos:
    global _CONTIGUOUS_FROM_0
    if pos is not None:
        return pos.to_c()
    if _CONTIGUOUS_FROM_0 is None:
        _CONTIGUOUS_FROM_0 = Pos([(0, 0, 1)]).to_c()
    return _CONTIGUOUS_FROM_0  # ctypes copies a structure on assignment into a tile record


# ------------------------------------------------------------ tensor checks --

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MA_BF16
    if t.dtype == torch.float32:
        return MA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last axis must be contiguous")


def _bshd_strides(t, name):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, S, H, d]")
    _check_dev(t, name)
    return (t.stride(0), t.stride(1), t.stride(2))


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _head_map_c(head_map, hq):
    if head_map is None:
        return None, None
    arr = (C.c_int32 * hq)(*[int(x) for x in head_map])
    return arr, C.cast(arr, C.POINTER(C.c_int32))


# ---------------------------------------------------------------- forward --

class Tile:
    """One (Q partition, KV partition) tile: q, k, v inputs and o, lse outputs (device tensors)."""

    def __init__(self, q, k, v, o, lse, q_pos: Optional[Pos] = None, k_pos: Optional[Pos] = None):
        self.q, self.k, self.v, self.o, self.lse = q, k, v, o, lse
        self.q_pos, self.k_pos = q_pos, k_pos


def mesh_attn_tile_fwd(tiles: Sequence[Tile], scale: float, mask_mode: int = MA_MASK_NONE, head_map=None,
                       stream=None, accumulate: bool = False, table: bool = False) -> None:
    """Partial (O, LSE) of every tile, enqueued on `stream` (default: current stream).
    With accumulate=True each tile's result is folded into the (O, LSE) its buffers hold.
    With table=True the call goes through mesh_attn_tile_fwd_tabled (the same results; the tile
    table is packed on the host, copied to the device on `stream` and launched from there)."""
    prepared = prepare_tile_fwd(tiles, scale, mask_mode, head_map, accumulate, table=table, stream=stream)
    if prepared is not None:
        launch_prepared_tile_fwd(prepared, stream)


def prepare_tile_fwd(tiles: Sequence[Tile], scale: float, mask_mode: int = MA_MASK_NONE, head_map=None,
                     accumulate: bool = False, table: bool = False, stream=None):
    """The checked argument block of mesh_attn_tile_fwd, to be launched (possibly many times) by
    launch_prepared_tile_fwd; it holds the tensors' addresses, so keep the tensors alive.
    With table=True the tile table is packed into pinned host memory and copied to the device on
    `stream` (default: current stream) here, once, for every launch of the prepared call."""
    tiles = list(tiles)
    if not tiles:
        return None
    t0 = tiles[0]
    B, _, Hq, d = t0.q.shape
    Hkv = t0.k.shape[2]
    dt = _dtype_code(t0.q)
    arr = (_abi.ma_tile * len(tiles))()
    for i, t in enumerate(tiles):
        for name, x in (("q", t.q), ("o", t.o)):
            if x.dim() != 4 or x.shape[0] != B or x.shape[2] != Hq or x.shape[3] != d or _dtype_code(x) != dt:
                raise ValueError(f"tile {i}: {name} shape/dtype mismatch")
            _check_dev(x, name)
        for name, x in (("k", t.k), ("v", t.v)):
            if x.dim() != 4 or x.shape[0] != B or x.shape[2] != Hkv or x.shape[3] != d or _dtype_code(x) != dt:
                raise ValueError(f"tile {i}: {name} shape/dtype mismatch")
            _check_dev(x, name)
        if t.o.shape[1] != t.q.shape[1] or t.v.shape[1] != t.k.shape[1]:
            raise ValueError(f"tile {i}: sequence lengths disagree")
        if tuple(t.lse.shape) != (B, Hq, t.q.shape[1]) or t.lse.dtype != _torch().float32:
            raise ValueError(f"tile {i}: lse must be float32 [B, Hq, Sq]")
        _check_dev(t.lse, "lse")
        for name, x, ref in (("q", t.q, t0.q), ("k", t.k, t0.k), ("v", t.v, t0.v), ("o", t.o, t0.o)):
            if x.stride()[:3] != ref.stride()[:3]:
                raise ValueError(f"tile {i}: {name} strides differ from tile 0")
        if t.lse.stride()[:2] != t0.lse.stride()[:2]:
            raise ValueError(f"tile {i}: lse strides differ from tile 0")
        c = arr[i]
        c.q, c.k, c.v, c.o, c.lse = t.q.data_ptr(), t.k.data_ptr(), t.v.data_ptr(), t.o.data_ptr(), t.lse.data_ptr()
        c.sq, c.sk = t.q.shape[1], t.k.shape[1]
        c.q_pos, c.k_pos = _pos_c(t.q_pos), _pos_c(t.k_pos)
    a = _abi.ma_tile_fwd_args()
    a.dtype, a.batch, a.hq, a.hkv, a.head_dim, a.mask_mode = dt, B, Hq, Hkv, d, int(mask_mode)
    a.scale, a.ntiles, a.accumulate = float(scale), len(tiles), 1 if accumulate else 0
    hm_keep, a.head_map = _head_map_c(head_map, Hq)
    a.tiles = C.cast(arr, C.POINTER(_abi.ma_tile))
    a.q_stride[:] = _bshd_strides(t0.q, "q")
    a.k_stride[:] = _bshd_strides(t0.k, "k")
    a.v_stride[:] = _bshd_strides(t0.v, "v")
    a.o_stride[:] = _bshd_strides(t0.o, "o")
    a.lse_stride[:] = (t0.lse.stride(0), t0.lse.stride(1))
    if not table:
        return (a, arr, hm_keep, None)
    torch = _torch()
    nbytes = lib().mesh_attn_tile_fwd_table_bytes(C.byref(a))
    if nbytes == 0:
        _abi.check(_abi.MA_ERR_INVALID, "mesh_attn_tile_fwd_table_bytes")
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    _abi.check(lib().mesh_attn_tile_fwd_pack(C.byref(a), C.c_void_p(host.data_ptr()), nbytes), "mesh_attn_tile_fwd_pack")
    s = stream if stream is not None else torch.cuda.current_stream()
    with torch.cuda.stream(s):
        dev = host.to(t0.q.device, non_blocking=True)
    return (a, arr, hm_keep, (host, dev, nbytes))


def launch_prepared_tile_fwd(prepared, stream=None) -> None:
    """Enqueue a forward prepared by prepare_tile_fwd (the C call only)."""
    if prepared[3] is None:
        _abi.check(lib().mesh_attn_tile_fwd(C.byref(prepared[0]), _stream_ptr(stream)), "mesh_attn_tile_fwd")
        return
    _, dev, nbytes = prepared[3]
    _abi.check(lib().mesh_attn_tile_fwd_tabled(C.byref(prepared[0]), C.c_void_p(dev.data_ptr()), nbytes,
                                               _stream_ptr(stream)), "mesh_attn_tile_fwd_tabled")


# ------------------------------------------------------------------ merge --

def mesh_attn_merge(o_in: Sequence, lse_in: Sequence, o_out, lse_out, stream=None) -> None:
    """Merge k partial (O [B,S,H,d], LSE [B,H,S]) pairs into (o_out, lse_out)."""
    k = len(o_in)
    if k != len(lse_in) or k < 1:
        raise ValueError("need k >= 1 matching O and LSE partials")
    B, S, H, d = o_out.shape
    dt = _dtype_code(o_out)
    _check_dev(o_out, "o_out")
    _check_dev(lse_out, "lse_out")
    # one comparison per property and partial (the checks run on every call)
    oshape, ostride, odtype, odev = o_out.shape, o_out.stride(), o_out.dtype, o_out.device
    for x in o_in:
        if x.shape != oshape or x.stride() != ostride or x.dtype != odtype or x.device != odev:
            raise ValueError("all O tensors must share shape, dtype, strides and device")
    lshape, lstride, f32 = lse_out.shape, lse_out.stride(), _torch().float32
    if tuple(lshape) != (B, H, S) or lse_out.dtype != f32:
        raise ValueError("all LSE tensors must be float32 [B, H, S] with equal strides")
    for x in lse_in:
        if x.shape != lshape or x.stride() != lstride or x.dtype != f32 or x.device != odev:
            raise ValueError("all LSE tensors must be float32 [B, H, S] with equal strides")
    optr = (C.c_void_p * k)(*[x.data_ptr() for x in o_in])
    lptr = (C.c_void_p * k)(*[x.data_ptr() for x in lse_in])
    a = _abi.ma_merge_args()
    a.dtype, a.batch, a.seqlen, a.heads, a.head_dim, a.k = dt, B, S, H, d, k
    a.o_in, a.lse_in = C.cast(optr, C.POINTER(C.c_void_p)), C.cast(lptr, C.POINTER(C.c_void_p))
    a.o_out, a.lse_out = o_out.data_ptr(), lse_out.data_ptr()
    a.o_stride[:] = _bshd_strides(o_out, "o_out")
    a.lse_stride[:] = (lse_out.stride(0), lse_out.stride(1))
    _abi.check(lib().mesh_attn_merge(C.byref(a), _stream_ptr(stream)), "mesh_attn_merge")


# ------------------------------------------------------------- add-reduce --

def mesh_attn_reduce_add(inputs: Sequence, out, stream=None) -> None:
    """out = sum of the k float32 tensors in `inputs` (same shape, contiguous), added in list order."""
    k = len(inputs)
    if k < 1:
        raise ValueError("need at least one input")
    torch = _torch()
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor")
    _check_dev(out, "out")
    for i, x in enumerate(inputs):
        if x.dtype != torch.float32 or not x.is_contiguous() or x.shape != out.shape:
            raise ValueError(f"input {i}: must be contiguous float32 of out's shape")
        _check_dev(x, f"input {i}")
    ptrs = (C.c_void_p * k)(*[x.data_ptr() for x in inputs])
    a = _abi.ma_reduce_args()
    a.k, a.n = k, out.numel()
    a.in_ = C.cast(ptrs, C.POINTER(C.c_void_p))
    a.out = out.data_ptr()
    _abi.check(lib().mesh_attn_reduce_add(C.byref(a), _stream_ptr(stream)), "mesh_attn_reduce_add")


# --------------------------------------------------------------- backward --

class BwdTile:
    """One tile of the backward: q, k, v, o, dout, lse inputs; dq, dk, dv float32 outputs."""

    def __init__(self, q, k, v, o, dout, lse, dq, dk, dv, q_pos: Optional[Pos] = None, k_pos: Optional[Pos] = None):
        self.q, self.k, self.v, self.o, self.dout, self.lse = q, k, v, o, dout, lse
        self.dq, self.dk, self.dv = dq, dk, dv
        self.q_pos, self.k_pos = q_pos, k_pos


def _bwd_args(tiles, scale, mask_mode, head_map, accumulate):
    torch = _torch()
    t0 = tiles[0]
    B, _, Hq, d = t0.q.shape
    Hkv = t0.k.shape[2]
    bf16, f32 = torch.bfloat16, torch.float32
    # tile 0's head/dim extents and strides, which every tile must share (read once)
    q_tail, k_tail = t0.q.shape[2:], t0.k.shape[2:]
    q_st, k_st = t0.q.stride()[:3], t0.k.stride()[:3]
    dq_st, dk_st, l_st = t0.dq.stride()[:3], t0.dk.stride()[:3], t0.lse.stride()[:2]

    def dev4(x, name):  # a device tensor with a contiguous last axis; its first three strides
        if not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        st = x.stride()
        if st[-1] != 1:
            raise ValueError(f"{name}: last axis must be contiguous")
        return st[:3]

    arr = (_abi.ma_bwd_tile * len(tiles))()
    for i, t in enumerate(tiles):
        sq, sk = t.q.shape[1], t.k.shape[1]
        for name, x in (("q", t.q), ("o", t.o), ("dout", t.dout)):
            shp = x.shape
            if x.dtype != bf16 or len(shp) != 4 or shp[0] != B or shp[2:] != q_tail or shp[1] != sq \
                    or dev4(x, name) != q_st:
                raise ValueError(f"tile {i}: {name} must be bf16 [B, Sq, Hq, d] with q's strides")
        for name, x in (("k", t.k), ("v", t.v)):
            shp = x.shape
            if x.dtype != bf16 or shp[0] != B or shp[2:] != k_tail or shp[1] != sk or dev4(x, name) != k_st:
                raise ValueError(f"tile {i}: {name} must be bf16 [B, Sk, Hkv, d] with k's strides")
        if t.dq.dtype != f32 or t.dq.shape != t.q.shape or dev4(t.dq, "dq") != dq_st:
            raise ValueError(f"tile {i}: dq must be float32 shaped like q")
        for name, x in (("dk", t.dk), ("dv", t.dv)):
            if x.dtype != f32 or x.shape != t.k.shape or dev4(x, name) != dk_st:
                raise ValueError(f"tile {i}: {name} must be float32 shaped like k")
        lse = t.lse
        if tuple(lse.shape) != (B, Hq, sq) or lse.dtype != f32 or lse.stride()[:2] != l_st:
            raise ValueError(f"tile {i}: lse must be float32 [B, Hq, Sq]")
        _check_dev(lse, "lse")
        c = arr[i]
        c.q, c.k, c.v, c.o, c.dout = t.q.data_ptr(), t.k.data_ptr(), t.v.data_ptr(), t.o.data_ptr(), t.dout.data_ptr()
        c.lse, c.dq, c.dk, c.dv = lse.data_ptr(), t.dq.data_ptr(), t.dk.data_ptr(), t.dv.data_ptr()
        c.sq, c.sk = sq, sk
        c.q_pos, c.k_pos = _pos_c(t.q_pos), _pos_c(t.k_pos)
    a = _abi.ma_tile_bwd_args()
    a.dtype, a.batch, a.hq, a.hkv, a.head_dim, a.mask_mode = MA_BF16, B, Hq, Hkv, d, int(mask_mode)
    a.scale, a.ntiles, a.accumulate = float(scale), len(tiles), int(bool(accumulate))
    keep, a.head_map = _head_map_c(head_map, Hq)
    a.tiles = C.cast(arr, C.POINTER(_abi.ma_bwd_tile))
    a.q_stride[:] = _bshd_strides(t0.q, "q")
    a.k_stride[:] = _bshd_strides(t0.k, "k")
    a.dq_stride[:] = _bshd_strides(t0.dq, "dq")
    a.dk_stride[:] = _bshd_strides(t0.dk, "dk")
    a.lse_stride[:] = (t0.lse.stride(0), t0.lse.stride(1))
    return a, (arr, keep)


def mesh_attn_tile_bwd_workspace_size(tiles: Sequence[BwdTile], scale: float, mask_mode: int, head_map=None) -> int:
    """Workspace bytes of mesh_attn_tile_bwd for these tiles under this mask (a masked call cuts
    multi-segment positions into pieces, each with its own slice)."""
    a, keep = _bwd_args(list(tiles), scale, mask_mode, head_map, False)
    return int(lib().mesh_attn_tile_bwd_workspace_size(C.byref(a)))


def mesh_attn_tile_bwd(tiles: Sequence[BwdTile], scale: float, mask_mode: int = MA_MASK_NONE, head_map=None,
                       accumulate: bool = False, workspace=None, stream=None) -> None:
    """dQ, dK, dV of every tile (dK/dV summed over tiles sharing a KV buffer), enqueued on `stream`.

    `workspace` is a device uint8 tensor of at least mesh_attn_tile_bwd_workspace_size bytes; when None
    one is allocated here through torch (the library itself never allocates)."""
    prepared = prepare_tile_bwd(tiles, scale, mask_mode, head_map, accumulate)
    if prepared is None:
        return
    if workspace is None:
        workspace = _torch().empty(max(prepared[2], 256), dtype=_torch().uint8, device=tiles[0].q.device)
    launch_prepared_tile_bwd(prepared, workspace, stream)


def prepare_tile_bwd(tiles: Sequence[BwdTile], scale: float, mask_mode: int = MA_MASK_NONE, head_map=None,
                     accumulate: bool = False):
    """The checked argument block of mesh_attn_tile_bwd and its workspace size in bytes, to be launched
    (possibly many times) by launch_prepared_tile_bwd; it holds the tensors' addresses, so keep the
    tensors alive.  None for an empty tile list."""
    tiles = list(tiles)
    if not tiles:
        return None
    a, keep = _bwd_args(tiles, scale, mask_mode, head_map, accumulate)
    return a, keep, int(lib().mesh_attn_tile_bwd_workspace_size(C.byref(a)))


def launch_prepared_tile_bwd(prepared, workspace, stream=None) -> None:
    """Enqueue a backward prepared by prepare_tile_bwd with `workspace`, a device uint8 tensor of at
    least prepared[2] bytes (the C call and these two checks only)."""
    if prepared is None:
        return
    a, _, need = prepared
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need or not workspace.is_cuda:
        raise ValueError(f"workspace must be a device buffer of >= {need} bytes")
    _abi.check(lib().mesh_attn_tile_bwd(C.byref(a), C.c_void_p(workspace.data_ptr()), nbytes, _stream_ptr(stream)),
               "mesh_attn_tile_bwd")


def mesh_attn_tile_bwd_noalloc(tiles: Sequence[BwdTile], scale: float, mask_mode: int = MA_MASK_NONE, head_map=None,
                               accumulate: bool = False, stream=None) -> None:
    """mesh_attn_tile_bwd with the library's built-in scratch as the workspace: no device memory is
    allocated (here or in the library).  Calls that overlap on one GPU race on that scratch."""
    tiles = list(tiles)
    if not tiles:
        return
    a, keep = _bwd_args(tiles, scale, mask_mode, head_map, accumulate)
    _abi.check(lib().mesh_attn_tile_bwd_noalloc(C.byref(a), _stream_ptr(stream)), "mesh_attn_tile_bwd_noalloc")


# ----------------------------------------------------------------- mapper --

def mesh_attn_map_mesh_tile(n: int, a: int, b: int, g: int, kvr: bool = True):
    q = (C.c_int32 * max(a, 1))()
    kv = (C.c_int32 * max(b, 1))()
    _abi.check(lib().mesh_attn_map_mesh_tile(n, a, b, g, int(kvr), q, kv), "mesh_attn_map_mesh_tile")
    return list(q)[:a], list(kv)[:b]


def mesh_attn_map_groups(n: int, a: int, b: int, g: int):
    q = (C.c_int32 * max(a, 1))()
    kv = (C.c_int32 * max(b, 1))()
    _abi.check(lib().mesh_attn_map_groups(n, a, b, g, q, kv), "mesh_attn_map_groups")
    return list(q)[:a], list(kv)[:b]


def mesh_attn_map_zigzag(N: int, r: int):
    out = (C.c_int32 * 2)()
    _abi.check(lib().mesh_attn_map_zigzag(N, r, out), "mesh_attn_map_zigzag")
    return tuple(out)


def mesh_attn_pos_contiguous(global_begin: int) -> Pos:
    p = _abi.ma_pos()
    _abi.check(lib().mesh_attn_pos_contiguous(global_begin, C.byref(p)), "mesh_attn_pos_contiguous")
    return Pos.from_c(p)


def mesh_attn_pos_zigzag(N: int, r: int, chunk_len: int) -> Pos:
    p = _abi.ma_pos()
    _abi.check(lib().mesh_attn_pos_zigzag(N, r, chunk_len, C.byref(p)), "mesh_attn_pos_zigzag")
    return Pos.from_c(p)


def mesh_attn_pos_striped(N: int, r: int) -> Pos:
    p = _abi.ma_pos()
    _abi.check(lib().mesh_attn_pos_striped(N, r, C.byref(p)), "mesh_attn_pos_striped")
    return Pos.from_c(p)


def mesh_attn_pos_at(pos: Pos, t: int) -> int:
    p = pos.to_c()
    return int(lib().mesh_attn_pos_at(C.byref(p), t))


def mesh_attn_classify(q_pos: Pos, sq: int, k_pos: Pos, sk: int, mask_mode: int) -> int:
    qp, kp = _pos_c(q_pos), _pos_c(k_pos)
    r = int(lib().mesh_attn_classify(C.byref(qp), sq, C.byref(kp), sk, int(mask_mode)))
    if r < 0:
        raise MeshAttnError(-r, "mesh_attn_classify")
    return r


def mesh_attn_count_allowed(q_pos: Pos, sq: int, k_pos: Pos, sk: int, mask_mode: int) -> int:
    qp, kp = _pos_c(q_pos), _pos_c(k_pos)
    r = int(lib().mesh_attn_count_allowed(C.byref(qp), sq, C.byref(kp), sk, int(mask_mode)))
    if r < 0:
        raise MeshAttnError(MA_ERR_INVALID, "mesh_attn_count_allowed")
    return r


def mesh_attn_build_worklist(q_pos: Sequence[Pos], sq: Sequence[int], k_pos: Sequence[Pos], sk: Sequence[int],
                             mask_mode: int):
    nq, nk = len(q_pos), len(k_pos)
    qa = (_abi.ma_pos * max(nq, 1))(*[p.to_c() for p in q_pos])
    ka = (_abi.ma_pos * max(nk, 1))(*[p.to_c() for p in k_pos])
    sqa = (C.c_int64 * max(nq, 1))(*sq)
    ska = (C.c_int64 * max(nk, 1))(*sk)
    cap = max(nq * nk, 1)
    oq, ok_, oc = (C.c_int32 * cap)(), (C.c_int32 * cap)(), (C.c_int32 * cap)()
    n = int(lib().mesh_attn_build_worklist(nq, qa, sqa, nk, ka, ska, int(mask_mode), cap, oq, ok_, oc))
    if n < 0:
        raise MeshAttnError(MA_ERR_INVALID, "mesh_attn_build_worklist")
    return [(oq[i], ok_[i], oc[i]) for i in range(n)]


def mesh_attn_version() -> int:
    return int(lib().mesh_attn_version())


# -------------------------------------------------------------- GOO plan --

_GOO_NAMES = {1: "AG-Q", 2: "AG-KV", 3: "RS-Q"}


def mesh_attn_goo_plan(k_q: int, k_kv: int, t_ag_q: float, t_ag_kv: float, t_rs_q: float, t_c, gamma: float):
    """Greedy GOO schedule: a list of steps (comm task or None, [("C", i, j), ...]); a comm task is
    ("AG-Q", i), ("AG-KV", j) or ("RS-Q", i).  t_c: one compute time or a k_q x k_kv nested list."""
    n = int(k_q) * int(k_kv)
    if isinstance(t_c, (list, tuple)):
        flat = [float(x) for row in t_c for x in row]
    else:
        flat = [float(t_c)] * max(n, 0)
    tc = (C.c_double * max(1, len(flat)))(*flat)
    cap = max(1, 2 * int(k_q) + int(k_kv) + max(n, 0))
    steps = (_abi.ma_goo_step * cap)()
    r = lib().mesh_attn_goo_plan(int(k_q), int(k_kv), float(t_ag_q), float(t_ag_kv), float(t_rs_q), tc,
                                 float(gamma), cap, steps)
    if r < 0:
        raise MeshAttnError(-r, "mesh_attn_goo_plan")
    out = []
    for s in steps[:r]:
        comm = None if s.comm_type == 0 else (_GOO_NAMES[s.comm_type], s.comm_index)
        out.append((comm, [("C", c // k_kv, c % k_kv) for c in s.compute[:s.ncompute]]))
    return out
