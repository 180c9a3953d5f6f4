"""The C-ABI library loads, exports every declared symbol, and validates arguments on the host (CPU only)."""
import ctypes as C
import os
import re

import pytest

from distributed_long_context_amd import _abi

HEADER_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(mesh_attn_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
        assert n in _abi.SIGNATURES, f"binding lacks {n}"
    assert L.mesh_attn_version() == 1


def _fwd_args(**kw):
    a = _abi.ma_tile_fwd_args()
    a.dtype, a.batch, a.hq, a.hkv, a.head_dim, a.mask_mode = _abi.MA_BF16, 1, 4, 2, 128, 0
    a.scale, a.ntiles = 0.1, 0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), _abi.MA_ERR_UNSUPPORTED),
    (dict(dtype=7), _abi.MA_ERR_INVALID),
    (dict(hq=3, hkv=2), _abi.MA_ERR_INVALID),
    (dict(hq=200, hkv=2), _abi.MA_ERR_INVALID),
    (dict(mask_mode=9), _abi.MA_ERR_INVALID),
    (dict(scale=0.0), _abi.MA_ERR_INVALID),
    (dict(scale=float("nan")), _abi.MA_ERR_INVALID),
    (dict(ntiles=1), _abi.MA_ERR_INVALID),  # null tile list
    (dict(ntiles=-1), _abi.MA_ERR_INVALID),
    (dict(accumulate=2), _abi.MA_ERR_INVALID),
])
def test_tile_fwd_rejects_bad_arguments(kw, code):
    a = _fwd_args(**kw)
    assert _abi.lib().mesh_attn_tile_fwd(C.byref(a), None) == code
    assert len(_abi.lib().mesh_attn_last_error()) > 0


def test_tile_fwd_rejects_bad_tiles_without_launching():
    L = _abi.lib()
    t = (_abi.ma_tile * 1)()
    a = _fwd_args(ntiles=1)
    a.tiles = C.cast(t, C.POINTER(_abi.ma_tile))
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID  # null pointers
    t[0].q = t[0].k = t[0].v = t[0].o = 4096
    t[0].lse = 4096
    t[0].sq, t[0].sk = 0, 5
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID  # sq = 0
    t[0].sq = 5
    t[0].q = 4100
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID  # misaligned
    t[0].q = 4096
    a.mask_mode = _abi.MA_MASK_CAUSAL
    t[0].q_pos.nseg = 2  # causal needs a single stride-1 segment
    t[0].q_pos.seg[1].local_begin = 2
    t[0].k_pos.nseg = 1
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID
    t[0].q_pos.nseg = 5
    a.mask_mode = _abi.MA_MASK_STRIPED_ZIGZAG
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID  # too many segments
    a.head_map = C.cast((C.c_int32 * 4)(0, 1, 2, 0), C.POINTER(C.c_int32))
    t[0].q_pos.nseg = 1
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID  # head_map entry 2 >= hkv


def test_merge_rejects_bad_arguments():
    L = _abi.lib()
    a = _abi.ma_merge_args()
    a.dtype, a.batch, a.seqlen, a.heads, a.head_dim, a.k = _abi.MA_BF16, 1, 8, 2, 128, 0
    assert L.mesh_attn_merge(C.byref(a), None) == _abi.MA_ERR_INVALID  # k = 0
    a.k = _abi.MA_MAX_MERGE + 1
    assert L.mesh_attn_merge(C.byref(a), None) == _abi.MA_ERR_INVALID  # k > 64
    a.k, a.head_dim = 2, 80
    assert L.mesh_attn_merge(C.byref(a), None) == _abi.MA_ERR_UNSUPPORTED
    a.head_dim = 128
    assert L.mesh_attn_merge(C.byref(a), None) == _abi.MA_ERR_INVALID  # null pointers


def test_bwd_rejects_bad_arguments():
    L = _abi.lib()
    a = _abi.ma_tile_bwd_args()
    a.dtype, a.batch, a.hq, a.hkv, a.head_dim, a.scale = _abi.MA_F32, 1, 2, 1, 128, 0.1
    assert L.mesh_attn_tile_bwd(C.byref(a), None, 0, None) in (_abi.MA_ERR_UNSUPPORTED, _abi.MA_ERR_INVALID)
    assert L.mesh_attn_tile_bwd(None, None, 0, None) == _abi.MA_ERR_INVALID


def test_null_args():
    L = _abi.lib()
    assert L.mesh_attn_tile_fwd(None, None) == _abi.MA_ERR_INVALID
    assert L.mesh_attn_merge(None, None) == _abi.MA_ERR_INVALID


def test_reduce_add_rejects_bad_arguments_without_launching():
    L = _abi.lib()
    ptrs = (C.c_void_p * 2)(4096, 4096)
    a = _abi.ma_reduce_args()
    a.k, a.n, a.out = 2, 16, 4096
    a.in_ = C.cast(ptrs, C.POINTER(C.c_void_p))
    for k in (0, _abi.MA_MAX_MERGE + 1):
        a.k = k
        assert L.mesh_attn_reduce_add(C.byref(a), None) == _abi.MA_ERR_INVALID
    a.k = 2
    a.n = -1
    assert L.mesh_attn_reduce_add(C.byref(a), None) == _abi.MA_ERR_INVALID
    a.n = 16
    a.out = 4100  # not 16-byte aligned
    assert L.mesh_attn_reduce_add(C.byref(a), None) == _abi.MA_ERR_INVALID
    a.out = 4096
    ptrs[1] = 4104
    assert L.mesh_attn_reduce_add(C.byref(a), None) == _abi.MA_ERR_INVALID
    ptrs[1] = None
    assert L.mesh_attn_reduce_add(C.byref(a), None) == _abi.MA_ERR_INVALID
    a.n = 0  # no-op before any pointer is looked at
    assert L.mesh_attn_reduce_add(C.byref(a), None) == _abi.MA_OK


def test_bwd_workspace_counts_one_segment_pieces():
    # Under a mask a two-segment Q partition runs as one piece per segment, each with its own
    # blocked LSE/D slice of ceil(rows / 64) blocks x 2 x 64 floats per (batch, head).
    L = _abi.lib()
    B, hq, sq = 2, 4, 130
    t = (_abi.ma_bwd_tile * 1)()
    t[0].sq, t[0].sk = sq, 96
    t[0].q_pos.nseg = 2
    t[0].q_pos.seg[0].local_begin, t[0].q_pos.seg[0].global_begin, t[0].q_pos.seg[0].stride = 0, 0, 1
    t[0].q_pos.seg[1].local_begin, t[0].q_pos.seg[1].global_begin, t[0].q_pos.seg[1].stride = 65, 1000, 1
    t[0].k_pos.nseg = 1
    t[0].k_pos.seg[0].stride = 1
    t[0].dq, t[0].dk, t[0].dv = 4096, 8192, 12288
    a = _abi.ma_tile_bwd_args()
    a.dtype, a.batch, a.hq, a.hkv, a.head_dim, a.scale, a.ntiles = _abi.MA_BF16, B, hq, 2, 128, 0.1, 1
    a.tiles = C.cast(t, C.POINTER(_abi.ma_bwd_tile))
    a.q_stride[:] = (sq * hq * 128, hq * 128, 128)
    a.dq_stride[:] = (sq * hq * 128, hq * 128, 128)

    def blocked(rows):
        return (B * hq * ((rows + 63) // 64) * 2 * 64 * 4 + 255) // 256 * 256

    a.mask_mode = _abi.MA_MASK_NONE  # positions unused: one piece
    assert L.mesh_attn_tile_bwd_workspace_size(C.byref(a)) == blocked(130)
    a.mask_mode = _abi.MA_MASK_STRIPED_ZIGZAG  # two pieces of 65 rows
    assert L.mesh_attn_tile_bwd_workspace_size(C.byref(a)) == 2 * blocked(65)


def _tile_arr(n, sq=64, sk=64, base=1 << 20, step=1 << 24):
    t = (_abi.ma_tile * n)()
    for i in range(n):
        b = base + i * step
        t[i].q, t[i].k, t[i].v, t[i].o, t[i].lse = b, b + 4096, b + 8192, b + 12288, b + 16384
        t[i].sq, t[i].sk = sq, sk
        t[i].q_pos.nseg = t[i].k_pos.nseg = 1
        t[i].q_pos.seg[0].stride = t[i].k_pos.seg[0].stride = 1
    return t


def test_tile_fwd_rejects_shifted_outputs_without_launching():
    # two tiles whose O is one buffer shifted by 10 rows (fewer than the 64 it holds): rejected
    L = _abi.lib()
    t = _tile_arr(2)
    a = _fwd_args(ntiles=2, hq=4, hkv=2)
    a.tiles = C.cast(t, C.POINTER(_abi.ma_tile))
    row = 4 * 128  # o_stride[1] in elements (hq * d)
    a.q_stride[:] = a.o_stride[:] = (64 * row, row, 128)
    a.k_stride[:] = a.v_stride[:] = (64 * 256, 256, 128)
    a.lse_stride[:] = (4 * 64, 64)
    t[1].o = t[0].o + 10 * row * 2
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID
    assert b"overlap" in L.mesh_attn_last_error()
    # LSE shifted by 3 positions of 64
    t[1].o = t[0].o + 64 * row * 2 * 4
    t[1].lse = t[0].lse + 3 * 4
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID


def test_tile_fwd_is_planned_before_launching():
    # a valid tile, then one too large for a launch: the error comes from the plan, before the
    # first tile is enqueued (an enqueue on this host, which has no GPU, would report a launch error)
    L = _abi.lib()
    t = _tile_arr(2)
    a = _fwd_args(ntiles=2, hq=128, hkv=1, batch=2)
    a.tiles = C.cast(t, C.POINTER(_abi.ma_tile))
    row = 128 * 128
    a.q_stride[:] = a.o_stride[:] = (0, row, 128)
    a.k_stride[:] = a.v_stride[:] = (0, 128, 128)
    a.lse_stride[:] = (0, 0)
    t[1].sq = (1 << 31) - 2
    assert L.mesh_attn_tile_fwd(C.byref(a), None) == _abi.MA_ERR_INVALID
    assert b"too large" in L.mesh_attn_last_error()


def _bwd_tiles(n, sq=64, sk=64, base=1 << 20, step=1 << 26):
    t = (_abi.ma_bwd_tile * n)()
    for i in range(n):
        b = base + i * step
        (t[i].q, t[i].k, t[i].v, t[i].o, t[i].dout, t[i].lse, t[i].dq, t[i].dk, t[i].dv) = \
            [b + 65536 * j for j in range(9)]
        t[i].sq, t[i].sk = sq, sk
        t[i].q_pos.nseg = t[i].k_pos.nseg = 1
        t[i].q_pos.seg[0].stride = t[i].k_pos.seg[0].stride = 1
    return t


def _bwd_args_c(t, n, hq=4, hkv=2, mask=_abi.MA_MASK_NONE):
    a = _abi.ma_tile_bwd_args()
    a.dtype, a.batch, a.hq, a.hkv, a.head_dim, a.scale, a.ntiles = _abi.MA_BF16, 1, hq, hkv, 128, 0.1, n
    a.mask_mode = mask
    a.tiles = C.cast(t, C.POINTER(_abi.ma_bwd_tile))
    a.q_stride[:] = a.dq_stride[:] = (0, hq * 128, 128)
    a.k_stride[:] = a.dk_stride[:] = (0, hkv * 128, 128)
    a.lse_stride[:] = (0, 0)
    return a


def test_bwd_rejects_shifted_gradient_outputs():
    L = _abi.lib()
    t = _bwd_tiles(2)
    a = _bwd_args_c(t, 2)
    t[1].dq = t[0].dq + 5 * 4 * 128 * 4  # dq of tile 1 = dq of tile 0 shifted by 5 rows of 64
    assert L.mesh_attn_tile_bwd(C.byref(a), C.c_void_p(1 << 30), 1 << 20, None) == _abi.MA_ERR_INVALID
    assert b"overlap" in L.mesh_attn_last_error()
    assert L.mesh_attn_tile_bwd_noalloc(C.byref(a), None) == _abi.MA_ERR_INVALID


def test_bwd_tiles_sharing_an_output_must_share_its_description():
    # A zero-byte workspace: a call that passes every argument check stops at the workspace check,
    # before anything is enqueued, so "workspace" in the error means the tiles were accepted.
    L = _abi.lib()

    def outcome(t, n, mask=_abi.MA_MASK_NONE):
        a = _bwd_args_c(t, n, mask=mask)
        rc = L.mesh_attn_tile_bwd(C.byref(a), None, 0, None)
        assert rc == _abi.MA_ERR_INVALID
        return L.mesh_attn_last_error()

    def share_kv(t, i, j):
        t[i].k, t[i].v, t[i].dk, t[i].dv, t[i].sk = t[j].k, t[j].v, t[j].dk, t[j].dv, t[j].sk

    def share_q(t, i, j):
        t[i].q, t[i].o, t[i].dout, t[i].lse, t[i].dq, t[i].sq = t[j].q, t[j].o, t[j].dout, t[j].lse, t[j].dq, t[j].sq

    n = 6
    t = _bwd_tiles(n)
    share_kv(t, 3, 1)
    share_kv(t, 5, 1)
    share_q(t, 4, 0)
    share_q(t, 2, 0)
    assert b"workspace" in outcome(t, n)
    for field in ("k", "v", "sk"):  # a third tile on the same dk/dv with another KV description
        t = _bwd_tiles(n)
        share_kv(t, 3, 1)
        share_kv(t, 5, 1)
        setattr(t[5], field, getattr(t[5], field) + 128)
        assert b"dk/dv" in outcome(t, n), field
    t = _bwd_tiles(n)
    t[4].dv = t[2].dk  # one tile's dv is another's dk
    assert b"dk/dv" in outcome(t, n)
    t = _bwd_tiles(n)
    t[4].dk = t[2].dv
    assert b"dk/dv" in outcome(t, n)
    t = _bwd_tiles(n)
    t[4].dk = t[4].dv = t[2].dk = t[2].dv  # both name one buffer for dk and dv, with another k
    assert b"dk/dv" in outcome(t, n)
    t = _bwd_tiles(n)
    share_kv(t, 4, 2)
    t[4].dk, t[4].dv = t[4].dk, t[0].dv  # same dk, another dv
    assert b"dk/dv" in outcome(t, n)
    for field in ("q", "o", "dout", "lse", "sq"):
        t = _bwd_tiles(n)
        share_q(t, 4, 0)
        share_q(t, 2, 0)
        setattr(t[4], field, getattr(t[4], field) + (1 if field == "sq" else 256))
        assert b"same dq" in outcome(t, n), field
    # positions count only under a mask
    t = _bwd_tiles(n)
    share_q(t, 4, 0)
    share_kv(t, 5, 1)
    t[4].q_pos.seg[0].global_begin = 64
    t[5].k_pos.seg[0].global_begin = 64
    assert b"workspace" in outcome(t, n)
    assert b"same dq" in outcome(t, n, mask=_abi.MA_MASK_CAUSAL)
    t[4].q_pos.seg[0].global_begin = 0
    assert b"dk/dv" in outcome(t, n, mask=_abi.MA_MASK_CAUSAL)
    t[5].k_pos.seg[0].global_begin = 0
    assert b"workspace" in outcome(t, n, mask=_abi.MA_MASK_CAUSAL)


def test_bwd_workspace_size_rejects_bad_segments():
    # under a mask the segments are expanded: a position map with more than MA_MAX_SEGMENTS
    # segments (or a bad stride) gives 0 instead of being read past its end
    L = _abi.lib()
    t = _bwd_tiles(1)
    a = _bwd_args_c(t, 1, mask=_abi.MA_MASK_STRIPED_ZIGZAG)
    assert L.mesh_attn_tile_bwd_workspace_size(C.byref(a)) > 0
    t[0].q_pos.nseg = _abi.MA_MAX_SEGMENTS + 1
    assert L.mesh_attn_tile_bwd_workspace_size(C.byref(a)) == 0
    t[0].q_pos.nseg = 1
    t[0].k_pos.seg[0].stride = 0
    assert L.mesh_attn_tile_bwd_workspace_size(C.byref(a)) == 0


def test_bwd_noalloc_rejects_workspace_beyond_its_scratch():
    # 128 heads x 16448 rows x 8 bytes of LSE/D blocks = 16.8 MiB per Q partition: two partitions
    # need more than the 32 MiB built-in scratch, which is refused before anything runs
    L = _abi.lib()
    t = _bwd_tiles(2, sq=16448, sk=64, step=1 << 33)
    a = _bwd_args_c(t, 2, hq=128, hkv=8)
    need = L.mesh_attn_tile_bwd_workspace_size(C.byref(a))
    assert need > _abi.MA_BWD_NOALLOC_MAX_WORKSPACE
    assert L.mesh_attn_tile_bwd_noalloc(C.byref(a), None) == _abi.MA_ERR_INVALID
    assert b"scratch" in L.mesh_attn_last_error()
    assert L.mesh_attn_tile_bwd_noalloc(None, None) == _abi.MA_ERR_INVALID


def test_python_workspace_helper_needs_the_mask_mode():
    import inspect
    import distributed_long_context_amd as ma
    params = inspect.signature(ma.mesh_attn_tile_bwd_workspace_size).parameters
    assert params["mask_mode"].default is inspect.Parameter.empty
    assert params["scale"].default is inspect.Parameter.empty


def _table_case(n, sq=210, sk=210, hq=32, hkv=8):
    """n tiles of the resident-KV class (unmasked bf16, d = 128, 129-256 keys), fake device pointers
    (host-only calls never touch them)."""
    t = _tile_arr(n, sq, sk, step=1 << 26)
    a = _fwd_args(ntiles=n, hq=hq, hkv=hkv)
    a.tiles = C.cast(t, C.POINTER(_abi.ma_tile))
    row = hq * 128
    a.q_stride[:] = a.o_stride[:] = (sq * row, row, 128)
    a.k_stride[:] = a.v_stride[:] = (sk * hkv * 128, hkv * 128, 128)
    a.lse_stride[:] = (hq * sq, sq)
    return a, t


def _parse_table(buf):
    import struct
    magic, ntiles, nwgs, nents, h = struct.unpack_from("<IiiiQ", buf, 0)
    tiles = []
    for i in range(ntiles):
        off = 32 + 120 * i  # q, k, v, o, lse, sq, sk, wg_begin, chunks
        tiles.append(struct.unpack_from("<5Q4i", buf, off))
    off = 32 + 120 * ntiles
    ents = [struct.unpack_from("<2i", buf, off + 8 * i) for i in range(nents)]  # tile, first unit
    off += 8 * nents
    wgs = [struct.unpack_from("<4i", buf, off + 16 * i) for i in range(nwgs)]  # entry, unit range, b*hkv+h
    return magic, h, tiles, ents, wgs


def test_tile_table_layout():
    # 40 tiles of 210 x 210 at 32/8 heads, each with its own K/V: 7 row blocks x 4 heads = 28 units,
    # one group and one chunk per tile, one workgroup per KV head; a tile of 64 keys (ring kernel)
    # in the middle stays out of the table
    L = _abi.lib()
    a, t = _table_case(41)
    t[20].sk = 64
    n = L.mesh_attn_tile_fwd_table_bytes(C.byref(a))
    assert n == 32 + 40 * 120 + 40 * 8 + 320 * 16
    buf = (C.c_ubyte * n)()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), buf, n) == _abi.MA_OK
    magic, h, tiles, ents, wgs = _parse_table(bytes(buf))
    assert magic == 0x5441424D and len(tiles) == 40 and len(wgs) == 320
    resident = [i for i in range(41) if i != 20]
    for k, (i, e) in enumerate(zip(resident, tiles)):
        assert e[:5] == (t[i].q, t[i].k, t[i].v, t[i].o, t[i].lse)
        assert e[5:] == (210, 210, 0, 0)  # sq, sk; workgroups come from the records
    assert ents == [(k, 28 * k) for k in range(40)]
    assert wgs == [(w // 8, 28 * (w // 8), 28 * (w // 8) + 28, w % 8) for w in range(320)]
    # the hash follows the tiles: another output pointer, another hash
    t[3].o += 1 << 20
    buf2 = (C.c_ubyte * n)()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), buf2, n) == _abi.MA_OK
    assert _parse_table(bytes(buf2))[1] != h


def test_tile_table_groups_tiles_sharing_kv():
    # tiles 0, 2, 4 share one K/V of 210 keys and tiles 1, 3 another of 200; tile 5 has the first
    # K/V's pointers but 150 keys (a group of its own).  Groups in (K, V, length) order: [5],
    # [0, 2, 4], [1, 3]; units ceil(sq / 32) x 4 numbered on across the groups; chunks of 32 units
    # (small call), each naming the entry that holds its first unit
    L = _abi.lib()
    a, t = _table_case(6)
    ka, kb = t[0].k, t[0].k + (1 << 30)
    for i, (sq, sk, k) in enumerate([(210, 210, ka), (37, 200, kb), (300, 210, ka), (64, 200, kb), (1, 210, ka),
                                     (129, 150, ka)]):
        t[i].sq, t[i].sk, t[i].k, t[i].v = sq, sk, k, k + (1 << 29)
    n = L.mesh_attn_tile_fwd_table_bytes(C.byref(a))
    buf = (C.c_ubyte * n)()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), buf, n) == _abi.MA_OK
    _, _, tiles, ents, wgs = _parse_table(bytes(buf))
    assert len(tiles) == 6
    assert ents == [(5, 0), (0, 20), (2, 48), (4, 88), (1, 92), (3, 100)]
    chunks = [(0, 0, 20), (1, 20, 52), (2, 52, 84), (2, 84, 92), (4, 92, 108)]
    assert wgs == [(e, ub, ue, h) for e, ub, ue in chunks for h in range(8)]
    assert n == 32 + 6 * 120 + 6 * 8 + 40 * 16


def test_tile_table_chunk_size_grows_with_the_call():
    # two tiles of 65536 rows on one K/V: 2 x 8192 units at 8 KV heads give 64 units a workgroup
    # (about 2048 workgroups), the second tile's first chunk naming the second entry
    L = _abi.lib()
    a, t = _table_case(2, sq=65536)
    t[1].k, t[1].v = t[0].k, t[0].v
    t[1].o, t[1].lse = t[0].o + (1 << 34), t[0].lse + (1 << 34)  # 512 MiB of O per tile: no overlap
    n = L.mesh_attn_tile_fwd_table_bytes(C.byref(a))
    buf = (C.c_ubyte * n)()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), buf, n) == _abi.MA_OK
    _, _, _, ents, wgs = _parse_table(bytes(buf))
    assert ents == [(0, 0), (1, 8192)]
    assert len(wgs) == 256 * 8
    assert wgs[0] == (0, 0, 64, 0) and wgs[127 * 8 + 7] == (0, 8128, 8192, 7)
    assert wgs[128 * 8] == (1, 8192, 8256, 0) and wgs[-1] == (1, 16320, 16384, 7)


@pytest.mark.parametrize("d,sks,resident", [
    (128, [128, 129, 256, 257], [False, True, True, False]),  # 129-256 keys at d = 128
    (64, [1, 512, 513], [True, True, False]),                  # 1-512 keys at d = 64
])
def test_tile_table_takes_the_resident_class_only(d, sks, resident):
    # the table holds exactly the unmasked bf16 tiles of the resident-KV key range, in call order
    L = _abi.lib()
    n = len(sks)
    a, t = _table_case(n)
    a.head_dim = d
    row, krow = 32 * d, 8 * d
    a.q_stride[:] = a.o_stride[:] = (210 * row, row, d)
    a.k_stride[:] = a.v_stride[:] = (600 * krow, krow, d)
    for i, sk in enumerate(sks):
        t[i].sk = sk
    nb = L.mesh_attn_tile_fwd_table_bytes(C.byref(a))
    buf = (C.c_ubyte * nb)()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), buf, nb) == _abi.MA_OK
    _, _, tiles, ents, wgs = _parse_table(bytes(buf))
    assert [e[0] for e in tiles] == [t[i].q for i in range(n) if resident[i]]
    assert len(ents) == sum(resident)
    # fp32 tiles never use the resident-KV kernel: the table is its header
    a.dtype = _abi.MA_F32
    a.q_stride[:] = a.o_stride[:] = (210 * row, row, d)
    assert L.mesh_attn_tile_fwd_table_bytes(C.byref(a)) == 32


@pytest.mark.parametrize("seed", range(12))
def test_tile_table_covers_every_unit_once(seed):
    # Random calls: tiles of random lengths on a few shared K/V buffers, some outside the resident
    # class.  Whatever the grouping and chunking, the table must hold the resident tiles in call
    # order, number each group's units on from the previous group, and give every (batch, KV head)
    # each unit of every tile exactly once, in workgroups that stay inside one group and name the
    # entry holding their first unit.
    import numpy as np
    rng = np.random.default_rng(seed)
    L = _abi.lib()
    hq, hkv = [(32, 8), (8, 8), (16, 2), (4, 1)][seed % 4]
    batch = 1 + seed % 2
    gmax = hq // hkv
    n = int(rng.integers(1, 48))
    nkv = int(rng.integers(1, 6))
    a, t = _table_case(n, hq=hq, hkv=hkv)
    a.batch = batch
    smax = 700 if seed < 9 else 60000  # long tiles: chunks of up to 128 units
    row = hq * 128
    a.q_stride[:] = a.o_stride[:] = (smax * row, row, 128)
    a.k_stride[:] = a.v_stride[:] = (smax * hkv * 128, hkv * 128, 128)
    a.lse_stride[:] = (hq * smax, smax)
    kv_base = [(1 << 40) + j * (1 << 32) for j in range(nkv)]
    for i in range(n):
        j = int(rng.integers(nkv))
        t[i].k, t[i].v = kv_base[j], kv_base[j] + (1 << 31)
        t[i].sq = int(rng.integers(1, smax + 1))
        t[i].sk = int(rng.choice([64, 100, 129, 200, 210, 256, 257, 600])) if rng.random() < 0.3 else 210
        t[i].o, t[i].lse = (1 << 44) + i * (1 << 30), (1 << 45) + i * (1 << 30)
    nb = L.mesh_attn_tile_fwd_table_bytes(C.byref(a))
    assert nb >= 32
    buf = (C.c_ubyte * nb)()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), buf, nb) == _abi.MA_OK
    magic, _, tiles, ents, wgs = _parse_table(bytes(buf))
    assert magic == 0x5441424D
    resident = [i for i in range(n) if 128 < t[i].sk <= 256]
    assert [e[0] for e in tiles] == [t[i].q for i in resident]
    assert nb == 32 + 120 * len(tiles) + 8 * len(ents) + 16 * len(wgs)
    # entries: every table tile once, units numbered on without gaps, groups contiguous
    assert sorted(e[0] for e in ents) == list(range(len(tiles)))
    key = lambda e: (tiles[e[0]][1], tiles[e[0]][2], tiles[e[0]][6])  # k, v, sk
    unit = 0
    for k, e in enumerate(ents):
        assert e[1] == unit
        unit += (tiles[e[0]][5] + 31) // 32 * gmax
        if k and key(ents[k - 1]) != key(e):
            assert key(e) not in {key(x) for x in ents[:k]}, "a group split in two"
    total = unit
    group_end = {}
    for k, e in enumerate(ents):
        nxt = [x[1] for x in ents[k + 1:] if key(x) != key(e)]
        group_end[k] = nxt[0] if nxt else total
    # workgroups: per (batch, KV head) a partition of [0, total) into ranges of at most 128 units
    seen = {bk: [] for bk in range(batch * hkv)}
    for ent, ub, ue, bk in wgs:
        assert 0 <= bk < batch * hkv and 0 <= ub < ue <= ub + 128
        assert ents[ent][1] <= ub and (ent + 1 == len(ents) or ents[ent + 1][1] > ub)
        assert ue <= group_end[ent], "a workgroup crosses into another group"
        seen[bk].append((ub, ue))
    for bk, ranges in seen.items():
        ranges.sort()
        assert [r[0] for r in ranges] == [0] + [r[1] for r in ranges[:-1]], bk
        assert (ranges[-1][1] if ranges else 0) == total


def test_tile_table_calls_reject_bad_buffers_without_launching():
    L = _abi.lib()
    a, _ = _table_case(3)
    n = L.mesh_attn_tile_fwd_table_bytes(C.byref(a))
    small = (C.c_ubyte * (n - 1))()
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), small, n - 1) == _abi.MA_ERR_INVALID
    assert L.mesh_attn_tile_fwd_pack(C.byref(a), None, n) == _abi.MA_ERR_INVALID
    # a launch on this host (no GPU) would report MA_ERR_LAUNCH: these are refused before it
    assert L.mesh_attn_tile_fwd_tabled(C.byref(a), None, n, None) == _abi.MA_ERR_INVALID
    assert L.mesh_attn_tile_fwd_tabled(C.byref(a), 0x100008, n, None) == _abi.MA_ERR_INVALID
    assert L.mesh_attn_tile_fwd_tabled(C.byref(a), 0x100000, n - 1, None) == _abi.MA_ERR_INVALID
    bad = _fwd_args(head_dim=96, ntiles=1)
    assert L.mesh_attn_tile_fwd_table_bytes(C.byref(bad)) == 0
    empty = _fwd_args(ntiles=0)
    assert L.mesh_attn_tile_fwd_table_bytes(C.byref(empty)) == 32
    assert L.mesh_attn_tile_fwd_tabled(C.byref(empty), None, 0, None) == _abi.MA_OK
