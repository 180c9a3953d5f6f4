"""ctypes mirror of include/mesh_attn.h and the loader of libmesh_attn.so.

Only marshalling lives here; every step of the path runs in the HIP library.
The loader fails loudly when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmesh_attn.so")

MA_OK, MA_ERR_INVALID, MA_ERR_UNSUPPORTED, MA_ERR_LAUNCH = 0, 1, 2, 3
MA_F32, MA_BF16 = 0, 1
MA_MASK_NONE, MA_MASK_CAUSAL, MA_MASK_STRIPED_ZIGZAG = 0, 1, 2
MA_TILE_EMPTY, MA_TILE_PARTIAL, MA_TILE_FULL = 0, 1, 2
MA_MAX_SEGMENTS, MA_MAX_MERGE, MA_MAX_HEADS, MA_MAX_TILES = 4, 64, 128, 4096
MA_BWD_NOALLOC_MAX_WORKSPACE = 32 << 20

I32, I64, F32 = C.c_int32, C.c_int64, C.c_float
VP = C.c_void_p


class ma_segment(C.Structure):
    _fields_ = [("local_begin", I64), ("global_begin", I64), ("stride", I64)]


class ma_pos(C.Structure):
    _fields_ = [("nseg", I32), ("reserved", I32), ("seg", ma_segment * MA_MAX_SEGMENTS)]


class ma_tile(C.Structure):
    _fields_ = [("q", VP), ("k", VP), ("v", VP), ("o", VP), ("lse", VP), ("sq", I64), ("sk", I64),
                ("q_pos", ma_pos), ("k_pos", ma_pos)]


class ma_tile_fwd_args(C.Structure):
    _fields_ = [("dtype", I32), ("batch", I32), ("hq", I32), ("hkv", I32), ("head_dim", I32), ("mask_mode", I32),
                ("scale", F32), ("ntiles", I32), ("accumulate", I32), ("reserved", I32),
                ("head_map", C.POINTER(I32)), ("tiles", C.POINTER(ma_tile)),
                ("q_stride", I64 * 3), ("k_stride", I64 * 3), ("v_stride", I64 * 3), ("o_stride", I64 * 3),
                ("lse_stride", I64 * 2)]


class ma_merge_args(C.Structure):
    _fields_ = [("dtype", I32), ("batch", I32), ("seqlen", I32), ("heads", I32), ("head_dim", I32), ("k", I32),
                ("o_in", C.POINTER(VP)), ("lse_in", C.POINTER(VP)), ("o_out", VP), ("lse_out", VP),
                ("o_stride", I64 * 3), ("lse_stride", I64 * 2)]


class ma_reduce_args(C.Structure):
    _fields_ = [("k", I32), ("reserved", I32), ("n", I64), ("in_", C.POINTER(VP)), ("out", VP)]


MA_GOO_MAX_COMPUTE = 16


class ma_goo_step(C.Structure):
    _fields_ = [("comm_type", I32), ("comm_index", I32), ("ncompute", I32), ("compute", I32 * MA_GOO_MAX_COMPUTE)]


class ma_bwd_tile(C.Structure):
    _fields_ = [("q", VP), ("k", VP), ("v", VP), ("o", VP), ("dout", VP), ("lse", VP), ("dq", VP), ("dk", VP),
                ("dv", VP), ("sq", I64), ("sk", I64), ("q_pos", ma_pos), ("k_pos", ma_pos)]


class ma_tile_bwd_args(C.Structure):
    _fields_ = [("dtype", I32), ("batch", I32), ("hq", I32), ("hkv", I32), ("head_dim", I32), ("mask_mode", I32),
                ("scale", F32), ("ntiles", I32), ("accumulate", I32), ("reserved", I32),
                ("head_map", C.POINTER(I32)), ("tiles", C.POINTER(ma_bwd_tile)),
                ("q_stride", I64 * 3), ("k_stride", I64 * 3), ("dq_stride", I64 * 3), ("dk_stride", I64 * 3),
                ("lse_stride", I64 * 2)]


# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "mesh_attn_tile_fwd": (I32, [C.POINTER(ma_tile_fwd_args), VP]),
    "mesh_attn_tile_fwd_table_bytes": (C.c_size_t, [C.POINTER(ma_tile_fwd_args)]),
    "mesh_attn_tile_fwd_pack": (I32, [C.POINTER(ma_tile_fwd_args), VP, C.c_size_t]),
    "mesh_attn_tile_fwd_tabled": (I32, [C.POINTER(ma_tile_fwd_args), VP, C.c_size_t, VP]),
    "mesh_attn_merge": (I32, [C.POINTER(ma_merge_args), VP]),
    "mesh_attn_reduce_add": (I32, [C.POINTER(ma_reduce_args), VP]),
    "mesh_attn_goo_plan": (I32, [I32, I32, C.c_double, C.c_double, C.c_double, C.POINTER(C.c_double), C.c_double,
                                 I32, C.POINTER(ma_goo_step)]),
    "mesh_attn_tile_bwd_workspace_size": (C.c_size_t, [C.POINTER(ma_tile_bwd_args)]),
    "mesh_attn_tile_bwd": (I32, [C.POINTER(ma_tile_bwd_args), VP, C.c_size_t, VP]),
    "mesh_attn_tile_bwd_noalloc": (I32, [C.POINTER(ma_tile_bwd_args), VP]),
    "mesh_attn_map_mesh_tile": (I32, [I32, I32, I32, I32, I32, C.POINTER(I32), C.POINTER(I32)]),
    "mesh_attn_map_groups": (I32, [I32, I32, I32, I32, C.POINTER(I32), C.POINTER(I32)]),
    "mesh_attn_map_zigzag": (I32, [I32, I32, C.POINTER(I32)]),
    "mesh_attn_pos_contiguous": (I32, [I64, C.POINTER(ma_pos)]),
    "mesh_attn_pos_zigzag": (I32, [I32, I32, I64, C.POINTER(ma_pos)]),
    "mesh_attn_pos_striped": (I32, [I32, I32, C.POINTER(ma_pos)]),
    "mesh_attn_pos_at": (I64, [C.POINTER(ma_pos), I64]),
    "mesh_attn_classify": (I32, [C.POINTER(ma_pos), I64, C.POINTER(ma_pos), I64, I32]),
    "mesh_attn_count_allowed": (I64, [C.POINTER(ma_pos), I64, C.POINTER(ma_pos), I64, I32]),
    "mesh_attn_build_worklist": (I32, [I32, C.POINTER(ma_pos), C.POINTER(I64), I32, C.POINTER(ma_pos),
                                       C.POINTER(I64), I32, I32, C.POINTER(I32), C.POINTER(I32), C.POINTER(I32)]),
    "mesh_attn_last_error": (C.c_char_p, []),
    "mesh_attn_version": (I32, []),
}

_lib = None


def lib():
    """Load libmesh_attn.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m distributed_long_context_amd.build` "
                "(hipcc, gfx950). There is no fallback path.")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class MeshAttnError(RuntimeError):
    def __init__(self, code, where):
        msg = lib().mesh_attn_last_error().decode(errors="replace")
        super().__init__(f"{where} failed with code {code}: {msg}")
        self.code = code


def check(code, where):
    if code != MA_OK:
        raise MeshAttnError(code, where)
