"""Helpers for GPU parity tests: move seeded synthetic inputs to the device and back.

Inputs come from ``synthetic`` (seeded N(0,1), stored as bf16 bits or fp32); the
oracle reads the very same stored values, upcast exactly to float64.
"""
import math
import sys

import numpy as np
import torch

import synthetic
from oracle import layout

DEV = "cuda:0"

# tolerances for the forward and merge, max abs error
BF16_O_TOL, BF16_LSE_TOL = 2e-2, 1e-3
F32_TOL = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the device."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def gen(workload, tensor, part, shape, dtype="bf16"):
    """(device tensor, exact float64 values) of a seeded N(0,1) draw."""
    if dtype == "bf16":
        bits, vals = synthetic.normal_bf16(workload, tensor, part, shape)
        return dev_bf16(bits), vals.astype(np.float64)
    vals = synthetic.normal_f32(workload, tensor, part, shape)
    return dev_f32(vals), vals.astype(np.float64)


def positions(pos, length):
    """Oracle-side expansion of a binding Pos (segments) into int64 positions."""
    return layout.expand_positions(pos.segments, length)


def check_close(name, got, ref, tol, normalised_also=True):
    """Max-abs error within tol; -inf entries must match exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), f"{name}: -inf pattern differs"
    assert not np.isnan(got).any(), f"{name}: NaN in result"
    fin = ~ninf_ref
    err = float(np.max(np.abs(got[fin] - ref[fin]), initial=0.0))
    scale = float(np.max(np.abs(ref[fin]), initial=0.0))
    log(f"  {name}: max_abs_err={err:.3e} (tol {tol:.1e}) max|ref|={scale:.3e}")
    assert err <= tol, f"{name}: max abs error {err} > {tol}"
    if normalised_also and scale > 0:
        assert err / scale <= max(tol, 2e-2), f"{name}: normalised error {err/scale} too large"
    return err


def oracle_forward_by_head(q, k, v, scale, threads=16):
    """The oracle forward (non-causal, default GQA map) of every query row, one query head per task.

    Each task calls oracle.attn_tile on one query head and its KV head (a [B, S, 1, d] slice of
    each), so the arithmetic is the oracle's own; the tasks only run side by side (NumPy releases
    the GIL inside its kernels).  Returns (O [B, Sq, Hq, d], LSE [B, Hq, Sq]) in float64."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attn_tile

    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, Sq, Hq, d))
    L = np.zeros((B, Hq, Sq))

    def one(h):
        kv = h // g
        Oh, Lh = attn_tile(q[:, :, h:h + 1], k[:, :, kv:kv + 1], v[:, :, kv:kv + 1], scale)
        O[:, :, h:h + 1] = Oh
        L[:, h:h + 1] = Lh

    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(Hq)))
    return O, L
