"""The backward entry point that allocates nothing (mesh_attn_tile_bwd_noalloc) against the backward
with a caller workspace (mesh_attn_tile_bwd): the same kernels on the same inputs, so dQ, dK and dV
must be bitwise equal.  Two calls in a row share the built-in scratch, the second with a smaller
input (its LSE/D slices land where the first call's were), and the smaller call is checked against
its own reference too; the first call also goes through the fp64 oracle.  A HIP graph captures the
entry point and replays it."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import BwdTile, Pos  # noqa: E402
from oracle import attn_tile, attn_tile_bwd  # noqa: E402
from gpu_helpers import DEV, gen, log, positions  # noqa: E402
from test_gpu_bwd import check_grad, stored_o_lse  # noqa: E402

import synthetic  # noqa: E402


def _case(wid, sq, sk, hq, hkv, d, nq, mode, qps, kp):
    """Tiles of nq Q partitions against one KV partition, twice: outputs for the reference call and
    for the no-allocation call, NaN-filled so that an unwritten element shows."""
    causal = mode != ma.MA_MASK_NONE
    scale = np.float32(1.0 / math.sqrt(d))
    k, kv = gen(wid, synthetic.T_K, 0, (1, sk, hkv, d))
    v, vv = gen(wid, synthetic.T_V, 0, (1, sk, hkv, d))
    kpos = positions(kp, sk) if causal else None
    ins, host = [], []
    for i in range(nq):
        q, qv = gen(wid, synthetic.T_Q, i, (1, sq, hq, d))
        do, dov = gen(wid, synthetic.T_DO, i, (1, sq, hq, d))
        qpos = positions(qps[i], sq) if causal else None
        O, L = attn_tile(qv, kv, vv, scale, None, causal, qpos, kpos)
        o_dev, o_used, l_dev, l_used = stored_o_lse(O, L)
        ins.append((q, o_dev, do, l_dev))
        host.append(dict(q=qv, o=o_used, do=dov, lse=l_used, q_pos=qpos))
    outs = []
    for _ in range(2):
        dk = torch.full((1, sk, hkv, d), float("nan"), dtype=torch.float32, device=DEV)
        dv = torch.full_like(dk, float("nan"))
        dqs = [torch.full((1, sq, hq, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(nq)]
        tiles = [BwdTile(q, k, v, o, do, l, dq, dk, dv, qps[i], kp) for i, ((q, o, do, l), dq) in
                 enumerate(zip(ins, dqs))]
        outs.append((tiles, dqs, dk, dv))
    return scale, outs, (kv, vv, kpos, host)


def _same(name, a, b):
    assert torch.equal(a, b), f"{name}: the no-allocation backward differs from the workspace backward"


def test_noalloc_backward_matches_workspace_backward_twice():
    # call 1: two causal Q partitions of 2000 rows against 2500 keys, 8/2 heads, d = 128
    qps1 = [Pos([(0, 3000, 1)]), Pos([(0, 1000, 1)])]
    kp1 = Pos([(0, 0, 1)])
    log("[no-alloc bwd] call 1: 2 x 2000 rows vs 2500 keys, causal, 8/2 heads, d=128")
    s1, (ref1, new1), (kv1, vv1, kpos1, host1) = _case(2900, 2000, 2500, 8, 2, 128, 2, ma.MA_MASK_CAUSAL, qps1, kp1)
    need1 = ma.mesh_attn_tile_bwd_workspace_size(ref1[0], float(s1), ma.MA_MASK_CAUSAL)
    assert 0 < need1 <= ma._abi.MA_BWD_NOALLOC_MAX_WORKSPACE
    # call 2: one smaller non-causal partition, 4/4 heads, d = 64
    log("[no-alloc bwd] call 2: 300 rows vs 500 keys, no mask, 4/4 heads, d=64")
    s2, (ref2, new2), _ = _case(2901, 300, 500, 4, 4, 64, 1, ma.MA_MASK_NONE, [None], None)
    need2 = ma.mesh_attn_tile_bwd_workspace_size(ref2[0], float(s2), ma.MA_MASK_NONE)
    assert 0 < need2 < need1

    ma.mesh_attn_tile_bwd(ref1[0], float(s1), ma.MA_MASK_CAUSAL)
    ma.mesh_attn_tile_bwd(ref2[0], float(s2), ma.MA_MASK_NONE)
    ma.mesh_attn_tile_bwd_noalloc(new1[0], float(s1), ma.MA_MASK_CAUSAL)
    ma.mesh_attn_tile_bwd_noalloc(new2[0], float(s2), ma.MA_MASK_NONE)
    torch.cuda.synchronize()
    for call, (ref, new) in enumerate(((ref1, new1), (ref2, new2)), 1):
        for i, (a, b) in enumerate(zip(ref[1], new[1])):
            _same(f"call {call} dQ{i}", a, b)
        _same(f"call {call} dK", ref[2], new[2])
        _same(f"call {call} dV", ref[3], new[3])
        assert not torch.isnan(new[2]).any() and not torch.isnan(new[3]).any()
    # the first call against the oracle as well
    dk_ref = dv_ref = 0
    for i, h in enumerate(host1):
        dq_r, dk_r, dv_r = attn_tile_bwd(h["q"], kv1, vv1, h["o"], h["do"], h["lse"], s1, None, True, h["q_pos"],
                                         kpos1)
        check_grad(f"dQ{i}", new1[1][i], dq_r)
        dk_ref = dk_ref + dk_r
        dv_ref = dv_ref + dv_r
    check_grad("dK", new1[2], dk_ref)
    check_grad("dV", new1[3], dv_ref)


def test_noalloc_backward_replays_under_graph_capture():
    """The caller the entry point is for: a HIP graph captures the no-allocation backward once (no
    allocation, no memset node) and replays it three times, with eager work and synchronisation
    between the replays; every replay must equal the eager call bitwise."""
    qps = [Pos([(0, 900, 1)])]
    kp = Pos([(0, 0, 1)])
    log("[no-alloc bwd] graph capture: 700 rows vs 900 keys, causal, 8/2 heads, d=128, 3 replays")
    s, (ref, new), _ = _case(2902, 700, 900, 8, 2, 128, 1, ma.MA_MASK_CAUSAL, qps, kp)
    ma.mesh_attn_tile_bwd_noalloc(ref[0], float(s), ma.MA_MASK_CAUSAL)
    ma.mesh_attn_tile_bwd_noalloc(new[0], float(s), ma.MA_MASK_CAUSAL)  # warm-up before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ma.mesh_attn_tile_bwd_noalloc(new[0], float(s), ma.MA_MASK_CAUSAL)
    torch.cuda.synchronize()
    for r in range(3):
        for t in new[1] + [new[2], new[3]]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(f"replay {r} dQ", ref[1][0], new[1][0])
        _same(f"replay {r} dK", ref[2], new[2])
        _same(f"replay {r} dV", ref[3], new[3])
