"""GPU parity of the add-reduce of partial gradients, and of a backward split across two
holders of the same KV partition whose partial dK/dV are then added ([Mesh] section 3.5)."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import BwdTile  # noqa: E402
from oracle import attn_tile, attn_tile_bwd, reduce_add  # noqa: E402
from gpu_helpers import DEV, F32_TOL, check_close, gen, host_f64, log  # noqa: E402
from test_gpu_bwd import check_grad, stored_o_lse  # noqa: E402

import synthetic  # noqa: E402


@pytest.mark.parametrize("k,n", [(1, 4096), (2, 1 << 20), (3, 5), (4, 3), (8, 1000003), (9, 77), (17, 8195),
                                 (64, 4099)])
def test_reduce_add_matches_oracle(k, n):
    log(f"[reduce_add] k={k} n={n}")
    parts = [synthetic.normal_f32(1100 + k, synthetic.T_O_IN, r, (n,)) for r in range(k)]
    ins = [torch.from_numpy(p).to(DEV) for p in parts]
    out = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    ma.mesh_attn_reduce_add(ins, out)
    torch.cuda.synchronize()
    check_close("sum", host_f64(out), reduce_add(parts), F32_TOL, normalised_also=False)


def test_reduce_add_in_place_and_repeatable():
    log("[reduce_add in place]")
    k, n = 5, 300001
    parts = [synthetic.normal_f32(1200, synthetic.T_O_IN, r, (n,)) for r in range(k)]
    ins = [torch.from_numpy(p).to(DEV) for p in parts]
    out = torch.empty((n,), dtype=torch.float32, device=DEV)
    ma.mesh_attn_reduce_add(ins, out)
    ma.mesh_attn_reduce_add(ins, ins[0])  # out == in[0]
    torch.cuda.synchronize()
    assert torch.equal(out, ins[0])  # same bits: the adds run in input order either way
    check_close("sum", host_f64(out), reduce_add(parts), F32_TOL, normalised_also=False)


def test_split_backward_then_add_reduce():
    # One KV partition met by four Q partitions held by two "holders" (two Q partitions each): every
    # holder runs its backward into its own dK/dV, and the add-reduce gives the full gradient.
    sq, sk, hq, hkv, d, nq = 192, 256, 8, 2, 128, 4
    log("[split backward + reduce]")
    scale = np.float32(1.0 / math.sqrt(d))
    k, kv = gen(1300, synthetic.T_K, 0, (1, sk, hkv, d))
    v, vv = gen(1300, synthetic.T_V, 0, (1, sk, hkv, d))
    holders = [[], []]
    dk_ref = np.zeros((1, sk, hkv, d))
    dv_ref = np.zeros((1, sk, hkv, d))
    for i in range(nq):
        q, qv = gen(1300, synthetic.T_Q, i, (1, sq, hq, d))
        do, dov = gen(1300, synthetic.T_DO, i, (1, sq, hq, d))
        O, L = attn_tile(qv, kv, vv, scale)
        o_dev, o_used, l_dev, l_used = stored_o_lse(O, L)
        _, dki, dvi = attn_tile_bwd(qv, kv, vv, o_used, dov, l_used, scale)
        dk_ref += dki
        dv_ref += dvi
        holders[i % 2].append((q, o_dev, do, l_dev))
    dks, dvs = [], []
    for h in holders:
        dk = torch.full((1, sk, hkv, d), float("nan"), dtype=torch.float32, device=DEV)
        dv = torch.full_like(dk, float("nan"))
        tiles = []
        for q, o_dev, do, l_dev in h:
            dq = torch.empty((1, sq, hq, d), dtype=torch.float32, device=DEV)
            tiles.append(BwdTile(q, k, v, o_dev, do, l_dev, dq, dk, dv))
        ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(tiles, float(scale), ma.MA_MASK_NONE)), dtype=torch.uint8,
                         device=DEV)
        ma.mesh_attn_tile_bwd(tiles, float(scale), ma.MA_MASK_NONE, workspace=ws)
        dks.append(dk)
        dvs.append(dv)
    dk_sum = torch.empty_like(dks[0])
    dv_sum = torch.empty_like(dvs[0])
    ma.mesh_attn_reduce_add(dks, dk_sum)
    ma.mesh_attn_reduce_add(dvs, dv_sum)
    torch.cuda.synchronize()
    check_grad("dK", dk_sum, dk_ref)
    check_grad("dV", dv_sum, dv_ref)
