"""GPU parity at the limits the C ABI declares: MA_MAX_HEADS query heads (single-byte head
tables in the kernel arguments; a 128-head group under one KV head) and MA_MAX_TILES tiles in
one forward call (137 launches of the tile table) and in one backward call (independent pairs: 4096
query groups and 4096 KV groups, 512 launches a side), each checked against the fp64 oracle."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import Pos, Tile, _abi  # noqa: E402
from oracle import attn_tile, attn_tile_bwd  # noqa: E402
from gpu_helpers import BF16_LSE_TOL, BF16_O_TOL, DEV, check_close, gen, host_f64, log, positions  # noqa: E402
from test_gpu_bwd import GRAD_REL_TOL, run_case  # noqa: E402

import synthetic  # noqa: E402

HQ_MAX = _abi.MA_MAX_HEADS


@pytest.mark.parametrize("hkv", [1, 8, HQ_MAX])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_max_heads_forward(hkv, d, causal):
    sq, sk = 40, 70
    wid = 2300 + hkv + d + (1 if causal else 0)
    log(f"[limits fwd] hq={HQ_MAX} hkv={hkv} d={d} causal={causal} sq={sq} sk={sk} seed={wid}")
    q, qv = gen(wid, synthetic.T_Q, 0, (1, sq, HQ_MAX, d))
    k, kv = gen(wid, synthetic.T_K, 0, (1, sk, hkv, d))
    v, vv = gen(wid, synthetic.T_V, 0, (1, sk, hkv, d))
    o = torch.full((1, sq, HQ_MAX, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((1, HQ_MAX, sq), float("nan"), dtype=torch.float32, device=DEV)
    scale = np.float32(1.0 / math.sqrt(d))
    qp, kp = (Pos([(0, 50, 1)]), Pos([(0, 0, 1)])) if causal else (None, None)
    mode = ma.MA_MASK_CAUSAL if causal else ma.MA_MASK_NONE
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, qp, kp)], float(scale), mode)
    torch.cuda.synchronize()
    O, L = attn_tile(qv, kv, vv, scale, None, causal, positions(qp, sq) if causal else None,
                     positions(kp, sk) if causal else None)
    check_close("O", host_f64(o), O, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(lse), L, BF16_LSE_TOL)


@pytest.mark.parametrize("hkv", [1, 8, HQ_MAX])
def test_max_heads_backward(hkv):
    log(f"[limits bwd] hq={HQ_MAX} hkv={hkv}")
    run_case(2400 + hkv, 40, 70, HQ_MAX, hkv, 64)


def test_max_heads_backward_causal_d128():
    log(f"[limits bwd] hq={HQ_MAX} hkv=8 d=128 causal")
    run_case(2500, 45, 66, HQ_MAX, 8, 128, mode=ma.MA_MASK_CAUSAL, qp=Pos([(0, 30, 1)]), kp=Pos([(0, 0, 1)]))


def test_max_tiles_one_call():
    """MA_MAX_TILES tiles: a 64 x 64 grid of partitions of 8 tokens (GQA 2/1, d = 64), every pair a
    tile of one call, every tile's (O, LSE) checked."""
    n, P, hq, hkv, d = 64, 8, 2, 1, 64
    assert n * n == _abi.MA_MAX_TILES
    log(f"[limits tiles] {n * n} tiles of {P} x {P}")
    wid = 2600
    q_all, qv = gen(wid, synthetic.T_Q, 0, (n, 1, P, hq, d))
    k_all, kv = gen(wid, synthetic.T_K, 0, (n, 1, P, hkv, d))
    v_all, vv = gen(wid, synthetic.T_V, 0, (n, 1, P, hkv, d))
    o_all = torch.full((n * n, 1, P, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    l_all = torch.full((n * n, 1, hq, P), float("nan"), dtype=torch.float32, device=DEV)
    tiles = [Tile(q_all[i], k_all[j], v_all[j], o_all[i * n + j], l_all[i * n + j], None, None)
             for i in range(n) for j in range(n)]
    scale = np.float32(0.125)
    ma.mesh_attn_tile_fwd(tiles, float(scale), ma.MA_MASK_NONE)
    torch.cuda.synchronize()
    o_h, l_h = host_f64(o_all), host_f64(l_all)
    eo = el = 0.0
    for i in range(n):
        for j in range(n):
            O, L = attn_tile(qv[i], kv[j], vv[j], scale)
            assert not np.isnan(o_h[i * n + j]).any() and not np.isnan(l_h[i * n + j]).any(), (i, j)
            eo = max(eo, float(np.max(np.abs(o_h[i * n + j] - O))))
            el = max(el, float(np.max(np.abs(l_h[i * n + j] - L))))
    log(f"  O max_abs_err={eo:.3e}  LSE max_abs_err={el:.3e}")
    assert eo <= BF16_O_TOL and el <= BF16_LSE_TOL


def test_max_tiles_backward_independent_pairs():
    """MA_MAX_TILES independent (Q partition, KV partition) pairs of 16 tokens (GQA 2/1, d = 64) in
    one backward call: every pair its own dQ and dK/dV group, so the call packs 4096 pieces a side
    into launches of 8.  O and LSE are the GPU forward's (checked against the oracle by the test
    above); the oracle's backward reads the same stored values.  Every pair's gradients checked."""
    m, P, hq, hkv, d = _abi.MA_MAX_TILES, 16, 2, 1, 64
    log(f"[limits bwd pairs] {m} independent pairs of {P} x {P}")
    wid = 2650
    q_all, qv = gen(wid, synthetic.T_Q, 0, (m, 1, P, hq, d))
    k_all, kv = gen(wid, synthetic.T_K, 0, (m, 1, P, hkv, d))
    v_all, vv = gen(wid, synthetic.T_V, 0, (m, 1, P, hkv, d))
    do_all, dov = gen(wid, synthetic.T_DO, 0, (m, 1, P, hq, d))
    o_all = torch.empty((m, 1, P, hq, d), dtype=torch.bfloat16, device=DEV)
    l_all = torch.empty((m, 1, hq, P), dtype=torch.float32, device=DEV)
    scale = np.float32(0.125)
    ma.mesh_attn_tile_fwd([Tile(q_all[i], k_all[i], v_all[i], o_all[i], l_all[i]) for i in range(m)], float(scale))
    dq_all = torch.full((m, 1, P, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    dk_all = torch.full((m, 1, P, hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    dv_all = torch.full_like(dk_all, float("nan"))
    ma.mesh_attn_tile_bwd([ma.BwdTile(q_all[i], k_all[i], v_all[i], o_all[i], do_all[i], l_all[i], dq_all[i], dk_all[i],
                                      dv_all[i]) for i in range(m)], float(scale))
    torch.cuda.synchronize()
    o_h, l_h = host_f64(o_all), host_f64(l_all)
    dq_h, dk_h, dv_h = host_f64(dq_all), host_f64(dk_all), host_f64(dv_all)
    worst = 0.0
    for i in range(m):
        refs = attn_tile_bwd(qv[i], kv[i], vv[i], o_h[i], dov[i], l_h[i], scale)
        for name, got, ref in zip(("dQ", "dK", "dV"), (dq_h[i], dk_h[i], dv_h[i]), refs):
            scl = max(float(np.max(np.abs(ref))), 1e-3)
            err = float(np.max(np.abs(got - ref)))
            worst = max(worst, err / scl)
            assert err <= GRAD_REL_TOL * scl, (i, name, err, scl)
    log(f"  worst max_abs_err / max|ref| over {m} pairs x 3 gradients: {worst:.2e}")
