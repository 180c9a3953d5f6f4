"""Full-shape parity of the Mesh 8 x 8 share's backward, its gradient add-reduce and the striped
causal share, in the launch configuration the bench times.

GPU 9 of n = 64 at S = 1,048,576 ([Mesh] section 3.3, KV partition rotation): Q partitions 8..15
against KV partitions {1, 9, ..., 57}, 16384 tokens each, 32/8 heads, d = 128, bf16.

* Backward ([Mesh] section 3.5): all 64 pairs in one mesh_attn_tile_bwd call, so dQ_i is summed
  over the 8 KV partitions inside the dQ kernel and dK/dV_j over the 8 Q partitions inside the
  dK/dV kernel.  An oracle forward of 131072 rows over 131072 keys per head does not finish on the
  host, so O and LSE are seeded stored inputs of a real forward's magnitude (O ~ sqrt(e/n) N(0,1)
  with n = 131072 keys, LSE ~ ln n + 1/2 + 0.3 N(0,1)); both sides read the same stored values.
  Sampled dQ rows are checked against the oracle over all 8 KV partitions, sampled dK/dV keys
  against the oracle over every row of all 8 Q partitions and all 32 query heads.
* Add-reduce: the eight 64M-float partial dQ of one Q partition (seeded fp32 stand-ins), summed
  on the device and checked on EVERY element against the fp64 oracle sum, within the bound of a
  left-to-right fp32 sum, (k - 1) 2^-24 sum_r |x_r|.
* Striped causal share ([Mesh] section 3.7, partition p holds tokens p + 64 t): every pair
  PARTIAL; the 64 tiles in one forward call and the 64 pairs in one backward call, checked on
  sampled rows and keys.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import BwdTile, Tile  # noqa: E402
from oracle import attn_tile, attn_tile_bwd, merge, reduce_add  # noqa: E402
from gpu_helpers import (BF16_LSE_TOL, BF16_O_TOL, DEV, F32_TOL, check_close, dev_bf16, gen, host_f64,  # noqa: E402
                         log, positions)
from test_gpu_workloads import empty_out, sample_rows  # noqa: E402

import synthetic  # noqa: E402

HQ, HKV, D = 32, 8, 128
SCALE = np.float32(1.0 / math.sqrt(D))
N_GPUS, A, B, G, P = 64, 8, 8, 9, 16384


def check_grad(name, got, ref):
    scale = max(float(np.max(np.abs(ref))), 1e-3)
    err = float(np.max(np.abs(got - ref)))
    log(f"  {name}: max_abs_err={err:.3e} max|ref|={scale:.3e} rel={err / scale:.2e}")
    assert np.isfinite(got).all() and err <= 2e-2 * scale, f"{name}: {err} > 2e-2 * {scale}"


def seeded_o_lse(wid, part, n_keys, shape_o, shape_l, lse_mu=None):
    """Stored O (bf16) and LSE (fp32) inputs of the backward with a real forward's magnitudes."""
    sigma = np.float32(math.sqrt(math.e / n_keys))
    ob = synthetic.f32_to_bf16_bits(synthetic.normal_f32(wid, synthetic.T_O_IN, part, shape_o) * sigma)
    mu = np.float32(math.log(n_keys) + 0.5) if lse_mu is None else lse_mu
    lv = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, part, shape_l) * np.float32(0.3) + mu).astype(np.float32)
    return (dev_bf16(ob), synthetic.bf16_bits_to_f32(ob).astype(np.float64), torch.from_numpy(lv).to(DEV),
            lv.astype(np.float64))


def test_mesh_8x8_1m_backward_full_shape():
    wid = 4  # the forward workload's Q, K, V
    log("[full shape] mesh 8x8 backward, P=16384, 64 pairs in one call")
    qparts, kparts = ma.mesh_attn_map_mesh_tile(N_GPUS, A, B, G, True)
    Q = {i: gen(wid, synthetic.T_Q, i, (1, P, HQ, D)) for i in qparts}
    K = {j: gen(wid, synthetic.T_K, j, (1, P, HKV, D)) for j in kparts}
    V = {j: gen(wid, synthetic.T_V, j, (1, P, HKV, D)) for j in kparts}
    dO = {i: gen(wid, synthetic.T_DO, i, (1, P, HQ, D)) for i in qparts}
    OL = {i: seeded_o_lse(wid, i, B * P, (1, P, HQ, D), (1, HQ, P)) for i in qparts}
    log("  inputs drawn")
    dq = {i: torch.full((1, P, HQ, D), float("nan"), dtype=torch.float32, device=DEV) for i in qparts}
    dk = {j: torch.full((1, P, HKV, D), float("nan"), dtype=torch.float32, device=DEV) for j in kparts}
    dv = {j: torch.full_like(dk[j], float("nan")) for j in kparts}
    btiles = [BwdTile(Q[i][0], K[j][0], V[j][0], OL[i][0], dO[i][0], OL[i][2], dq[i], dk[j], dv[j])
              for i in qparts for j in kparts]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, float(SCALE), ma.MA_MASK_NONE)),
                     dtype=torch.uint8, device=DEV)
    ma.mesh_attn_tile_bwd(btiles, float(SCALE), ma.MA_MASK_NONE, workspace=ws)
    torch.cuda.synchronize()
    log("  backward done")
    for i in qparts:
        assert torch.isfinite(dq[i]).all(), f"dQ{i} not finite"
    for j in kparts:
        assert torch.isfinite(dk[j]).all() and torch.isfinite(dv[j]).all(), f"dK/dV{j} not finite"
    kall = np.concatenate([K[j][1] for j in kparts], axis=1)
    vall = np.concatenate([V[j][1] for j in kparts], axis=1)
    for i in (qparts[0], G, qparts[7]):
        rows = sample_rows(P, 400 + i, extra=6)
        dq_r, _, _ = attn_tile_bwd(Q[i][1][:, rows], kall, vall, OL[i][1][:, rows], dO[i][1][:, rows],
                                   OL[i][3][:, :, rows], SCALE)
        check_grad(f"dQ Q{i}", host_f64(dq[i])[:, rows], dq_r)
    for j in (kparts[0], kparts[5]):
        keys = sample_rows(P, 500 + j, extra=4)
        dk_r = dv_r = 0
        for i in qparts:
            _, a_, b_ = attn_tile_bwd(Q[i][1], K[j][1][:, keys], V[j][1][:, keys], OL[i][1], dO[i][1], OL[i][3],
                                      SCALE)
            dk_r = dk_r + a_
            dv_r = dv_r + b_
        check_grad(f"dK KV{j}", host_f64(dk[j])[:, keys], dk_r)
        check_grad(f"dV KV{j}", host_f64(dv[j])[:, keys], dv_r)


def test_reduce_add_8_partial_dq_full_shape():
    # the addition of the gradient reduce-scatter for one Q partition: 8 partial dQ of
    # [1, 16384, 32, 128] float32 (64M floats, 256 MiB each), in one call as the bench times it
    log("[full shape] add-reduce of 8 x 64M floats")
    k, shape = 8, (1, P, HQ, D)
    parts = [synthetic.normal_f32(4100, synthetic.T_O_IN, r, shape) for r in range(k)]
    ins = [torch.from_numpy(p).to(DEV) for p in parts]
    out = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    ma.mesh_attn_reduce_add(ins, out)
    torch.cuda.synchronize()
    got = host_f64(out)
    ref = reduce_add(parts)
    absum = reduce_add([np.abs(p) for p in parts])
    err = np.abs(got - ref)
    bound = (k - 1) * 2.0 ** -24 * absum * (1 + 1e-6)
    log(f"  max_abs_err={float(err.max()):.3e}; elements over the fp32 summation bound: {int((err > bound).sum())}")
    assert not np.isnan(got).any()
    assert (err <= bound).all()
    check_close("sum", got, ref, F32_TOL, normalised_also=False)


def test_mesh_8x8_striped_causal_share_full_size():
    wid = 8
    mode = ma.MA_MASK_STRIPED_ZIGZAG
    log("[full shape] mesh 8x8 striped causal share, P=16384")
    qparts, kparts = ma.mesh_attn_map_mesh_tile(N_GPUS, A, B, G, True)
    Q = {i: gen(wid, synthetic.T_Q, i, (1, P, HQ, D)) for i in qparts}
    K = {j: gen(wid, synthetic.T_K, j, (1, P, HKV, D)) for j in kparts}
    V = {j: gen(wid, synthetic.T_V, j, (1, P, HKV, D)) for j in kparts}
    qpos = {i: ma.mesh_attn_pos_striped(N_GPUS, i) for i in qparts}
    kpos = {j: ma.mesh_attn_pos_striped(N_GPUS, j) for j in kparts}
    assert all(ma.mesh_attn_classify(qpos[i], P, kpos[j], P, mode) == ma.MA_TILE_PARTIAL
               for i in qparts for j in kparts)
    tiles = {(i, j): Tile(Q[i][0], K[j][0], V[j][0], *empty_out(P), qpos[i], kpos[j]) for i in qparts for j in kparts}
    ma.mesh_attn_tile_fwd(list(tiles.values()), float(SCALE), mode)
    merged = {}
    for i in (qparts[0], qparts[6]):
        o, lse = empty_out(P)
        ma.mesh_attn_merge([tiles[(i, j)].o for j in kparts], [tiles[(i, j)].lse for j in kparts], o, lse)
        merged[i] = (o, lse)
    torch.cuda.synchronize()
    log("  forward done")
    kall = np.concatenate([K[j][1] for j in kparts], axis=1)
    vall = np.concatenate([V[j][1] for j in kparts], axis=1)
    kp_all = np.concatenate([positions(kpos[j], P) for j in kparts])
    for i in merged:
        rows = sample_rows(P, 600 + i, extra=8)
        Oref, Lref = attn_tile(Q[i][1], kall, vall, SCALE, None, True, positions(qpos[i], P), kp_all, rows=rows)
        check_close(f"merged O Q{i}", host_f64(merged[i][0])[:, rows], Oref, BF16_O_TOL)
        check_close(f"merged LSE Q{i}", host_f64(merged[i][1])[:, :, rows], Lref, BF16_LSE_TOL)
    # two tiles' own partials: the pair where Q's phase is below KV's (row 0 sees no key) and above
    for i, j in ((qparts[0], kparts[3]), (qparts[7], kparts[0])):
        rows = sample_rows(P, 700 + i + j, extra=6)
        Ot, Lt = attn_tile(Q[i][1], K[j][1], V[j][1], SCALE, None, True, positions(qpos[i], P),
                           positions(kpos[j], P), rows=rows)
        check_close(f"tile O ({i},{j})", host_f64(tiles[(i, j)].o)[:, rows], Ot, BF16_O_TOL)
        check_close(f"tile LSE ({i},{j})", host_f64(tiles[(i, j)].lse)[:, :, rows], Lt, BF16_LSE_TOL)
    del tiles, merged
    torch.cuda.empty_cache()
    # backward: 64 pairs in one call
    dO = {i: gen(wid, synthetic.T_DO, i, (1, P, HQ, D)) for i in qparts}
    OL = {i: seeded_o_lse(wid, i, B * P // 2, (1, P, HQ, D), (1, HQ, P)) for i in qparts}
    dq = {i: torch.full((1, P, HQ, D), float("nan"), dtype=torch.float32, device=DEV) for i in qparts}
    dk = {j: torch.full((1, P, HKV, D), float("nan"), dtype=torch.float32, device=DEV) for j in kparts}
    dv = {j: torch.full_like(dk[j], float("nan")) for j in kparts}
    btiles = [BwdTile(Q[i][0], K[j][0], V[j][0], OL[i][0], dO[i][0], OL[i][2], dq[i], dk[j], dv[j], qpos[i], kpos[j])
              for i in qparts for j in kparts]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, float(SCALE), mode)), dtype=torch.uint8,
                     device=DEV)
    ma.mesh_attn_tile_bwd(btiles, float(SCALE), mode, workspace=ws)
    torch.cuda.synchronize()
    log("  backward done")
    qp_host = {i: positions(qpos[i], P) for i in qparts}
    for i in (qparts[0], qparts[7]):
        assert torch.isfinite(dq[i]).all()
        rows = sample_rows(P, 800 + i, extra=6)
        dq_r, _, _ = attn_tile_bwd(Q[i][1][:, rows], kall, vall, OL[i][1][:, rows], dO[i][1][:, rows],
                                   OL[i][3][:, :, rows], SCALE, None, True, qp_host[i][rows], kp_all)
        check_grad(f"dQ Q{i}", host_f64(dq[i])[:, rows], dq_r)
    for j in (kparts[0], kparts[6]):
        assert torch.isfinite(dk[j]).all() and torch.isfinite(dv[j]).all()
        keys = sample_rows(P, 900 + j, extra=4)
        kp = positions(kpos[j], P)[keys]
        dk_r = dv_r = 0
        for i in qparts:
            _, a_, b_ = attn_tile_bwd(Q[i][1], K[j][1][:, keys], V[j][1][:, keys], OL[i][1], dO[i][1], OL[i][3],
                                      SCALE, None, True, qp_host[i], kp)
            dk_r = dk_r + a_
            dv_r = dv_r + b_
        check_grad(f"dK KV{j}", host_f64(dk[j])[:, keys], dk_r)
        check_grad(f"dV KV{j}", host_f64(dv[j])[:, keys], dv_r)
