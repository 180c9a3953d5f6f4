"""Full-size parity of the five workloads, in the launch configuration the bench uses.

At these sizes the oracle checks sampled outputs: each output row depends only
on its own query row (forward, merge, dQ) and each dK/dV row only on its own
key, so sampled rows and keys are checked exactly against the fp64 oracle, and
properties that hold at any size are checked on every row.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import BwdTile, Pos, Tile  # noqa: E402
from oracle import attn_tile, attn_tile_bwd, merge, layout  # noqa: E402
from gpu_helpers import (BF16_LSE_TOL, BF16_O_TOL, DEV, check_close, dev_bf16, gen, host_f64, log,  # noqa: E402
                         oracle_forward_by_head, positions)
from test_gpu_bwd import stored_o_lse  # noqa: E402

import synthetic  # noqa: E402

HQ, HKV, D = 32, 8, 128
SCALE = np.float32(1.0 / math.sqrt(D))


def sample_rows(n, wid, extra=16):
    rng = np.random.default_rng([wid, 77])
    fixed = [0, 1, 31, 32, 63, 64, 127, n // 2, n - 65, n - 64, n - 2, n - 1]
    rows = sorted(set([r for r in fixed if 0 <= r < n] + list(rng.choice(n, size=min(extra, n), replace=False))))
    return np.array(rows, dtype=np.int64)


def empty_out(sq):
    return (torch.empty((1, sq, HQ, D), dtype=torch.bfloat16, device=DEV),
            torch.empty((1, HQ, sq), dtype=torch.float32, device=DEV))


def test_gqa_tile_8k_forward():
    # single non-causal tile, Q 8192 x KV 8192, 32/8 heads, d=128, bf16
    wid, S = 2, 8192
    log("[workload gqa-tile-8k fwd]")
    q, qv = gen(wid, synthetic.T_Q, 0, (1, S, HQ, D))
    k, kv = gen(wid, synthetic.T_K, 0, (1, S, HKV, D))
    v, vv = gen(wid, synthetic.T_V, 0, (1, S, HKV, D))
    o, lse = empty_out(S)
    p0 = ma.mesh_attn_pos_contiguous(0)
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, p0, p0)], float(SCALE), ma.MA_MASK_NONE)
    torch.cuda.synchronize()
    rows = sample_rows(S, wid)
    Oref, Lref = attn_tile(qv, kv, vv, SCALE, rows=rows)
    Og, Lg = host_f64(o), host_f64(lse)
    check_close("O[rows]", Og[:, rows], Oref, BF16_O_TOL)
    check_close("LSE[rows]", Lg[:, :, rows], Lref, BF16_LSE_TOL)
    # every row: finite, and each output is a convex combination of the V column values
    assert np.isfinite(Og).all() and np.isfinite(Lg).all()
    vmax = np.abs(vv).max(axis=1)                      # [1, Hkv, d]
    bound = np.repeat(vmax, HQ // HKV, axis=1)         # [1, Hq, d]
    assert (np.abs(Og) <= bound[:, None] * (1 + 2 ** -7) + 1e-6).all()


def test_zigzag_causal_128k_rank5_forward_and_merge():
    # S = 131072 in 32 chunks of 4096; rank 5 of 16 owns chunks {5, 26}; causal on global positions
    wid, N, r, C = 3, 16, 5, 4096
    log("[workload zigzag-causal-128k]")
    qchunks = ma.mesh_attn_map_zigzag(N, r)
    assert qchunks == layout.zigzag_chunks(N, r) == (5, 26)
    Q = {c: gen(wid, synthetic.T_Q, c, (1, C, HQ, D)) for c in qchunks}
    K = [gen(wid, synthetic.T_K, j, (1, C, HKV, D)) for j in range(2 * N)]
    V = [gen(wid, synthetic.T_V, j, (1, C, HKV, D)) for j in range(2 * N)]
    qpos = [ma.mesh_attn_pos_contiguous(c * C) for c in qchunks]
    kpos = [ma.mesh_attn_pos_contiguous(j * C) for j in range(2 * N)]
    wl = ma.mesh_attn_build_worklist(qpos, [C, C], kpos, [C] * (2 * N), ma.MA_MASK_CAUSAL)
    assert len(wl) == 33 and sum(c == ma.MA_TILE_PARTIAL for _, _, c in wl) == 2
    tiles = []
    for i, j, _ in wl:
        o, lse = empty_out(C)
        tiles.append(Tile(Q[qchunks[i]][0], K[j][0], V[j][0], o, lse, qpos[i], kpos[j]))
    ma.mesh_attn_tile_fwd(tiles, float(SCALE), ma.MA_MASK_CAUSAL)
    merged = []
    for i in range(2):
        mine = [t for t, (ii, _, _) in zip(tiles, wl) if ii == i]
        assert len(mine) == (6 if i == 0 else 27)
        o, lse = empty_out(C)
        ma.mesh_attn_merge([t.o for t in mine], [t.lse for t in mine], o, lse)
        merged.append((o, lse))
    # the same share with the KV chunks gathered into one buffer: one causal tile per Q chunk, no merge
    kg = torch.cat([x[0] for x in K], dim=1)
    vg = torch.cat([x[0] for x in V], dim=1)
    fused = [empty_out(C) for _ in qchunks]
    ftiles = [Tile(Q[c][0], kg[:, :(c + 1) * C], vg[:, :(c + 1) * C], fused[i][0], fused[i][1], qpos[i],
                   ma.mesh_attn_pos_contiguous(0)) for i, c in enumerate(qchunks)]
    ma.mesh_attn_tile_fwd(ftiles, float(SCALE), ma.MA_MASK_CAUSAL)
    torch.cuda.synchronize()
    kall = np.concatenate([x[1] for x in K], axis=1)
    vall = np.concatenate([x[1] for x in V], axis=1)
    kp_all = np.arange(2 * N * C)
    for i, c in enumerate(qchunks):
        rows = sample_rows(C, wid + i)
        qp = positions(qpos[i], C)
        Oref, Lref = attn_tile(Q[c][1], kall, vall, SCALE, None, True, qp, kp_all, rows=rows)
        check_close(f"merged O chunk {c}", host_f64(merged[i][0])[:, rows], Oref, BF16_O_TOL)
        check_close(f"merged LSE chunk {c}", host_f64(merged[i][1])[:, :, rows], Lref, BF16_LSE_TOL)
        # fused: one tile per Q chunk over the gathered KV buffer (chunks 0..c, one contiguous range)
        check_close(f"fused O chunk {c}", host_f64(fused[i][0])[:, rows], Oref, BF16_O_TOL)
        check_close(f"fused LSE chunk {c}", host_f64(fused[i][1])[:, :, rows], Lref, BF16_LSE_TOL)
        # the diagonal (partially masked) tile's own partial
        t = [t for t, (ii, jj, _) in zip(tiles, wl) if ii == i and jj == c][0]
        Ot, Lt = attn_tile(Q[c][1], K[c][1], V[c][1], SCALE, None, True, qp, positions(kpos[c], C), rows=rows)
        check_close(f"diagonal O chunk {c}", host_f64(t.o)[:, rows], Ot, BF16_O_TOL)
        check_close(f"diagonal LSE chunk {c}", host_f64(t.lse)[:, :, rows], Lt, BF16_LSE_TOL)


def test_zigzag_diagonal_mask_probe_full_size():
    # Q = 0 on the 4096 x 4096 diagonal tile of chunk 26: exp(LSE[t]) is exactly t + 1 for every row.
    C = 4096
    log("[workload mask probe 4096 diagonal]")
    q = torch.zeros((1, C, HQ, D), dtype=torch.bfloat16, device=DEV)
    k, _ = gen(3, synthetic.T_K, 26, (1, C, HKV, D))
    v, _ = gen(3, synthetic.T_V, 26, (1, C, HKV, D))
    o, lse = empty_out(C)
    p = ma.mesh_attn_pos_contiguous(26 * C)
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, p, p)], float(SCALE), ma.MA_MASK_CAUSAL)
    torch.cuda.synchronize()
    counts = np.rint(np.exp(host_f64(lse)[0])).astype(np.int64)
    assert np.array_equal(counts, np.broadcast_to(np.arange(1, C + 1), counts.shape))


def test_mesh_8x8_1m_forward_and_merge():
    # One GPU (g = 9) of n = 64 at S = 1,048,576: partitions of 16384 tokens, 8 x 8 tile with KV rotation,
    # non-causal; 8-way merges per Q partition plus 7 incoming seeded partials for the owned partition; the
    # fused forward over the gathered KV and the GOO replay of 4 x 4 chunk tasks on the same inputs.
    wid, n, a, b, g, P = 4, 64, 8, 8, 9, 16384
    log("[workload mesh-8x8-1m]")
    qparts, kparts = ma.mesh_attn_map_mesh_tile(n, a, b, g, True)
    assert (qparts, kparts) == layout.mesh_tile(n, a, b, g, True)
    Q = {i: gen(wid, synthetic.T_Q, i, (1, P, HQ, D)) for i in qparts}
    K = {j: gen(wid, synthetic.T_K, j, (1, P, HKV, D)) for j in kparts}
    V = {j: gen(wid, synthetic.T_V, j, (1, P, HKV, D)) for j in kparts}
    tiles = {}
    for i in qparts:
        for j in kparts:
            o, lse = empty_out(P)
            tiles[(i, j)] = Tile(Q[i][0], K[j][0], V[j][0], o, lse)
    ma.mesh_attn_tile_fwd(list(tiles.values()), float(SCALE), ma.MA_MASK_NONE)
    mu = np.float32(math.log(b * P) + 0.5)
    inc = []
    for r in range(a - 1):
        oi, oiv = gen(wid, synthetic.T_O_IN, r, (1, P, HQ, D))
        li = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, r, (1, HQ, P)) + mu).astype(np.float32)
        inc.append((oi, oiv, torch.from_numpy(li).to(DEV), li.astype(np.float64)))
    merged = {}
    for i in qparts:
        os_ = [tiles[(i, j)].o for j in kparts]
        ls_ = [tiles[(i, j)].lse for j in kparts]
        if i == g:
            os_ += [x[0] for x in inc]
            ls_ += [x[2] for x in inc]
        o, lse = empty_out(P)
        ma.mesh_attn_merge(os_, ls_, o, lse)
        merged[i] = (o, lse)
    # the same share with the 8 KV partitions gathered into one buffer: one tile per Q partition, and
    # only the owned partition's merge with the 7 incoming partials
    kg = torch.cat([K[j][0] for j in kparts], dim=1)
    vg = torch.cat([V[j][0] for j in kparts], dim=1)
    fused = {i: empty_out(P) for i in qparts}
    ma.mesh_attn_tile_fwd([Tile(Q[i][0], kg, vg, fused[i][0], fused[i][1]) for i in qparts], float(SCALE),
                          ma.MA_MASK_NONE)
    ma.mesh_attn_merge([fused[g][0]] + [x[0] for x in inc], [fused[g][1]] + [x[2] for x in inc],
                       fused[g][0], fused[g][1])
    # the GOO replay the bench times ([Mesh] section 3.4): k_Q = k_KV = 4 chunks per partition, chunk c of
    # every Q (KV) partition gathered into one buffer, the compute tasks C-i-j of the greedy plan in its
    # order, each folded into its Q chunk's (O, LSE) (the first task of a chunk overwrites)
    kq = kkv = 4
    cq, ck = P // kq, P // kkv
    gq = [torch.cat([Q[i][0][:, c * cq:(c + 1) * cq] for i in qparts], dim=1) for c in range(kq)]
    gk = [torch.cat([K[j][0][:, c * ck:(c + 1) * ck] for j in kparts], dim=1) for c in range(kkv)]
    gv = [torch.cat([V[j][0][:, c * ck:(c + 1) * ck] for j in kparts], dim=1) for c in range(kkv)]
    acc = [empty_out(a * cq) for _ in range(kq)]
    order = [(ci, cj) for _, comp in ma.mesh_attn_goo_plan(kq, kkv, 0.5, 1.0, 0.5, 0.5, 1.0) for _, ci, cj in comp]
    assert sorted(order) == [(ci, cj) for ci in range(kq) for cj in range(kkv)]
    started = set()
    for ci, cj in order:
        ma.mesh_attn_tile_fwd([Tile(gq[ci], gk[cj], gv[cj], acc[ci][0], acc[ci][1])], float(SCALE),
                              ma.MA_MASK_NONE, accumulate=ci in started)
        started.add(ci)
    torch.cuda.synchronize()
    kall = np.concatenate([K[j][1] for j in kparts], axis=1)
    vall = np.concatenate([V[j][1] for j in kparts], axis=1)
    for r, i in enumerate(qparts):
        rows = sample_rows(P, wid + i, extra=6 if i != g else 16)
        Oloc, Lloc = attn_tile(Q[i][1], kall, vall, SCALE, rows=rows)
        # row t of Q partition i is row r*cq + t%cq of gathered chunk t//cq
        where = [(int(t) // cq, r * cq + int(t) % cq) for t in rows]
        got_o = np.concatenate([host_f64(acc[c][0][:, at:at + 1]) for c, at in where], axis=1)
        got_l = np.concatenate([host_f64(acc[c][1][:, :, at:at + 1]) for c, at in where], axis=2)
        check_close(f"GOO replay O Q{i}", got_o, Oloc, BF16_O_TOL)
        check_close(f"GOO replay LSE Q{i}", got_l, Lloc, BF16_LSE_TOL)
        if i == g:
            Oref, Lref = merge([(Oloc, Lloc)] + [(x[1][:, rows], x[3][:, :, rows]) for x in inc])
        else:
            Oref, Lref = Oloc, Lloc
        check_close(f"merged O Q{i}", host_f64(merged[i][0])[:, rows], Oref, BF16_O_TOL)
        check_close(f"merged LSE Q{i}", host_f64(merged[i][1])[:, :, rows], Lref, BF16_LSE_TOL)
        check_close(f"fused O Q{i}", host_f64(fused[i][0])[:, rows], Oref, BF16_O_TOL)
        check_close(f"fused LSE Q{i}", host_f64(fused[i][1])[:, :, rows], Lref, BF16_LSE_TOL)
    # one partial tile on its own
    i, j = qparts[3], kparts[5]
    rows = sample_rows(P, 99)
    Ot, Lt = attn_tile(Q[i][1], K[j][1], V[j][1], SCALE, rows=rows)
    check_close("tile O", host_f64(tiles[(i, j)].o)[:, rows], Ot, BF16_O_TOL)
    check_close("tile LSE", host_f64(tiles[(i, j)].lse)[:, :, rows], Lt, BF16_LSE_TOL)


def test_gqa_bwd_4x8k():
    # Backward at the 8k GQA shape: 4 Q partitions of 8192 against one KV partition of 8192, non-causal;
    # dK/dV summed over the 4 partitions.  O and LSE are the oracle's forward of each Q partition against
    # the KV partition (every row, every head), stored as bf16 O and fp32 LSE; both sides read those
    # stored values, so the gradients are those of a consistent forward.
    wid, S, nq = 5, 8192, 4
    log("[workload gqa-bwd-4x8k]")
    k, kv = gen(wid, synthetic.T_K, 0, (1, S, HKV, D))
    v, vv = gen(wid, synthetic.T_V, 0, (1, S, HKV, D))
    dk = torch.empty((1, S, HKV, D), dtype=torch.float32, device=DEV)
    dv = torch.empty_like(dk)
    tiles, host = [], []
    for i in range(nq):
        q, qv = gen(wid, synthetic.T_Q, i, (1, S, HQ, D))
        do, dov = gen(wid, synthetic.T_DO, i, (1, S, HQ, D))
        O, L = oracle_forward_by_head(qv, kv, vv, SCALE)
        o_dev, o_used, l_dev, l_used = stored_o_lse(O, L)
        log(f"  oracle forward of Q partition {i} done")
        dq = torch.empty((1, S, HQ, D), dtype=torch.float32, device=DEV)
        tiles.append(BwdTile(q, k, v, o_dev, do, l_dev, dq, dk, dv))
        host.append(dict(q=qv, o=o_used, do=dov, lse=l_used))
    ma.mesh_attn_tile_bwd(tiles, float(SCALE), ma.MA_MASK_NONE)
    torch.cuda.synchronize()

    def check(name, got, ref):
        scale = max(float(np.max(np.abs(ref))), 1e-3)
        err = float(np.max(np.abs(got - ref)))
        log(f"  {name}: max_abs_err={err:.3e} max|ref|={scale:.3e} rel={err/scale:.2e}")
        assert np.isfinite(got).all() and err <= 2e-2 * scale

    # dQ on sampled rows of each partition (needs all keys)
    for i, h in enumerate(host):
        rows = sample_rows(S, wid + 10 * i, extra=8)
        dq_r, _, _ = attn_tile_bwd(h["q"][:, rows], kv, vv, h["o"][:, rows], h["do"][:, rows], h["lse"][:, :, rows], SCALE)
        check(f"dQ part {i}", host_f64(tiles[i].dq)[:, rows], dq_r)
    # dK/dV on sampled keys (needs every query row of every partition)
    keys = sample_rows(S, wid + 100, extra=12)
    dk_r = dv_r = 0
    for h in host:
        _, a_, b_ = attn_tile_bwd(h["q"], kv[:, keys], vv[:, keys], h["o"], h["do"], h["lse"], SCALE)
        dk_r = dk_r + a_
        dv_r = dv_r + b_
    check("dK[keys]", host_f64(dk)[:, keys], dk_r)
    check("dV[keys]", host_f64(dv)[:, keys], dv_r)
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_zigzag_causal_128k_rank5_backward():
    # Backward of the causal zigzag share: dQ for chunks {5, 26}, partial dK/dV for KV chunks 0..26,
    # 33 computed pairs in one call (EMPTY pairs skipped, the two diagonal pairs masked per element).
    # O and LSE are seeded stored inputs with a real forward's magnitudes (O ~ 0.02 N(0,1),
    # LSE ~ ln(allowed keys) + 0.5 + 0.3 N(0,1)); both sides read the same values.
    wid, N, r, C = 6, 16, 5, 4096
    log("[workload zigzag-causal-128k backward]")
    qchunks = ma.mesh_attn_map_zigzag(N, r)
    nkv = max(qchunks) + 1
    K = [gen(wid, synthetic.T_K, j, (1, C, HKV, D)) for j in range(nkv)]
    V = [gen(wid, synthetic.T_V, j, (1, C, HKV, D)) for j in range(nkv)]
    qpos = [ma.mesh_attn_pos_contiguous(c * C) for c in qchunks]
    kpos = [ma.mesh_attn_pos_contiguous(j * C) for j in range(nkv)]
    wl = ma.mesh_attn_build_worklist(qpos, [C, C], kpos, [C] * nkv, ma.MA_MASK_CAUSAL)
    assert len(wl) == 33
    dk = [torch.empty((1, C, HKV, D), dtype=torch.float32, device=DEV) for _ in range(nkv)]
    dv = [torch.empty_like(x) for x in dk]
    host, dev_in = [], []
    for i, c in enumerate(qchunks):
        q, qv = gen(wid, synthetic.T_Q, c, (1, C, HQ, D))
        do, dov = gen(wid, synthetic.T_DO, c, (1, C, HQ, D))
        ob = synthetic.f32_to_bf16_bits(synthetic.normal_f32(wid, synthetic.T_O_IN, c, (1, C, HQ, D)) * np.float32(0.02))
        ov = synthetic.bf16_bits_to_f32(ob).astype(np.float64)
        n_allowed = (c * C + np.arange(C) + 1).astype(np.float32)
        lv = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, c, (1, HQ, C)) * np.float32(0.3)
              + np.log(n_allowed)[None, None, :] + np.float32(0.5)).astype(np.float32)
        dq = torch.empty((1, C, HQ, D), dtype=torch.float32, device=DEV)
        dev_in.append((q, dev_bf16(ob), do, torch.from_numpy(lv).to(DEV), dq))
        host.append(dict(q=qv, o=ov, do=dov, lse=lv.astype(np.float64), q_pos=positions(qpos[i], C)))
    tiles = [BwdTile(dev_in[i][0], K[j][0], V[j][0], dev_in[i][1], dev_in[i][2], dev_in[i][3], dev_in[i][4],
                     dk[j], dv[j], qpos[i], kpos[j]) for i, j, _ in wl]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(tiles, float(SCALE), ma.MA_MASK_CAUSAL)), dtype=torch.uint8,
                     device=DEV)
    ma.mesh_attn_tile_bwd(tiles, float(SCALE), ma.MA_MASK_CAUSAL, workspace=ws)
    torch.cuda.synchronize()

    def check(name, got, ref):
        scale = max(float(np.max(np.abs(ref))), 1e-3)
        err = float(np.max(np.abs(got - ref)))
        log(f"  {name}: max_abs_err={err:.3e} max|ref|={scale:.3e} rel={err/scale:.2e}")
        assert np.isfinite(got).all() and err <= 2e-2 * scale

    kall = np.concatenate([x[1] for x in K], axis=1)
    vall = np.concatenate([x[1] for x in V], axis=1)
    kp_all = np.arange(nkv * C, dtype=np.int64)
    for i, h in enumerate(host):
        rows = sample_rows(C, wid + 10 * i, extra=8)
        dq_r, _, _ = attn_tile_bwd(h["q"][:, rows], kall, vall, h["o"][:, rows], h["do"][:, rows],
                                   h["lse"][:, :, rows], SCALE, None, True, h["q_pos"][rows], kp_all)
        check(f"dQ chunk {qchunks[i]}", host_f64(dev_in[i][4])[:, rows], dq_r)
    # dK/dV on sampled keys of KV chunks met by both Q chunks (0, 5: diagonal of chunk 5), by one (13),
    # and the diagonal of chunk 26
    for j in (0, 5, 13, 26):
        keys = sample_rows(C, wid + 100 + j, extra=6)
        kp = positions(kpos[j], C)[keys]
        dk_r = dv_r = 0
        for h in host:
            _, a_, b_ = attn_tile_bwd(h["q"], K[j][1][:, keys], V[j][1][:, keys], h["o"], h["do"], h["lse"], SCALE,
                                      None, True, h["q_pos"], kp)
            dk_r = dk_r + a_
            dv_r = dv_r + b_
        check(f"dK chunk {j}", host_f64(dk[j])[:, keys], dk_r)
        check(f"dV chunk {j}", host_f64(dv[j])[:, keys], dv_r)
    for j in range(nkv):
        assert torch.isfinite(dk[j]).all() and torch.isfinite(dv[j]).all()


def test_mesh_8x8_striped_causal_share():
    # The Mesh 8 x 8 share of GPU 9 (n = 64, KV rotation) under the causal mask with the striped
    # layout of [Mesh] section 3.7 (partition p holds tokens p + 64 t), at 2048 tokens per partition:
    # every pair is PARTIAL.  Forward: 64 tiles in one call, 8-way merges, sampled rows against the
    # oracle over all 8 KV partitions.  Backward: 64 pairs in one call with seeded stored O and LSE;
    # sampled dQ rows and sampled dK/dV keys.
    wid, n, a, b, g, P = 7, 64, 8, 8, 9, 2048
    log("[workload mesh-8x8 striped causal, P=2048]")
    mode = ma.MA_MASK_STRIPED_ZIGZAG
    qparts, kparts = ma.mesh_attn_map_mesh_tile(n, a, b, g, True)
    Q = {i: gen(wid, synthetic.T_Q, i, (1, P, HQ, D)) for i in qparts}
    K = {j: gen(wid, synthetic.T_K, j, (1, P, HKV, D)) for j in kparts}
    V = {j: gen(wid, synthetic.T_V, j, (1, P, HKV, D)) for j in kparts}
    qpos = {i: ma.mesh_attn_pos_striped(n, i) for i in qparts}
    kpos = {j: ma.mesh_attn_pos_striped(n, j) for j in kparts}
    tiles = {(i, j): Tile(Q[i][0], K[j][0], V[j][0], *empty_out(P), qpos[i], kpos[j]) for i in qparts for j in kparts}
    assert all(ma.mesh_attn_classify(qpos[i], P, kpos[j], P, mode) == ma.MA_TILE_PARTIAL for i, j in tiles)
    ma.mesh_attn_tile_fwd(list(tiles.values()), float(SCALE), mode)
    merged = {}
    for i in qparts:
        o, lse = empty_out(P)
        ma.mesh_attn_merge([tiles[(i, j)].o for j in kparts], [tiles[(i, j)].lse for j in kparts], o, lse)
        merged[i] = (o, lse)
    torch.cuda.synchronize()
    kall = np.concatenate([K[j][1] for j in kparts], axis=1)
    vall = np.concatenate([V[j][1] for j in kparts], axis=1)
    kp_all = np.concatenate([positions(kpos[j], P) for j in kparts])
    for i in (qparts[0], qparts[5]):
        rows = sample_rows(P, wid + i, extra=8)
        Oref, Lref = attn_tile(Q[i][1], kall, vall, SCALE, None, True, positions(qpos[i], P), kp_all, rows=rows)
        check_close(f"merged O Q{i}", host_f64(merged[i][0])[:, rows], Oref, BF16_O_TOL)
        check_close(f"merged LSE Q{i}", host_f64(merged[i][1])[:, :, rows], Lref, BF16_LSE_TOL)
    del tiles, merged
    # backward
    host, dev_in = {}, {}
    for i in qparts:
        do, dov = gen(wid, synthetic.T_DO, i, (1, P, HQ, D))
        ob = synthetic.f32_to_bf16_bits(synthetic.normal_f32(wid, synthetic.T_O_IN, i, (1, P, HQ, D)) * np.float32(0.02))
        ov = synthetic.bf16_bits_to_f32(ob).astype(np.float64)
        lv = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, i, (1, HQ, P)) * np.float32(0.3)
              + np.float32(math.log(b * P / 2) + 0.5)).astype(np.float32)
        dq = torch.empty((1, P, HQ, D), dtype=torch.float32, device=DEV)
        dev_in[i] = (do, dev_bf16(ob), torch.from_numpy(lv).to(DEV), dq)
        host[i] = dict(do=dov, o=ov, lse=lv.astype(np.float64), q_pos=positions(qpos[i], P))
    dk = {j: torch.empty((1, P, HKV, D), dtype=torch.float32, device=DEV) for j in kparts}
    dv = {j: torch.empty_like(dk[j]) for j in kparts}
    btiles = [BwdTile(Q[i][0], K[j][0], V[j][0], dev_in[i][1], dev_in[i][0], dev_in[i][2], dev_in[i][3], dk[j], dv[j],
                      qpos[i], kpos[j]) for i in qparts for j in kparts]
    ma.mesh_attn_tile_bwd(btiles, float(SCALE), mode)
    torch.cuda.synchronize()

    def check(name, got, ref):
        scale = max(float(np.max(np.abs(ref))), 1e-3)
        err = float(np.max(np.abs(got - ref)))
        log(f"  {name}: max_abs_err={err:.3e} max|ref|={scale:.3e} rel={err/scale:.2e}")
        assert np.isfinite(got).all() and err <= 2e-2 * scale

    for i in (qparts[0], qparts[7]):
        rows = sample_rows(P, wid + 10 * i, extra=6)
        h = host[i]
        dq_r, _, _ = attn_tile_bwd(Q[i][1][:, rows], kall, vall, h["o"][:, rows], h["do"][:, rows],
                                   h["lse"][:, :, rows], SCALE, None, True, h["q_pos"][rows], kp_all)
        check(f"dQ Q{i}", host_f64(dev_in[i][3])[:, rows], dq_r)
    for j in (kparts[0], kparts[6]):
        keys = sample_rows(P, wid + 100 + j, extra=4)
        kp = positions(kpos[j], P)[keys]
        dk_r = dv_r = 0
        for i in qparts:
            h = host[i]
            _, a_, b_ = attn_tile_bwd(Q[i][1], K[j][1][:, keys], V[j][1][:, keys], h["o"], h["do"], h["lse"], SCALE,
                                      None, True, h["q_pos"], kp)
            dk_r = dk_r + a_
            dv_r = dv_r + b_
        check(f"dK KV{j}", host_f64(dk[j])[:, keys], dk_r)
        check(f"dV KV{j}", host_f64(dv[j])[:, keys], dv_r)
