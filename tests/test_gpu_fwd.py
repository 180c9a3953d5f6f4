"""GPU parity of the tile forward and the LSE merge against the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import Pos, Tile  # noqa: E402
from oracle import attn_tile, merge  # noqa: E402
from gpu_helpers import (BF16_LSE_TOL, BF16_O_TOL, DEV, F32_TOL, check_close, gen, host_f64, log,  # noqa: E402
                         positions)

import synthetic  # noqa: E402


def run_fwd(tiles, scale, mask, head_map=None):
    ma.mesh_attn_tile_fwd(tiles, scale, mask, head_map)
    torch.cuda.synchronize()


def make_case(wid, sq, sk, hq, hkv, d, dtype="bf16", B=1, zero_q=False):
    q, qv = gen(wid, synthetic.T_Q, 0, (B, sq, hq, d), dtype)
    k, kv = gen(wid, synthetic.T_K, 0, (B, sk, hkv, d), dtype)
    v, vv = gen(wid, synthetic.T_V, 0, (B, sk, hkv, d), dtype)
    if zero_q:
        q.zero_()
        qv = np.zeros_like(qv)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = torch.full((B, sq, hq, d), float("nan"), dtype=tdt, device=DEV)
    lse = torch.full((B, hq, sq), float("nan"), dtype=torch.float32, device=DEV)
    return (q, k, v, o, lse), (qv, kv, vv)


def _two_seg(n, g0, g1, st1):
    """Two-segment (zigzag-like) positions; one segment when the partition is too short to split."""
    half = (n + 1) // 2
    return Pos([(0, g0, 1), (half, g1, st1)]) if half < n else Pos([(0, g0, 1)])


MASKS = {
    "none": (ma.MA_MASK_NONE, None, None),
    "causal_diag": (ma.MA_MASK_CAUSAL, lambda sq, sk: Pos([(0, 1000, 1)]), lambda sq, sk: Pos([(0, 1000, 1)])),
    "causal_offset": (ma.MA_MASK_CAUSAL, lambda sq, sk: Pos([(0, 5000 + sk // 2, 1)]), lambda sq, sk: Pos([(0, 5000, 1)])),
    "causal_future": (ma.MA_MASK_CAUSAL, lambda sq, sk: Pos([(0, 7, 1)]), lambda sq, sk: Pos([(0, 7 + sq // 3, 1)])),
    "striped": (ma.MA_MASK_STRIPED_ZIGZAG, lambda sq, sk: ma.mesh_attn_pos_striped(4, 1),
                lambda sq, sk: ma.mesh_attn_pos_striped(4, 3)),
    "zigzag": (ma.MA_MASK_STRIPED_ZIGZAG, lambda sq, sk: _two_seg(sq, 0, 3 * sq, 1),
               lambda sq, sk: _two_seg(sk, 0, 2 * sq, 2)),
}

SHAPES = [(1, 1), (17, 64), (64, 64), (100, 257), (257, 130), (300, 333), (128, 1000)]
GQA = [(4, 4), (8, 4), (8, 2), (16, 2)]


def _cases():
    out = []
    i = 0
    for s in SHAPES:
        for mname in MASKS:
            hq, hkv = GQA[i % len(GQA)]
            d = 128 if i % 3 else 64
            out.append((s[0], s[1], hq, hkv, d, mname))
            i += 1
    return out


@pytest.mark.parametrize("sq,sk,hq,hkv,d,mname", _cases())
def test_fwd_bf16_small_shapes(sq, sk, hq, hkv, d, mname):
    mode, qpf, kpf = MASKS[mname]
    wid = 100 + sq * 7 + sk * 13 + hq + d
    log(f"[fwd bf16] sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} mask={mname} seed={wid}")
    (q, k, v, o, lse), (qv, kv, vv) = make_case(wid, sq, sk, hq, hkv, d)
    qp = qpf(sq, sk) if qpf else None
    kp = kpf(sq, sk) if kpf else None
    scale = 1.0 / math.sqrt(d)
    run_fwd([Tile(q, k, v, o, lse, qp, kp)], scale, mode)
    causal = mode != ma.MA_MASK_NONE
    Oref, Lref = attn_tile(qv, kv, vv, np.float32(scale), None, causal,
                           positions(qp, sq) if causal else None, positions(kp, sk) if causal else None)
    check_close("O", host_f64(o), Oref, BF16_O_TOL)
    check_close("LSE", host_f64(lse), Lref, BF16_LSE_TOL)
    # fully masked rows are exactly (0, -inf)
    Og = host_f64(o)
    for b, h, t in zip(*np.nonzero(np.isneginf(Lref))):
        assert np.all(Og[b, t, h] == 0.0)


@pytest.mark.parametrize("sk", [960, 1024, 1025, 1090])
@pytest.mark.parametrize("mname", ["none", "causal_offset", "striped"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_bf16_kernel_size_switch(sk, mname, d):
    """Key counts on both sides of the switch between the four-wave kernel (at most 16 key
    blocks: 960, 1024) and the eight-wave kernel (1025, 1090), each also with a ragged last
    block, unmasked and masked, against the oracle."""
    mode, qpf, kpf = MASKS[mname]
    sq, hq, hkv = 200, 8, 2
    wid = 1700 + sk + d
    log(f"[fwd size switch] sk={sk} mask={mname} d={d} seed={wid}")
    (q, k, v, o, lse), (qv, kv, vv) = make_case(wid, sq, sk, hq, hkv, d)
    qp = qpf(sq, sk) if qpf else None
    kp = kpf(sq, sk) if kpf else None
    scale = 1.0 / math.sqrt(d)
    run_fwd([Tile(q, k, v, o, lse, qp, kp)], scale, mode)
    causal = mode != ma.MA_MASK_NONE
    Oref, Lref = attn_tile(qv, kv, vv, np.float32(scale), None, causal,
                           positions(qp, sq) if causal else None, positions(kp, sk) if causal else None)
    check_close("O", host_f64(o), Oref, BF16_O_TOL)
    check_close("LSE", host_f64(lse), Lref, BF16_LSE_TOL)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_bf16_head_map_and_batch(d):
    sq, sk, hq, hkv, B = 130, 200, 6, 3, 2
    head_map = [2, 0, 1, 1, 0, 2]
    log(f"[fwd bf16 head_map] d={d} B={B}")
    (q, k, v, o, lse), (qv, kv, vv) = make_case(300 + d, sq, sk, hq, hkv, d, B=B)
    qp, kp = Pos([(0, 150, 1)]), Pos([(0, 0, 1)])
    run_fwd([Tile(q, k, v, o, lse, qp, kp)], 0.09, ma.MA_MASK_CAUSAL, head_map)
    Oref, Lref = attn_tile(qv, kv, vv, np.float32(0.09), head_map, True, positions(qp, sq), positions(kp, sk))
    check_close("O", host_f64(o), Oref, BF16_O_TOL)
    check_close("LSE", host_f64(lse), Lref, BF16_LSE_TOL)


@pytest.mark.parametrize("mname", ["causal_diag", "causal_offset", "striped", "zigzag"])
def test_mask_probe_counts_are_exact(mname):
    # Q = 0 makes every score 0, so exp(LSE[t]) is the exact number of allowed keys.
    mode, qpf, kpf = MASKS[mname]
    sq, sk = 333, 517
    log(f"[mask probe] {mname}")
    (q, k, v, o, lse), (qv, kv, vv) = make_case(400, sq, sk, 8, 2, 128, zero_q=True)
    qp, kp = qpf(sq, sk), kpf(sq, sk)
    run_fwd([Tile(q, k, v, o, lse, qp, kp)], 0.125, mode)
    L = host_f64(lse)
    qa, ka = positions(qp, sq), positions(kp, sk)
    n_ref = (ka[None, :] <= qa[:, None]).sum(axis=1)
    for h in range(8):
        n_gpu = np.where(np.isneginf(L[0, h]), 0, np.rint(np.exp(L[0, h]))).astype(np.int64)
        assert np.array_equal(n_gpu, n_ref), mname


def test_empty_tile_is_filled():
    log("[fwd empty tile]")
    (q, k, v, o, lse), _ = make_case(500, 64, 64, 4, 1, 128)
    run_fwd([Tile(q, k, v, o, lse, Pos([(0, 0, 1)]), Pos([(0, 64, 1)]))], 0.1, ma.MA_MASK_CAUSAL)
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_many_tiles_one_call():
    # more tiles than one launch packs; mixed classes (EMPTY, PARTIAL, FULL) in one call
    log("[fwd many tiles]")
    n, P, hq, hkv, d = 11, 96, 4, 2, 128
    parts = [gen(600, synthetic.T_Q, i, (1, P, hq, d)) for i in range(n)]
    kparts = [gen(600, synthetic.T_K, i, (1, P, hkv, d)) for i in range(n)]
    vparts = [gen(600, synthetic.T_V, i, (1, P, hkv, d)) for i in range(n)]
    tiles, refs = [], []
    for i in range(n):
        j = (i * 5) % n
        o = torch.empty((1, P, hq, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((1, hq, P), dtype=torch.float32, device=DEV)
        qp, kp = Pos([(0, i * P, 1)]), Pos([(0, j * P, 1)])
        tiles.append(Tile(parts[i][0], kparts[j][0], vparts[j][0], o, lse, qp, kp))
        refs.append(attn_tile(parts[i][1], kparts[j][1], vparts[j][1], np.float32(0.1), None, True,
                              positions(qp, P), positions(kp, P)))
    run_fwd(tiles, 0.1, ma.MA_MASK_CAUSAL)
    for t, (Oref, Lref) in zip(tiles, refs):
        check_close("O", host_f64(t.o), Oref, BF16_O_TOL, normalised_also=False)
        check_close("LSE", host_f64(t.lse), Lref, BF16_LSE_TOL)


@pytest.mark.parametrize("dtype,mode", [("bf16", "causal"), ("bf16", "striped"), ("bf16", "none"), ("f32", "striped")])
def test_many_tiles_in_one_call(dtype, mode):
    """64 tiles of one call (8 x 8 partitions of 40 tokens, GQA 4/2, d = 64) cross the batches of
    tiles one launch holds, FULL and PARTIAL tiles interleaved (and EMPTY ones skipped), each
    tile's (O, LSE) checked against the oracle."""
    log(f"[many tiles] {dtype} {mode}")
    n, P, hq, hkv, d = 8, 40, 4, 2, 64
    mask = {"causal": ma.MA_MASK_CAUSAL, "striped": ma.MA_MASK_STRIPED_ZIGZAG, "none": ma.MA_MASK_NONE}[mode]
    scale = np.float32(0.125)
    qs = [gen(1500 + n, synthetic.T_Q, i, (1, P, hq, d), dtype) for i in range(n)]
    ks = [gen(1500 + n, synthetic.T_K, j, (1, P, hkv, d), dtype) for j in range(n)]
    vs = [gen(1500 + n, synthetic.T_V, j, (1, P, hkv, d), dtype) for j in range(n)]
    pos = (lambda i: ma.mesh_attn_pos_striped(n, i)) if mode == "striped" else (lambda i: Pos([(0, i * P, 1)]))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tiles, refs = [], []
    for i in range(n):
        for j in range(n):
            qp, kp = pos(i), pos(j)
            if mode != "none" and ma.mesh_attn_classify(qp, P, kp, P, mask) == ma.MA_TILE_EMPTY:
                continue
            o = torch.full((1, P, hq, d), float("nan"), dtype=tdt, device=DEV)
            lse = torch.full((1, hq, P), float("nan"), dtype=torch.float32, device=DEV)
            tiles.append(Tile(qs[i][0], ks[j][0], vs[j][0], o, lse, qp, kp))
            causal = mode != "none"
            refs.append(attn_tile(qs[i][1], ks[j][1], vs[j][1], scale, None, causal,
                                  positions(qp, P) if causal else None, positions(kp, P) if causal else None))
    assert len(tiles) > 30
    run_fwd(tiles, float(scale), mask)
    tol_o, tol_l = (BF16_O_TOL, BF16_LSE_TOL) if dtype == "bf16" else (F32_TOL, F32_TOL)
    for t, (Oref, Lref) in zip(tiles, refs):
        check_close("O", host_f64(t.o), Oref, tol_o, normalised_also=False)
        check_close("LSE", host_f64(t.lse), Lref, tol_l)


def test_fp32_mha_s256_four_partitions():
    # fp32, 1 head, d=64, S=256 in 4 partitions of 64: all 16 tiles, then a 4-way merge per Q partition,
    # compared with unsplit attention (tolerance 1e-5 on O and LSE).
    log("[fp32 s256 n4]")
    S, n, d = 256, 4, 64
    P = S // n
    q, qv = gen(1, synthetic.T_Q, 0, (1, S, 1, d), "f32")
    k, kv = gen(1, synthetic.T_K, 0, (1, S, 1, d), "f32")
    v, vv = gen(1, synthetic.T_V, 0, (1, S, 1, d), "f32")
    scale = np.float32(1.0 / math.sqrt(d))
    tiles = []
    for i in range(n):
        for j in range(n):
            o = torch.empty((1, P, 1, d), dtype=torch.float32, device=DEV)
            lse = torch.empty((1, 1, P), dtype=torch.float32, device=DEV)
            tiles.append(Tile(q[:, i * P:(i + 1) * P], k[:, j * P:(j + 1) * P], v[:, j * P:(j + 1) * P], o, lse))
    run_fwd(tiles, float(scale), ma.MA_MASK_NONE)
    for i in range(n):
        for j in range(n):
            Oref, Lref = attn_tile(qv[:, i * P:(i + 1) * P], kv[:, j * P:(j + 1) * P], vv[:, j * P:(j + 1) * P], scale)
            t = tiles[i * n + j]
            check_close(f"O[{i},{j}]", host_f64(t.o), Oref, F32_TOL, normalised_also=False)
            check_close(f"LSE[{i},{j}]", host_f64(t.lse), Lref, F32_TOL)
    Ofull, Lfull = attn_tile(qv, kv, vv, scale)
    for i in range(n):
        o_out = torch.empty((1, P, 1, d), dtype=torch.float32, device=DEV)
        l_out = torch.empty((1, 1, P), dtype=torch.float32, device=DEV)
        row = tiles[i * n:(i + 1) * n]
        ma.mesh_attn_merge([t.o for t in row], [t.lse for t in row], o_out, l_out)
        torch.cuda.synchronize()
        check_close(f"merged O[{i}]", host_f64(o_out), Ofull[:, i * P:(i + 1) * P], F32_TOL, normalised_also=False)
        check_close(f"merged LSE[{i}]", host_f64(l_out), Lfull[:, :, i * P:(i + 1) * P], F32_TOL)


@pytest.mark.parametrize("k,dtype,d,H", [(1, "bf16", 128, 3), (2, "bf16", 64, 3), (6, "bf16", 128, 3),
                                         (27, "bf16", 128, 3), (64, "bf16", 128, 3), (5, "f32", 64, 3),
                                         (9, "f32", 128, 3), (3, "bf16", 128, 4), (12, "bf16", 64, 6),
                                         (2, "f32", 128, 2), (10, "f32", 64, 4)])
def test_merge_matches_oracle(k, dtype, d, H):
    """Odd head counts take one head per workgroup tile, even ones head pairs; 77 rows leave a ragged tile."""
    B, S = 2, 77
    log(f"[merge] k={k} dtype={dtype} d={d} H={H}")
    wid = 700 + k + 100 * (H % 2 == 0)
    Os, Ls, Oh, Lh = [], [], [], []
    for r in range(k):
        o, ov = gen(wid, synthetic.T_O_IN, r, (B, S, H, d), dtype)
        lv = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, r, (B, H, S)) * 3 + 10).astype(np.float32)
        if r == 1:  # rows that one partial did not reach
            lv[:, 0, :10] = -np.inf
        if r < 3 and k > 3:
            lv[:, 1, 5] = -np.inf
        Os.append(o); Oh.append(ov)
        Ls.append(torch.from_numpy(lv).to(DEV)); Lh.append(lv.astype(np.float64))
    if k > 3:  # one row with every partial empty
        for r in range(k):
            Ls[r][0, 2, 7] = float("-inf"); Lh[r][0, 2, 7] = -np.inf
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o_out = torch.empty((B, S, H, d), dtype=tdt, device=DEV)
    l_out = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    ma.mesh_attn_merge(Os, Ls, o_out, l_out)
    torch.cuda.synchronize()
    Oref, Lref = merge(list(zip(Oh, Lh)))
    tol_o, tol_l = (BF16_O_TOL, BF16_LSE_TOL) if dtype == "bf16" else (F32_TOL, F32_TOL)
    check_close("O", host_f64(o_out), Oref, tol_o, normalised_also=False)
    check_close("LSE", host_f64(l_out), Lref, tol_l)
    if k > 3:
        assert torch.all(o_out[0, 7, 2].float() == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_merge_head_major_strides(d):
    """Partials and output as (B, H, S, d) storage seen through [B, S, H, d] views (row stride d,
    head stride S*d): the kernel follows the strides it is given."""
    B, S, H, k = 2, 45, 4, 5
    log(f"[merge head-major strides] d={d}")
    Os, Ls, Oh, Lh = [], [], [], []
    for r in range(k):
        o, ov = gen(900 + d, synthetic.T_O_IN, r, (B, S, H, d))
        Os.append(o.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3))
        Oh.append(ov)
        lv = (synthetic.normal_f32(900 + d, synthetic.T_LSE_IN, r, (B, H, S)) * 2 + 4).astype(np.float32)
        Ls.append(torch.from_numpy(lv).to(DEV)); Lh.append(lv.astype(np.float64))
    o_out = torch.empty((B, H, S, d), dtype=torch.bfloat16, device=DEV).permute(0, 2, 1, 3)
    l_out = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    ma.mesh_attn_merge(Os, Ls, o_out, l_out)
    torch.cuda.synchronize()
    Oref, Lref = merge(list(zip(Oh, Lh)))
    check_close("O", host_f64(o_out), Oref, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(l_out), Lref, BF16_LSE_TOL)


def test_merge_in_place():
    log("[merge in place]")
    B, S, H, d, k = 1, 50, 2, 128, 4
    Os, Ls, Oh, Lh = [], [], [], []
    for r in range(k):
        o, ov = gen(800, synthetic.T_O_IN, r, (B, S, H, d))
        lv = synthetic.normal_f32(800, synthetic.T_LSE_IN, r, (B, H, S)) + 5
        Os.append(o); Oh.append(ov); Ls.append(torch.from_numpy(lv).to(DEV)); Lh.append(lv.astype(np.float64))
    Oref, Lref = merge(list(zip(Oh, Lh)))
    ma.mesh_attn_merge(Os, Ls, Os[0], Ls[0])
    torch.cuda.synchronize()
    check_close("O", host_f64(Os[0]), Oref, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(Ls[0]), Lref, BF16_LSE_TOL)


def _ring_case(wid, P, n, hq, hkv, d, dtype):
    """One query partition (positions 3P..4P) and n KV partitions at positions jP..(j+1)P."""
    q, qv = gen(wid, synthetic.T_Q, 3, (1, P, hq, d), dtype)
    ks = [gen(wid, synthetic.T_K, j, (1, P, hkv, d), dtype) for j in range(n)]
    vs = [gen(wid, synthetic.T_V, j, (1, P, hkv, d), dtype) for j in range(n)]
    return q, qv, ks, vs


@pytest.mark.parametrize("dtype,d,mode,one_call", [("bf16", 128, ma.MA_MASK_CAUSAL, False),
                                                    ("bf16", 64, ma.MA_MASK_CAUSAL, True),
                                                    ("bf16", 128, ma.MA_MASK_NONE, True),
                                                    ("f32", 64, ma.MA_MASK_CAUSAL, False)])
def test_fwd_accumulate_ring_equals_unsplit(dtype, d, mode, one_call):
    # ring order 3, 4, 5, 0, 1, 2 around a query partition at positions [3P, 4P): under the causal
    # mask tile 3 is PARTIAL (the diagonal), 4 and 5 are EMPTY (no-ops when accumulating) and 0-2 FULL.
    P, n, hq, hkv = 200, 6, 8, 2
    log(f"[fwd accumulate ring] dtype={dtype} d={d} mode={mode} one_call={one_call}")
    q, qv, ks, vs = _ring_case(900 + d, P, n, hq, hkv, d, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = torch.full((1, P, hq, d), float("nan"), dtype=tdt, device=DEV)
    lse = torch.full((1, hq, P), float("nan"), dtype=torch.float32, device=DEV)
    qp = Pos([(0, 3 * P, 1)])
    order = [3, 4, 5, 0, 1, 2]
    tiles = [Tile(q, ks[j][0], vs[j][0], o, lse, qp, Pos([(0, j * P, 1)])) for j in order]
    scale = 1.0 / math.sqrt(d)
    if one_call:
        o.zero_()
        lse.fill_(float("-inf"))
        ma.mesh_attn_tile_fwd(tiles, scale, mode, accumulate=True)
    else:
        ma.mesh_attn_tile_fwd(tiles[:1], scale, mode)
        for t in tiles[1:]:
            ma.mesh_attn_tile_fwd([t], scale, mode, accumulate=True)
    torch.cuda.synchronize()
    kall = np.concatenate([ks[j][1] for j in range(n)], axis=1)
    vall = np.concatenate([vs[j][1] for j in range(n)], axis=1)
    causal = mode != ma.MA_MASK_NONE
    Oref, Lref = attn_tile(qv, kall, vall, np.float32(scale), None, causal,
                           positions(qp, P) if causal else None, np.arange(n * P, dtype=np.int64) if causal else None)
    tol_o, tol_l = (BF16_O_TOL, BF16_LSE_TOL) if dtype == "bf16" else (F32_TOL, F32_TOL)
    check_close("O", host_f64(o), Oref, tol_o, normalised_also=False)
    check_close("LSE", host_f64(lse), Lref, tol_l)


def test_fwd_accumulate_into_incoming_partial():
    # the buffers start with a seeded incoming partial (with rows at -inf); the result must be the
    # oracle merge of that partial with the tile's own attention
    B, P, hq, hkv, d = 1, 150, 4, 1, 128
    log("[fwd accumulate incoming]")
    (q, k, v, o, lse), (qv, kv, vv) = make_case(950, P, 300, hq, hkv, d)
    o_in, ov = gen(950, synthetic.T_O_IN, 0, (B, P, hq, d))
    lv = (synthetic.normal_f32(950, synthetic.T_LSE_IN, 0, (B, hq, P)) + 6).astype(np.float32)
    lv[0, 1, :20] = -np.inf
    ov[0, :20, 1] = 0.0
    o_in[0, :20, 1] = 0
    o.copy_(o_in)
    lse.copy_(torch.from_numpy(lv))
    qp, kp = Pos([(0, 100, 1)]), Pos([(0, 0, 1)])  # causal: query rows 0..149 see keys up to 100+t
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, qp, kp)], 0.08, ma.MA_MASK_CAUSAL, accumulate=True)
    torch.cuda.synchronize()
    Ot, Lt = attn_tile(qv, kv, vv, np.float32(0.08), None, True, positions(qp, P), positions(kp, 300))
    Oref, Lref = merge([(ov, lv.astype(np.float64)), (Ot, Lt)])
    check_close("O", host_f64(o), Oref, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(lse), Lref, BF16_LSE_TOL)


@pytest.mark.parametrize("d,acc", [(128, False), (64, False), (128, True)])
def test_small_tiles_mixed_call(d, acc):
    """30 small tiles in one call, the case of the resident-KV and four-wave kernels: 22 tiles of
    [CHARM+]'s smallest partition size (210 x 210, GQA 32/8) with tiles of one key block (48 keys), a
    single query row, the four-wave kernel's 16-block limit (1000 keys) and ragged sizes, every tensor
    a prefix view of a longer buffer (shared strides), more workgroups than two per CU; optionally
    folded into seeded incoming partials.  Every row of every tile is checked against the oracle."""
    hq, hkv = 32, 8
    scale = np.float32(1.0 / math.sqrt(d))
    shapes = [(210, 210)] * 22 + [(210, 48), (37, 48), (64, 64), (100, 130), (210, 1000), (1, 5), (33, 210),
                                  (210, 65)]
    log(f"[small tiles mixed call] d={d} acc={acc} tiles={len(shapes)}")
    wid = 2600 + d + (1 if acc else 0)
    smax = 1024  # every tensor is a prefix view of a buffer of this length, so all tiles share strides

    def view(t, axis_len, kind):
        shape = (1, smax, t.shape[2], t.shape[3]) if kind == "bshd" else (1, t.shape[1], smax)
        buf = torch.full(shape, float("nan"), dtype=t.dtype, device=DEV)
        v = buf[:, :axis_len] if kind == "bshd" else buf[:, :, :axis_len]
        v.copy_(t)
        return v

    tiles, refs = [], []
    for i, (sq, sk) in enumerate(shapes):
        q, qv = gen(wid, synthetic.T_Q, i, (1, sq, hq, d))
        k, kv = gen(wid, synthetic.T_K, i, (1, sk, hkv, d))
        v, vv = gen(wid, synthetic.T_V, i, (1, sk, hkv, d))
        O, L = attn_tile(qv, kv, vv, scale)
        if acc:
            ob, ov = gen(wid, synthetic.T_O_IN, i, (1, sq, hq, d))
            li = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, i, (1, hq, sq)) + np.float32(math.log(sk))).astype(
                np.float32)
            o, lse = ob, torch.from_numpy(li).to(DEV)
            O, L = merge([(ov, li.astype(np.float64)), (O, L)])
        else:
            o = torch.full((1, sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            lse = torch.full((1, hq, sq), float("nan"), dtype=torch.float32, device=DEV)
        tiles.append(Tile(view(q, sq, "bshd"), view(k, sk, "bshd"), view(v, sk, "bshd"), view(o, sq, "bshd"),
                          view(lse, sq, "bhs")))
        refs.append((O, L))
    assert sum(((sq + 31) // 32 * (hq // hkv) + 3) // 4 * hkv for sq, _ in shapes) > 2 * 256
    ma.mesh_attn_tile_fwd(tiles, float(scale), ma.MA_MASK_NONE, accumulate=acc)
    torch.cuda.synchronize()
    for t, (Oref, Lref) in zip(tiles, refs):
        check_close("O", host_f64(t.o), Oref, BF16_O_TOL, normalised_also=False)
        check_close("LSE", host_f64(t.lse), Lref, BF16_LSE_TOL)


# (d, sq, sk, hq, hkv, batch, head_map): unmasked bf16 tiles of the resident-KV kernel's range
# (128 < sk <= 256 keys at d = 128, sk <= 512 at d = 64) and the sizes just outside it
RESIDENT_CASES = [
    (128, 1100, 129, 32, 8, 1, None),  # 35 row blocks x 4 heads: five chunks of 32 units per KV head
    (128, 300, 210, 32, 8, 1, None),   # [CHARM+]'s smallest partition size, ragged last block
    (128, 2, 256, 8, 2, 2, None),      # one row block: most waves have no unit; full last block
    (128, 77, 257, 4, 4, 1, None),     # one key past the range (ring kernel)
    (128, 64, 128, 8, 4, 1, None),     # the last size below it (ring kernel)
    (64, 500, 1, 8, 2, 1, None),       # a single key
    (64, 300, 511, 6, 3, 2, [0, 0, 0, 1, 2, 2]),  # groups of 3, 1 and 2 query heads
    (64, 33, 512, 16, 2, 1, None),
    (64, 40, 513, 16, 2, 1, None),     # one key past the range
]


@pytest.mark.parametrize("table", [False, True])
@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("case", range(len(RESIDENT_CASES)))
def test_fwd_resident_kv_tiles(case, acc, table):
    """Two tiles of one shape in one call, plain or folded into seeded incoming partials; every row
    of both checked against the oracle.  Through the tile table the two tiles share one K/V, so
    they form one group whose units the workgroups take across the tile boundary."""
    d, sq, sk, hq, hkv, B, head_map = RESIDENT_CASES[case]
    log(f"[fwd resident kv] d={d} sq={sq} sk={sk} hq={hq} hkv={hkv} B={B} acc={acc} table={table}")
    scale = np.float32(1.0 / math.sqrt(d))
    wid = 2700 + 2 * case + (1 if acc else 0)
    tiles, refs = [], []
    for i in range(2):
        q, qv = gen(wid, synthetic.T_Q, i, (B, sq, hq, d))
        if i == 0 or not table:
            k, kv = gen(wid, synthetic.T_K, i, (B, sk, hkv, d))
            v, vv = gen(wid, synthetic.T_V, i, (B, sk, hkv, d))
        O, L = attn_tile(qv, kv, vv, scale, head_map)
        if acc:
            o, ov = gen(wid, synthetic.T_O_IN, i, (B, sq, hq, d))
            li = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, i, (B, hq, sq)) + np.float32(math.log(sk + 1))).astype(
                np.float32)
            lse = torch.from_numpy(li).to(DEV)
            O, L = merge([(ov, li.astype(np.float64)), (O, L)])
        else:
            o = torch.full((B, sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            lse = torch.full((B, hq, sq), float("nan"), dtype=torch.float32, device=DEV)
        tiles.append(Tile(q, k, v, o, lse))
        refs.append((O, L))
    ma.mesh_attn_tile_fwd(tiles, float(scale), ma.MA_MASK_NONE, head_map, accumulate=acc, table=table)
    torch.cuda.synchronize()
    for t, (Oref, Lref) in zip(tiles, refs):
        check_close("O", host_f64(t.o), Oref, BF16_O_TOL, normalised_also=False)
        check_close("LSE", host_f64(t.lse), Lref, BF16_LSE_TOL)


def _tile_set(wid, shapes, hq, hkv, d, acc, shared=(), kv_of=None):
    """Tiles of the given (sq, sk) shapes with seeded inputs; with acc, outputs hold seeded incoming
    partials (two identical copies of every output: for the table path and the kernel-argument path).
    `shared` lists groups of tile indices that name one output (applied in list order); kv_of[i],
    when given, is the tile whose K and V tile i uses (the same tensors; equal sk)."""
    owner = {}
    for grp in shared:
        for i in grp[1:]:
            owner[i] = grp[0]
    smax = max(max(sq, sk) for sq, sk in shapes)  # every tensor a prefix view of a buffer this long

    def view(t, n, kind):
        shape = (1, smax, t.shape[2], t.shape[3]) if kind == "bshd" else (1, t.shape[1], smax)
        buf = torch.full(shape, float("nan"), dtype=t.dtype, device=DEV)
        out = buf[:, :n] if kind == "bshd" else buf[:, :, :n]
        out.copy_(t)
        return out

    ins, outs = [], [[], []]
    for i, (sq, sk) in enumerate(shapes):
        q, qv = gen(wid, synthetic.T_Q, i, (1, sq, hq, d))
        if kv_of is not None and kv_of[i] != i:
            j = kv_of[i]
            assert j < i and shapes[j][1] == sk
            ins.append((view(q, sq, "bshd"), ins[j][1], ins[j][2], qv, ins[j][4], ins[j][5]))
        else:
            k, kv = gen(wid, synthetic.T_K, i, (1, sk, hkv, d))
            v, vv = gen(wid, synthetic.T_V, i, (1, sk, hkv, d))
            ins.append((view(q, sq, "bshd"), view(k, sk, "bshd"), view(v, sk, "bshd"), qv, kv, vv))
        for c in range(2):
            if i in owner:
                outs[c].append(outs[c][owner[i]])
                continue
            if acc:
                o, ov = gen(wid, synthetic.T_O_IN, i, (1, sq, hq, d))
                li = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, i, (1, hq, sq)) + np.float32(math.log(sk))).astype(
                    np.float32)
                outs[c].append((view(o, sq, "bshd"), view(torch.from_numpy(li).to(DEV), sq, "bhs"), ov,
                                li.astype(np.float64)))
            else:
                outs[c].append((view(torch.full((1, sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV), sq,
                                     "bshd"),
                                view(torch.full((1, hq, sq), float("nan"), dtype=torch.float32, device=DEV), sq, "bhs"),
                                None, None))
    tiles = [[Tile(x[0], x[1], x[2], o[0], o[1]) for x, o in zip(ins, outs[c])] for c in range(2)]
    return ins, outs, tiles


@pytest.mark.parametrize("d,acc", [(128, False), (64, False), (128, True)])
def test_fwd_tile_table_matches_kernel_arguments(d, acc):
    """One call of 100 tiles through mesh_attn_tile_fwd_tabled (the resident-KV tiles from a device
    table, one launch for all of them) and through mesh_attn_tile_fwd (launches of at most 30 tiles
    from kernel arguments): bitwise equal.  Tiles outside the resident class are mixed in, and with
    accumulate two groups of tiles name one output each, so the table launch is cut where they
    repeat; sampled tiles and the shared outputs are checked against the oracle."""
    hq, hkv = 32, 8
    scale = np.float32(1.0 / math.sqrt(d))
    res = 210 if d == 128 else 400
    shapes = [(res, res)] * 92 + [(res, 64), (37, 1000), (300, 129), (256, 256), (1, 200), (97, res), (res, 33),
                                  (64, 257)]
    shared = ((5, 6, 7), (40, 41)) if acc else ()
    log(f"[fwd tile table] d={d} acc={acc} tiles={len(shapes)}")
    ins, outs, tiles = _tile_set(2800 + d + (1 if acc else 0), shapes, hq, hkv, d, acc, shared)
    ma.mesh_attn_tile_fwd(tiles[0], float(scale), ma.MA_MASK_NONE, accumulate=acc, table=True)
    ma.mesh_attn_tile_fwd(tiles[1], float(scale), ma.MA_MASK_NONE, accumulate=acc)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(tiles[0][i].o, tiles[1][i].o) and torch.equal(tiles[0][i].lse, tiles[1][i].lse), i
    firsts = {g[0]: g for g in shared}
    skip = {i for g in shared for i in g[1:]}
    for i in [0, 5, 40, 91, 92, 94, 95, 97]:
        if i in skip:
            continue
        grp = firsts.get(i, (i,))
        parts = [attn_tile(ins[j][3], ins[j][4], ins[j][5], scale) for j in grp]
        if acc:
            parts = [(outs[0][i][2], outs[0][i][3])] + parts
        Oref, Lref = merge(parts) if len(parts) > 1 else parts[0]
        check_close(f"O tile {i}", host_f64(tiles[0][i].o), Oref, BF16_O_TOL, normalised_also=False)
        check_close(f"LSE tile {i}", host_f64(tiles[0][i].lse), Lref, BF16_LSE_TOL)


@pytest.mark.parametrize("d,acc", [(128, False), (64, False), (128, True)])
def test_fwd_tile_table_groups_tiles_sharing_kv(d, acc):
    """A Mesh-like block: 12 query partitions of ragged lengths against 3 KV partitions (36 tiles,
    every KV partition shared by 12 tiles), through the tile table, where the tiles of one KV
    partition form a group and a workgroup runs units of several tiles against one LDS copy of
    K/V, and through kernel arguments: bitwise equal, and sampled tiles against the oracle."""
    hq, hkv = 32, 8
    scale = np.float32(1.0 / math.sqrt(d))
    sqs = [210, 37, 300, 1, 129, 256, 64, 500, 33, 210, 97, 2000]
    sks = [210, 256, 150] if d == 128 else [400, 512, 3]
    shapes, kv_of = [], []
    for j, sk in enumerate(sks):
        for i, sq in enumerate(sqs):
            kv_of.append(len(shapes) if i == 0 else j * len(sqs))
            shapes.append((sq, sk))
    # with accumulate, tiles 0 and 9 (one K/V, rows 210 both) and tiles 9 and 21 (query partition 9
    # against two K/V) name one output each, applied in list order: the table call is cut there
    shared = ((0, 9, 21),) if acc else ()
    log(f"[fwd tile table groups] d={d} acc={acc} tiles={len(shapes)}")
    ins, outs, tiles = _tile_set(2860 + d + (1 if acc else 0), shapes, hq, hkv, d, acc, shared, kv_of)
    ma.mesh_attn_tile_fwd(tiles[0], float(scale), ma.MA_MASK_NONE, accumulate=acc, table=True)
    ma.mesh_attn_tile_fwd(tiles[1], float(scale), ma.MA_MASK_NONE, accumulate=acc)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(tiles[0][i].o, tiles[1][i].o) and torch.equal(tiles[0][i].lse, tiles[1][i].lse), i
    skip = {i for g in shared for i in g[1:]}
    for i in [0, 1, 3, 11, 13, 20, 23, 26, 35]:
        if i in skip:
            continue
        grp = shared[0] if shared and i == shared[0][0] else (i,)
        parts = [attn_tile(ins[j][3], ins[j][4], ins[j][5], scale) for j in grp]
        if acc:
            parts = [(outs[0][i][2], outs[0][i][3])] + parts
        O, L = merge(parts) if len(parts) > 1 else parts[0]
        check_close(f"O tile {i}", host_f64(tiles[0][i].o), O, BF16_O_TOL, normalised_also=False)
        check_close(f"LSE tile {i}", host_f64(tiles[0][i].lse), L, BF16_LSE_TOL)


@pytest.mark.parametrize("acc", [False, True])
def test_fwd_tile_table_under_a_causal_mask(acc):
    """A causal 6 x 6 block of 210-token partitions (contiguous positions): the 15 tiles below the
    diagonal are FULL and run from the tile table (groups of up to five tiles per KV partition),
    the 6 diagonal tiles are PARTIAL and run the masked kernel from kernel arguments, the 15 above
    are EMPTY (filled with (0, -inf), or left as they are with accumulate).  The tabled call must
    equal the kernel-argument call bitwise; sampled tiles of each class against the oracle."""
    hq, hkv, d, P, n = 32, 8, 128, 210, 6
    scale = np.float32(1.0 / math.sqrt(d))
    wid = 2870 + (1 if acc else 0)
    log(f"[fwd tile table causal] acc={acc}")
    qs = [gen(wid, synthetic.T_Q, i, (1, P, hq, d)) for i in range(n)]
    ks = [gen(wid, synthetic.T_K, j, (1, P, hkv, d)) for j in range(n)]
    vs = [gen(wid, synthetic.T_V, j, (1, P, hkv, d)) for j in range(n)]
    pos = [Pos([(0, i * P, 1)]) for i in range(n)]
    tiles, incoming = [[], []], {}
    for i in range(n):
        for j in range(n):
            for c in range(2):
                if acc:
                    o, ov = gen(wid, synthetic.T_O_IN, i * n + j, (1, P, hq, d))
                    li = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, i * n + j, (1, hq, P)) +
                          np.float32(math.log(P))).astype(np.float32)
                    incoming[(i, j)] = (ov, li.astype(np.float64))
                    lse = torch.from_numpy(li).to(DEV)
                else:
                    o = torch.full((1, P, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
                    lse = torch.full((1, hq, P), float("nan"), dtype=torch.float32, device=DEV)
                tiles[c].append(Tile(qs[i][0], ks[j][0], vs[j][0], o, lse, q_pos=pos[i], k_pos=pos[j]))
    ma.mesh_attn_tile_fwd(tiles[0], float(scale), ma.MA_MASK_CAUSAL, accumulate=acc, table=True)
    ma.mesh_attn_tile_fwd(tiles[1], float(scale), ma.MA_MASK_CAUSAL, accumulate=acc)
    torch.cuda.synchronize()
    for t0, t1 in zip(tiles[0], tiles[1]):
        assert torch.equal(t0.o, t1.o) and torch.equal(t0.lse, t1.lse)
    for i, j in [(1, 0), (5, 2), (3, 3), (0, 0), (2, 4)]:  # FULL, FULL, PARTIAL, PARTIAL, EMPTY
        t = tiles[0][i * n + j]
        if j > i:  # no allowed pair
            if acc:
                O, L = incoming[(i, j)]
            else:
                O, L = np.zeros((1, P, hq, d)), np.full((1, hq, P), -np.inf)
        else:
            O, L = attn_tile(qs[i][1], ks[j][1], vs[j][1], scale, None, True,
                             positions(pos[i], P), positions(pos[j], P))
            if acc:
                O, L = merge([incoming[(i, j)], (O, L)])
        check_close(f"O tile ({i},{j})", host_f64(t.o), O, BF16_O_TOL, normalised_also=False)
        check_close(f"LSE tile ({i},{j})", host_f64(t.lse), L, BF16_LSE_TOL)


def test_fwd_tile_table_with_no_resident_tile():
    """A tabled call whose tiles are all outside the resident-KV class (the table holds only its
    header): the same launches as mesh_attn_tile_fwd, bitwise."""
    hq, hkv, d = 32, 8, 128
    scale = np.float32(1.0 / math.sqrt(d))
    shapes = [(300, 600), (64, 1000), (1, 64), (210, 840)]
    log("[fwd tile table] no resident tile")
    _, _, tiles = _tile_set(2880, shapes, hq, hkv, d, False)
    prep = ma.prepare_tile_fwd(tiles[0], float(scale), ma.MA_MASK_NONE, table=True)
    assert prep[3][2] == 32  # the header only
    ma.launch_prepared_tile_fwd(prep)
    ma.mesh_attn_tile_fwd(tiles[1], float(scale), ma.MA_MASK_NONE)
    torch.cuda.synchronize()
    for t0, t1 in zip(tiles[0], tiles[1]):
        assert torch.equal(t0.o, t1.o) and torch.equal(t0.lse, t1.lse)
        assert not torch.isnan(t0.o.float()).any()


def test_fwd_tile_table_of_other_arguments_is_not_run():
    """A device table packed for one set of tiles, handed to the call of another set of the same
    shapes: the resident-KV launch finds the header's hash different and writes nothing (the
    outputs keep their NaN fill); the call with its own table then computes them."""
    from distributed_long_context_amd import _abi
    import ctypes as C
    hq, hkv, d = 32, 8, 128
    scale = float(np.float32(1.0 / math.sqrt(d)))
    shapes = [(210, 210)] * 12
    log("[fwd tile table] stale table")
    _, _, ta = _tile_set(2850, shapes, hq, hkv, d, False)
    _, _, tb = _tile_set(2851, shapes, hq, hkv, d, False)
    pa = ma.prepare_tile_fwd(ta[0], scale, ma.MA_MASK_NONE, table=True)
    pb = ma.prepare_tile_fwd(tb[0], scale, ma.MA_MASK_NONE, table=True)
    _, dev_a, n_a = pa[3]
    L = _abi.lib()
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.mesh_attn_tile_fwd_tabled(C.byref(pb[0]), C.c_void_p(dev_a.data_ptr()), n_a, s) == _abi.MA_OK
    torch.cuda.synchronize()
    for t in tb[0]:
        assert torch.isnan(t.o.float()).all() and torch.isnan(t.lse).all()
    for t in ta[0]:  # the tiles the table was packed for are not touched either
        assert torch.isnan(t.o.float()).all()
    ma.launch_prepared_tile_fwd(pb)
    ma.mesh_attn_tile_fwd(tb[1], scale, ma.MA_MASK_NONE)
    torch.cuda.synchronize()
    for t0, t1 in zip(tb[0], tb[1]):
        assert torch.equal(t0.o, t1.o) and torch.equal(t0.lse, t1.lse)
