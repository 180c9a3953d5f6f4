"""Seeded random sweep of the forward and backward against the fp64 oracle (through the C ABI).

Each case draws its shape, batch, GQA map, head dim, mask mode and position map (contiguous,
striped, or two to four segments) from a fixed seed, so the sweep is the same on every run;
the tolerances are the ones of the other parity tests.
"""
import math
import random

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import BwdTile, Pos, Tile  # noqa: E402
from oracle import attn_tile, attn_tile_bwd, merge  # noqa: E402
from gpu_helpers import BF16_LSE_TOL, BF16_O_TOL, DEV, check_close, gen, host_f64, log, positions  # noqa: E402
from test_gpu_bwd import check_grad, stored_o_lse  # noqa: E402

import synthetic  # noqa: E402


def _segments(rng, n, base):
    """One to four segments over n local tokens with random global starts and strides."""
    cuts = sorted(rng.sample(range(1, n), min(n - 1, rng.randint(0, 3)))) if n > 1 else []
    lbs = [0] + cuts
    segs = []
    g = base
    for lb in lbs:
        st = rng.choice([1, 1, 2, 3])
        segs.append((lb, g, st))
        g += rng.randint(0, 400)
    return Pos(segs)


def _case(seed):
    rng = random.Random(seed)
    hq, hkv = rng.choice([(4, 4), (8, 2), (8, 1), (6, 3), (4, 2)])
    d = rng.choice([64, 128])
    B = rng.choice([1, 1, 2])
    # key counts on both sides of the forward's switch between its four-wave (at most 1024 keys)
    # and eight-wave instances
    sq, sk = rng.randint(1, 260), (rng.randint(1, 330) if rng.random() < 0.7 else rng.randint(1025, 1400))
    kind = rng.choice(["none", "causal", "striped", "segments"])
    if kind == "none":
        return dict(hq=hq, hkv=hkv, d=d, B=B, sq=sq, sk=sk, mode=ma.MA_MASK_NONE, qp=None, kp=None)
    if kind == "causal":
        qb, kb = rng.randint(0, 400), rng.randint(0, 400)
        return dict(hq=hq, hkv=hkv, d=d, B=B, sq=sq, sk=sk, mode=ma.MA_MASK_CAUSAL, qp=Pos([(0, qb, 1)]),
                    kp=Pos([(0, kb, 1)]))
    if kind == "striped":
        N = rng.choice([2, 4, 8])
        return dict(hq=hq, hkv=hkv, d=d, B=B, sq=sq, sk=sk, mode=ma.MA_MASK_STRIPED_ZIGZAG,
                    qp=ma.mesh_attn_pos_striped(N, rng.randrange(N)), kp=ma.mesh_attn_pos_striped(N, rng.randrange(N)))
    return dict(hq=hq, hkv=hkv, d=d, B=B, sq=sq, sk=sk, mode=ma.MA_MASK_STRIPED_ZIGZAG,
                qp=_segments(rng, sq, rng.randint(0, 300)), kp=_segments(rng, sk, 0))


# seed 72: four key segments folded into an incoming partial with |O| near 3.5; when the segments
# of a tile were separate folds, each rounding O to bf16, its error reached 0.021 (bar 0.02)
@pytest.mark.parametrize("seed", list(range(120)))
def test_random_forward(seed):
    c = _case(1000 + seed)
    log(f"[random fwd {seed}] {c}")
    B, sq, sk, hq, hkv, d = c["B"], c["sq"], c["sk"], c["hq"], c["hkv"], c["d"]
    wid = 2000 + seed
    q, qv = gen(wid, synthetic.T_Q, 0, (B, sq, hq, d))
    k, kv = gen(wid, synthetic.T_K, 0, (B, sk, hkv, d))
    v, vv = gen(wid, synthetic.T_V, 0, (B, sk, hkv, d))
    scale = np.float32(1.0 / math.sqrt(d))
    causal = c["mode"] != ma.MA_MASK_NONE
    qpos = positions(c["qp"], sq) if causal else None
    kpos = positions(c["kp"], sk) if causal else None
    Oref, Lref = attn_tile(qv, kv, vv, scale, None, causal, qpos, kpos)
    o = torch.full((B, sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, hq, sq), float("nan"), dtype=torch.float32, device=DEV)
    accumulate = seed % 3 == 0
    if accumulate:  # fold into a seeded incoming partial
        oi, oiv = gen(wid, synthetic.T_O_IN, 0, (B, sq, hq, d))
        li = (synthetic.normal_f32(wid, synthetic.T_LSE_IN, 0, (B, hq, sq)) + 4).astype(np.float32)
        o.copy_(oi)
        lse.copy_(torch.from_numpy(li))
        Oref, Lref = merge([(oiv, li.astype(np.float64)), (Oref, Lref)])
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, c["qp"], c["kp"])], float(scale), c["mode"], accumulate=accumulate)
    torch.cuda.synchronize()
    check_close("O", host_f64(o), Oref, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(lse), Lref, BF16_LSE_TOL)


@pytest.mark.parametrize("seed", range(100))
def test_random_backward(seed):
    c = _case(3000 + seed)
    log(f"[random bwd {seed}] {c}")
    B, sq, sk, hq, hkv, d = c["B"], c["sq"], c["sk"], c["hq"], c["hkv"], c["d"]
    wid = 4000 + seed
    q, qv = gen(wid, synthetic.T_Q, 0, (B, sq, hq, d))
    k, kv = gen(wid, synthetic.T_K, 0, (B, sk, hkv, d))
    v, vv = gen(wid, synthetic.T_V, 0, (B, sk, hkv, d))
    do, dov = gen(wid, synthetic.T_DO, 0, (B, sq, hq, d))
    scale = np.float32(1.0 / math.sqrt(d))
    causal = c["mode"] != ma.MA_MASK_NONE
    qpos = positions(c["qp"], sq) if causal else None
    kpos = positions(c["kp"], sk) if causal else None
    O, L = attn_tile(qv, kv, vv, scale, None, causal, qpos, kpos)
    o_dev, o_used, l_dev, l_used = stored_o_lse(O, L)
    dq = torch.full((B, sq, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full((B, sk, hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full_like(dk, float("nan"))
    ma.mesh_attn_tile_bwd([BwdTile(q, k, v, o_dev, do, l_dev, dq, dk, dv, c["qp"], c["kp"])], float(scale), c["mode"])
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = attn_tile_bwd(qv, kv, vv, o_used, dov, l_used, scale, None, causal, qpos, kpos)
    check_grad("dQ", dq, dq_r)
    check_grad("dK", dk, dk_r)
    check_grad("dV", dv, dv_r)


@pytest.mark.parametrize("seed", range(24))
def test_random_head_map(seed):
    """Irregular explicit GQA maps (groups of unequal size, KV heads no query head reads):
    forward and backward of one drawn tile."""
    rng = random.Random(7000 + seed)
    c = _case(90000 + seed)
    hkv = rng.randint(1, 6)
    hq = rng.randint(hkv, 12)
    hm = [rng.randrange(hkv) for _ in range(hq)]
    log(f"[random head map {seed}] hq={hq} hkv={hkv} map={hm} {c}")
    B, sq, sk, d = c["B"], c["sq"], c["sk"], c["d"]
    wid = 6000 + seed
    q, qv = gen(wid, synthetic.T_Q, 0, (B, sq, hq, d))
    k, kv = gen(wid, synthetic.T_K, 0, (B, sk, hkv, d))
    v, vv = gen(wid, synthetic.T_V, 0, (B, sk, hkv, d))
    scale = np.float32(1.0 / math.sqrt(d))
    causal = c["mode"] != ma.MA_MASK_NONE
    qpos = positions(c["qp"], sq) if causal else None
    kpos = positions(c["kp"], sk) if causal else None
    O, L = attn_tile(qv, kv, vv, scale, hm, causal, qpos, kpos)
    o = torch.full((B, sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, hq, sq), float("nan"), dtype=torch.float32, device=DEV)
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, c["qp"], c["kp"])], float(scale), c["mode"], hm)
    torch.cuda.synchronize()
    check_close("O", host_f64(o), O, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(lse), L, BF16_LSE_TOL)
    o_dev, o_used, l_dev, l_used = stored_o_lse(O, L)
    do, dov = gen(wid, synthetic.T_DO, 0, (B, sq, hq, d))
    dq = torch.full((B, sq, hq, d), float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full((B, sk, hkv, d), float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full_like(dk, float("nan"))
    ma.mesh_attn_tile_bwd([BwdTile(q, k, v, o_dev, do, l_dev, dq, dk, dv, c["qp"], c["kp"])], float(scale),
                          c["mode"], hm)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = attn_tile_bwd(qv, kv, vv, o_used, dov, l_used, scale, hm, causal, qpos, kpos)
    check_grad("dQ", dq, dq_r)
    check_grad("dK", dk, dk_r)
    check_grad("dV", dv, dv_r)


@pytest.mark.parametrize("seed", range(16))
def test_random_multi_tile_calls(seed):
    """One accumulate forward call over a random set of (Q partition, KV partition) pairs in random
    order, each folding into its Q partition's output, then one backward call over the same pairs
    (dQ summed per Q partition, dK/dV per KV partition).  Seeds 6-15 are wide calls (6-20
    partitions a side): more groups than one backward launch holds, partner sets split over
    launches."""
    rng = random.Random(8000 + seed)
    hkv = rng.choice([1, 2, 4])
    hq = hkv * rng.choice([1, 2, 4])
    d = rng.choice([64, 128])
    mode = rng.choice(["none", "causal", "striped"])
    mask = {"none": ma.MA_MASK_NONE, "causal": ma.MA_MASK_CAUSAL, "striped": ma.MA_MASK_STRIPED_ZIGZAG}[mode]
    nq, nk = rng.randint(1, 5), rng.randint(1, 12)
    P = rng.choice([16, 33, 64, 100, 129])
    if seed >= 6:
        nq, nk, P = rng.randint(6, 20), rng.randint(6, 20), rng.choice([16, 33, 64])
    log(f"[random multi-tile {seed}] hq={hq} hkv={hkv} d={d} {mode} nq={nq} nk={nk} P={P}")
    wid = 7100 + seed
    scale = np.float32(1.0 / math.sqrt(d))
    causal = mode != "none"
    n = max(nq, nk)
    pos = (lambda i: None) if not causal else (
        (lambda i: ma.mesh_attn_pos_striped(n, i)) if mode == "striped" else (lambda i: Pos([(0, i * P, 1)])))
    qs = [gen(wid, synthetic.T_Q, i, (1, P, hq, d)) for i in range(nq)]
    ks = [gen(wid, synthetic.T_K, j, (1, P, hkv, d)) for j in range(nk)]
    vs = [gen(wid, synthetic.T_V, j, (1, P, hkv, d)) for j in range(nk)]
    dos = [gen(wid, synthetic.T_DO, i, (1, P, hq, d)) for i in range(nq)]
    pairs = [(i, j) for i in range(nq) for j in range(nk) if rng.random() < 0.7] or [(0, 0)]
    rng.shuffle(pairs)
    qp, kp = [pos(i) for i in range(nq)], [pos(j) for j in range(nk)]
    outs = [(torch.zeros((1, P, hq, d), dtype=torch.bfloat16, device=DEV),
             torch.full((1, hq, P), float("-inf"), dtype=torch.float32, device=DEV)) for _ in range(nq)]
    ma.mesh_attn_tile_fwd([Tile(qs[i][0], ks[j][0], vs[j][0], outs[i][0], outs[i][1], qp[i], kp[j]) for i, j in pairs],
                          float(scale), mask, accumulate=True)
    torch.cuda.synchronize()
    refs = {}
    for i, j in pairs:
        refs.setdefault(i, []).append(attn_tile(qs[i][1], ks[j][1], vs[j][1], scale, None, causal,
                                                positions(qp[i], P) if causal else None,
                                                positions(kp[j], P) if causal else None))
    stored = {}
    for i in refs:
        Oref, Lref = merge(refs[i])
        check_close("O", host_f64(outs[i][0]), Oref, BF16_O_TOL, normalised_also=False)
        check_close("LSE", host_f64(outs[i][1]), Lref, BF16_LSE_TOL)
        stored[i] = stored_o_lse(Oref, Lref)
    dqs = [torch.full((1, P, hq, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(nq)]
    dks = [torch.full((1, P, hkv, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(nk)]
    dvs = [torch.full((1, P, hkv, d), float("nan"), dtype=torch.float32, device=DEV) for _ in range(nk)]
    ma.mesh_attn_tile_bwd([BwdTile(qs[i][0], ks[j][0], vs[j][0], stored[i][0], dos[i][0], stored[i][2], dqs[i], dks[j],
                                   dvs[j], qp[i], kp[j]) for i, j in pairs], float(scale), mask)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = {}, {}, {}
    for i, j in pairs:
        a, b, c = attn_tile_bwd(qs[i][1], ks[j][1], vs[j][1], stored[i][1], dos[i][1], stored[i][3], scale, None,
                                causal, positions(qp[i], P) if causal else None,
                                positions(kp[j], P) if causal else None)
        dq_r[i] = dq_r.get(i, 0) + a
        dk_r[j] = dk_r.get(j, 0) + b
        dv_r[j] = dv_r.get(j, 0) + c
    for i in dq_r:
        check_grad("dQ", dqs[i], dq_r[i])
    for j in dk_r:
        check_grad("dK", dks[j], dk_r[j])
        check_grad("dV", dvs[j], dv_r[j])


def _head_major(t):
    """The same values stored [B, H, S, d], viewed as [B, S, H, d] (explicit strides in the ABI)."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


@pytest.mark.parametrize("seed", range(8))
def test_random_head_major_layout(seed):
    """Forward and backward of a drawn tile with every [B, S, H, d] tensor in head-major storage."""
    c = _case(20000 + seed)
    log(f"[random head-major {seed}] {c}")
    B, sq, sk, hq, hkv, d = c["B"], c["sq"], c["sk"], c["hq"], c["hkv"], c["d"]
    wid = 21000 + seed
    q, qv = gen(wid, synthetic.T_Q, 0, (B, sq, hq, d))
    k, kv = gen(wid, synthetic.T_K, 0, (B, sk, hkv, d))
    v, vv = gen(wid, synthetic.T_V, 0, (B, sk, hkv, d))
    q, k, v = _head_major(q), _head_major(k), _head_major(v)
    scale = np.float32(1.0 / math.sqrt(d))
    causal = c["mode"] != ma.MA_MASK_NONE
    qpos = positions(c["qp"], sq) if causal else None
    kpos = positions(c["kp"], sk) if causal else None
    O, L = attn_tile(qv, kv, vv, scale, None, causal, qpos, kpos)
    o = _head_major(torch.full((B, sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV))
    lse = torch.full((B, hq, sq), float("nan"), dtype=torch.float32, device=DEV)
    ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, c["qp"], c["kp"])], float(scale), c["mode"])
    torch.cuda.synchronize()
    check_close("O", host_f64(o), O, BF16_O_TOL, normalised_also=False)
    check_close("LSE", host_f64(lse), L, BF16_LSE_TOL)
    o_dev, o_used, l_dev, l_used = stored_o_lse(O, L)
    do, dov = gen(wid, synthetic.T_DO, 0, (B, sq, hq, d))
    o_dev, do = _head_major(o_dev), _head_major(do)
    dq = _head_major(torch.full((B, sq, hq, d), float("nan"), dtype=torch.float32, device=DEV))
    dk = _head_major(torch.full((B, sk, hkv, d), float("nan"), dtype=torch.float32, device=DEV))
    dv = _head_major(torch.full((B, sk, hkv, d), float("nan"), dtype=torch.float32, device=DEV))
    ma.mesh_attn_tile_bwd([BwdTile(q, k, v, o_dev, do, l_dev, dq, dk, dv, c["qp"], c["kp"])], float(scale), c["mode"])
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = attn_tile_bwd(qv, kv, vv, o_used, dov, l_used, scale, None, causal, qpos, kpos)
    check_grad("dQ", dq, dq_r)
    check_grad("dK", dk, dk_r)
    check_grad("dV", dv, dv_r)


@pytest.mark.parametrize("seed", range(32))
def test_random_tile_table(seed):
    """A random Mesh-like call through the tile table and through kernel arguments: query and KV
    partitions of random lengths (mostly in the resident-KV range, some outside it), a random
    subset of their pairs, batch, GQA map (sometimes an irregular explicit one) and head dim; with
    accumulate every tile folds into its query partition's output, otherwise each tile has its
    own.  The two calls must agree bitwise; sampled outputs against the oracle."""
    rng = random.Random(9100 + seed)
    d = rng.choice([64, 128])
    hkv = rng.choice([1, 2, 4, 8])
    hq = hkv * rng.choice([1, 2, 4])
    hm = None
    if rng.random() < 0.3:
        hm = [rng.randrange(hkv) for _ in range(hq)]
    B = rng.choice([1, 1, 2])
    acc = rng.random() < 0.5
    lo, hi = (129, 256) if d == 128 else (1, 512)
    nq, nk = rng.randint(1, 6), rng.randint(1, 4)
    sqs = [rng.randint(1, 300) for _ in range(nq)]
    sks = [rng.randint(lo, hi) if rng.random() < 0.8 else rng.choice([64, 600]) for _ in range(nk)]
    pairs = [(i, j) for i in range(nq) for j in range(nk) if rng.random() < 0.8] or [(0, 0)]
    rng.shuffle(pairs)
    log(f"[random tile table {seed}] d={d} hq={hq} hkv={hkv} map={hm} B={B} acc={acc} sq={sqs} sk={sks} "
        f"pairs={len(pairs)}")
    wid = 9200 + seed
    scale = np.float32(1.0 / math.sqrt(d))
    smax = max(sqs + sks)

    def view(t, n, kind):  # every tensor a prefix of a buffer smax long: one set of strides per call
        shape = (B, smax, t.shape[2], t.shape[3]) if kind == "bshd" else (B, t.shape[1], smax)
        buf = torch.full(shape, float("nan"), dtype=t.dtype, device=DEV)
        out = buf[:, :n] if kind == "bshd" else buf[:, :, :n]
        out.copy_(t)
        return out

    def drawn(tensor, i, n, h):
        dev, host = gen(wid, tensor, i, (B, n, h, d))
        return view(dev, n, "bshd"), host

    qs = [drawn(synthetic.T_Q, i, sqs[i], hq) for i in range(nq)]
    ks = [drawn(synthetic.T_K, j, sks[j], hkv) for j in range(nk)]
    vs = [drawn(synthetic.T_V, j, sks[j], hkv) for j in range(nk)]

    def outputs():
        if acc:  # one (O, LSE) per query partition, starting from a seeded incoming partial
            outs = []
            for i in range(nq):
                o, _ = drawn(synthetic.T_O_IN, i, sqs[i], hq)
                li = synthetic.normal_f32(wid, synthetic.T_LSE_IN, i, (B, hq, sqs[i])) + np.float32(4)
                outs.append((o, view(torch.from_numpy(li.astype(np.float32)).to(DEV), sqs[i], "bhs")))
            return [outs[i] for i, _ in pairs]
        nan = float("nan")
        return [(view(torch.full((B, sqs[i], hq, d), nan, dtype=torch.bfloat16, device=DEV), sqs[i], "bshd"),
                 view(torch.full((B, hq, sqs[i]), nan, dtype=torch.float32, device=DEV), sqs[i], "bhs"))
                for i, _ in pairs]

    runs = []
    for table in (True, False):
        outs = outputs()
        tiles = [Tile(qs[i][0], ks[j][0], vs[j][0], o, lse) for (i, j), (o, lse) in zip(pairs, outs)]
        ma.mesh_attn_tile_fwd(tiles, float(scale), ma.MA_MASK_NONE, hm, accumulate=acc, table=table)
        runs.append(outs)
    torch.cuda.synchronize()
    for (o0, l0), (o1, l1) in zip(*runs):
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
    if acc:
        i = pairs[0][0]
        parts = [(gen(wid, synthetic.T_O_IN, i, (B, sqs[i], hq, d))[1],
                  (synthetic.normal_f32(wid, synthetic.T_LSE_IN, i, (B, hq, sqs[i])) + np.float32(4)).astype(
                      np.float64))]
        parts += [attn_tile(qs[i][1], ks[j][1], vs[j][1], scale, hm) for ii, j in pairs if ii == i]
        O, L = merge(parts)
        o, lse = runs[0][pairs.index(next(p for p in pairs if p[0] == i))]
        check_close("O", host_f64(o), O, BF16_O_TOL, normalised_also=False)
        check_close("LSE", host_f64(lse), L, BF16_LSE_TOL)
    else:
        for t in rng.sample(range(len(pairs)), min(2, len(pairs))):
            i, j = pairs[t]
            O, L = attn_tile(qs[i][1], ks[j][1], vs[j][1], scale, hm)
            check_close(f"O pair {pairs[t]}", host_f64(runs[0][t][0]), O, BF16_O_TOL, normalised_also=False)
            check_close(f"LSE pair {pairs[t]}", host_f64(runs[0][t][1]), L, BF16_LSE_TOL)
