"""The C++ mapper (through the C ABI) against the oracle's brute-force mapper, bit-exact (CPU only)."""
import numpy as np
import pytest

import distributed_long_context_amd as ma
from distributed_long_context_amd import Pos
from oracle import layout

FACTORS = [(n, a, n // a) for n in (1, 4, 6, 9, 15, 16, 64) for a in range(1, n + 1) if n % a == 0]


@pytest.mark.parametrize("n,a,b", FACTORS)
def test_mesh_tiles_and_groups_match_assignment_matrix(n, a, b):
    for kvr in (False, True):
        A = layout.assignment_matrix(n, a, b, "kvr" if kvr else "basic")
        for g in range(n):
            qs, ks = ma.mesh_attn_map_mesh_tile(n, a, b, g, kvr)
            assert (qs, ks) == layout.mesh_tile(n, a, b, g, kvr)
            IQ, IKV, _, _ = layout.footprint(A, g)
            assert sorted(qs) == IQ and sorted(ks) == IKV
    for g in range(n):
        qg, kg = ma.mesh_attn_map_groups(n, a, b, g)
        assert qg == layout.q_group(n, a, b, g) and kg == layout.kv_group(n, a, b, g)


def test_mesh_tile_rejects_bad_factorisation():
    with pytest.raises(ma.MeshAttnError):
        ma.mesh_attn_map_mesh_tile(16, 3, 5, 0)
    with pytest.raises(ma.MeshAttnError):
        ma.mesh_attn_map_mesh_tile(16, 4, 4, 16)


@pytest.mark.parametrize("N", [1, 2, 5, 16, 64])
def test_zigzag_and_striped(N):
    for r in range(N):
        assert ma.mesh_attn_map_zigzag(N, r) == layout.zigzag_chunks(N, r)
        c = 5
        p = ma.mesh_attn_pos_zigzag(N, r, c)
        got = [ma.mesh_attn_pos_at(p, t) for t in range(2 * c)]
        assert got == list(layout.expand_positions(layout.zigzag_rank_positions(N, r, c), 2 * c))
        s = ma.mesh_attn_pos_striped(N, r)
        assert [ma.mesh_attn_pos_at(s, t) for t in range(7)] == list(layout.expand_positions(layout.striped(N, r), 7))
    assert [ma.mesh_attn_pos_at(ma.mesh_attn_pos_contiguous(37), t) for t in range(4)] == [37, 38, 39, 40]


def _random_pos(rng, length):
    nseg = int(rng.integers(1, 5))
    cuts = sorted(rng.choice(np.arange(1, length), size=min(nseg - 1, length - 1), replace=False)) if length > 1 else []
    lbs = [0] + [int(c) for c in cuts]
    return Pos([(lb, int(rng.integers(0, 60)), int(rng.integers(1, 4))) for lb in lbs])


def test_classify_and_count_match_enumeration():
    rng = np.random.default_rng(7)
    for _ in range(400):
        sq, sk = int(rng.integers(1, 20)), int(rng.integers(1, 20))
        qp, kp = _random_pos(rng, sq), _random_pos(rng, sk)
        qa = layout.expand_positions(qp.segments, sq)
        ka = layout.expand_positions(kp.segments, sk)
        assert ma.mesh_attn_classify(qp, sq, kp, sk, ma.MA_MASK_STRIPED_ZIGZAG) == layout.classify(qa, ka)
        assert ma.mesh_attn_count_allowed(qp, sq, kp, sk, ma.MA_MASK_STRIPED_ZIGZAG) == layout.allowed_count(qa, ka)
        assert [ma.mesh_attn_pos_at(qp, t) for t in range(sq)] == list(qa)
    assert ma.mesh_attn_classify(Pos([(0, 0, 1)]), 4, Pos([(0, 100, 1)]), 4, ma.MA_MASK_NONE) == ma.MA_TILE_FULL


def test_zigzag_share_worklist_and_pair_count():
    # Zigzag share of rank 5 of 16 at S = 131072 (32 chunks of 4096) against every KV chunk.
    N, r, C = 16, 5, 4096
    q_pos = [ma.mesh_attn_pos_contiguous(c * C) for c in ma.mesh_attn_map_zigzag(N, r)]
    k_pos = [ma.mesh_attn_pos_contiguous(j * C) for j in range(2 * N)]
    wl = ma.mesh_attn_build_worklist(q_pos, [C, C], k_pos, [C] * (2 * N), ma.MA_MASK_CAUSAL)
    ref = layout.worklist([layout.expand_positions(p.segments, C) for p in q_pos],
                          [layout.expand_positions(p.segments, C) for p in k_pos])
    assert wl == ref and len(wl) == 33
    total = sum(ma.mesh_attn_count_allowed(q_pos[i], C, k_pos[j], C, ma.MA_MASK_CAUSAL) for i, j, _ in wl)
    assert total == 536_875_008


def test_mesh_share_64_gpus():
    # One GPU of n = 64 (8 x 8 tile with KV partition rotation): GPU 9 -> Q 8..15, KV {1, 9, ..., 57}.
    qs, ks = ma.mesh_attn_map_mesh_tile(64, 8, 8, 9, True)
    assert qs == list(range(8, 16)) and ks == [1 + 8 * t for t in range(8)]
    assert (qs, ks) == layout.mesh_tile(64, 8, 8, 9, True)
