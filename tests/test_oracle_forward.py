"""Pins for the oracle's forward tile and merge (CPU only).

Each check compares the oracle with something other than itself: a pure-Python
brute force that materialises the softmax row, closed forms, or the invariant
that merging partials over any KV split equals unsplit attention.
"""
import math
import itertools

import numpy as np
import pytest

from oracle import attn_tile, merge
from oracle import layout

RNG = np.random.default_rng(1234)


def brute_force(q, k, v, scale, head_map, q_pos=None, k_pos=None):
    """Triple loop with math.exp, softmax normalised by its own sum (no max shift)."""
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kv = head_map[h]
            for t in range(Sq):
                keys = [u for u in range(Sk) if q_pos is None or k_pos[u] <= q_pos[t]]
                if not keys:
                    L[b][h][t] = -math.inf
                    continue
                ex = {}
                for u in keys:
                    s = 0.0
                    for c in range(d):
                        s += float(q[b, t, h, c]) * float(k[b, u, kv, c])
                    ex[u] = math.exp(scale * s)
                z = sum(ex.values())
                L[b][h][t] = math.log(z)
                for c in range(d):
                    O[b][t][h][c] = sum(ex[u] / z * float(v[b, u, kv, c]) for u in keys)
    return np.array(O), np.array(L)


MASK_CASES = [
    ("none", None, None),
    ("causal_offset", layout.contiguous(5), layout.contiguous(0)),
    ("causal_same", layout.contiguous(0), layout.contiguous(0)),
    ("causal_future", layout.contiguous(0), layout.contiguous(3)),
    ("striped", layout.striped(3, 1), layout.striped(3, 2)),
    ("zigzag", [(0, 0, 1), (3, 20, 1)], [(0, 2, 1), (4, 17, 2)]),
]


@pytest.mark.parametrize("mask", MASK_CASES, ids=[m[0] for m in MASK_CASES])
@pytest.mark.parametrize("hq,hkv,head_map", [(1, 1, None), (4, 2, None), (3, 2, [1, 0, 1])])
def test_forward_matches_brute_force(mask, hq, hkv, head_map):
    name, qseg, kseg = mask
    B, Sq, Sk, d = 2, 7, 9, 3
    q = RNG.standard_normal((B, Sq, hq, d))
    k = RNG.standard_normal((B, Sk, hkv, d))
    v = RNG.standard_normal((B, Sk, hkv, d))
    scale = 0.7
    hm = head_map if head_map is not None else [h // (hq // hkv) for h in range(hq)]
    causal = qseg is not None
    qp = layout.expand_positions(qseg, Sq) if causal else None
    kp = layout.expand_positions(kseg, Sk) if causal else None
    O, L = attn_tile(q, k, v, scale, head_map, causal, qp, kp)
    Ob, Lb = brute_force(q, k, v, scale, hm, qp, kp)
    assert np.array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    assert np.max(np.abs(L[fin] - Lb[fin]), initial=0.0) < 1e-12
    assert np.max(np.abs(O - Ob)) < 1e-12
    # fully masked rows are exactly (0, -inf)
    for b, h, t in zip(*np.nonzero(~fin)):
        assert np.all(O[b, t, h] == 0.0) and L[b, h, t] == -np.inf


def test_rows_subset_equals_full():
    q = RNG.standard_normal((1, 40, 2, 4)); k = RNG.standard_normal((1, 33, 1, 4)); v = RNG.standard_normal((1, 33, 1, 4))
    qp = layout.expand_positions(layout.contiguous(10), 40); kp = layout.expand_positions(layout.contiguous(0), 33)
    O, L = attn_tile(q, k, v, 0.5, None, True, qp, kp)
    rows = [0, 3, 39, 17]
    Os, Ls = attn_tile(q, k, v, 0.5, None, True, qp, kp, rows=rows)
    assert np.array_equal(Os, O[:, rows]) and np.array_equal(Ls, L[:, :, rows])


def test_constant_v_gives_v():
    # Closed form: v[u] = c for every key -> O[t] = c whenever a key is allowed.
    q = RNG.standard_normal((1, 11, 2, 5)) * 3; k = RNG.standard_normal((1, 13, 2, 5)) * 3
    c = RNG.standard_normal(5)
    v = np.broadcast_to(c, (1, 13, 2, 5)).copy()
    qp = layout.expand_positions(layout.contiguous(4), 11); kp = layout.expand_positions(layout.contiguous(0), 13)
    O, L = attn_tile(q, k, v, 0.3, None, True, qp, kp)
    assert np.isfinite(L).all()
    assert np.max(np.abs(O - c)) < 1e-13


def test_single_key():
    # Closed form: one key -> weight 1, O = v_0, LSE = s_00.
    q = RNG.standard_normal((1, 6, 3, 4)); k = RNG.standard_normal((1, 1, 3, 4)); v = RNG.standard_normal((1, 1, 3, 4))
    O, L = attn_tile(q, k, v, 0.9, [0, 1, 2], False)
    for h in range(3):
        assert np.max(np.abs(O[0, :, h] - v[0, 0, h])) < 1e-15
        s = 0.9 * (q[0, :, h] @ k[0, 0, h])
        assert np.max(np.abs(L[0, h] - s)) < 1e-14


@pytest.mark.parametrize("qseg,kseg", [(layout.contiguous(0), layout.contiguous(0)),
                                       (layout.striped(4, 3), layout.striped(4, 1)),
                                       ([(0, 0, 1), (6, 40, 1)], layout.contiguous(0))])
def test_zero_q_counts_allowed_keys(qseg, kseg):
    # Closed form: all scores 0 -> LSE[t] = ln(n_t), O[t] = mean of the allowed V rows.
    Sq, Sk = 12, 45
    q = np.zeros((1, Sq, 1, 4)); k = RNG.standard_normal((1, Sk, 1, 4)); v = RNG.standard_normal((1, Sk, 1, 4))
    qp = layout.expand_positions(qseg, Sq); kp = layout.expand_positions(kseg, Sk)
    O, L = attn_tile(q, k, v, 1.0, None, True, qp, kp)
    for t in range(Sq):
        keys = [u for u in range(Sk) if kp[u] <= qp[t]]
        if keys:
            assert abs(L[0, 0, t] - math.log(len(keys))) < 1e-14
            assert np.max(np.abs(O[0, t, 0] - v[0, keys, 0].mean(axis=0))) < 1e-14
        else:
            assert L[0, 0, t] == -np.inf and np.all(O[0, t, 0] == 0)


def _split_merge(q, k, v, scale, splits, causal=False, qp=None, kp=None, hm=None):
    parts = []
    for idx in splits:
        idx = np.asarray(idx, dtype=np.int64)
        if len(idx) == 0:
            B, Sq, Hq, d = q.shape
            parts.append((np.zeros(q.shape), np.full((B, Hq, Sq), -np.inf)))
            continue
        parts.append(attn_tile(q, k[:, idx], v[:, idx], scale, hm, causal, qp, None if kp is None else kp[idx]))
    return merge(parts)


@pytest.mark.parametrize("causal", [False, True])
def test_split_merge_equals_unsplit(causal):
    # Invariant: merging partials over any partition of the keys equals unsplit attention.
    B, Sq, Sk, d = 1, 16, 40, 6
    q = RNG.standard_normal((B, Sq, 4, d)); k = RNG.standard_normal((B, Sk, 2, d)); v = RNG.standard_normal((B, Sk, 2, d))
    qp = layout.expand_positions(layout.contiguous(20), Sq) if causal else None
    kp = layout.expand_positions(layout.contiguous(0), Sk) if causal else None
    ref_O, ref_L = attn_tile(q, k, v, 0.4, None, causal, qp, kp)
    perm = RNG.permutation(Sk)
    for splits in ([perm[:13], perm[13:14], perm[14:], []], [perm[i::5] for i in range(5)], [np.arange(Sk)]):
        O, L = _split_merge(q, k, v, 0.4, splits, causal, qp, kp)
        assert np.max(np.abs(O - ref_O)) < 1e-13
        fin = np.isfinite(ref_L)
        assert np.array_equal(fin, np.isfinite(L))
        assert np.max(np.abs(L[fin] - ref_L[fin]), initial=0.0) < 1e-13
        # merge order does not matter
        parts = []
        for idx in splits:
            if len(idx):
                parts.append(attn_tile(q, k[:, idx], v[:, idx], 0.4, None, causal, qp, None if kp is None else kp[idx]))
        for order in itertools.islice(itertools.permutations(range(len(parts))), 6):
            O2, L2 = merge([parts[i] for i in order])
            assert np.max(np.abs(O2 - O)) < 1e-13


def test_ring_simulation_exactness_magnitude():
    # The ring-attention page simulates S=512, d=64, n=8 in float64 and reports a max abs error of
    # about 1e-15 against full attention.  The same experiment through the oracle's tile + merge:
    S, d, n = 512, 64, 8
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((1, S, 1, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d)
    full_O, _ = attn_tile(Q, K, V, scale)
    b = S // n
    for r in range(n):
        parts = [attn_tile(Q[:, r * b:(r + 1) * b], K[:, j * b:(j + 1) * b], V[:, j * b:(j + 1) * b], scale) for j in range(n)]
        O, _ = merge(parts)
        assert np.max(np.abs(O - full_O[:, r * b:(r + 1) * b])) < 1e-13


def test_merge_identities():
    B, S, H, d = 1, 5, 2, 3
    O1 = RNG.standard_normal((B, S, H, d)); L1 = RNG.standard_normal((B, H, S))
    ninf = np.full((B, H, S), -np.inf)
    # merge with an empty partial is the identity
    O, L = merge([(O1, L1), (RNG.standard_normal((B, S, H, d)), ninf)])
    assert np.max(np.abs(O - O1)) < 1e-15 and np.max(np.abs(L - L1)) < 1e-15
    # merging a partial with itself keeps O and adds ln 2 to the LSE
    O, L = merge([(O1, L1), (O1, L1)])
    assert np.max(np.abs(O - O1)) < 1e-15 and np.max(np.abs(L - (L1 + math.log(2)))) < 1e-14
    # all inputs empty -> (0, -inf), no NaN
    O, L = merge([(O1, ninf), (O1, ninf)])
    assert np.all(O == 0) and np.all(L == -np.inf)
    # weights by hand: lse 0 and ln 3 -> weights 1/4 and 3/4, lse = ln 4
    Oa = np.ones((1, 1, 1, 1)); Ob = np.full((1, 1, 1, 1), 5.0)
    O, L = merge([(Oa, np.zeros((1, 1, 1))), (Ob, np.full((1, 1, 1), math.log(3)))])
    assert abs(O.item() - (0.25 + 3.75)) < 1e-15 and abs(L.item() - math.log(4)) < 1e-15


def test_merge_large_lse_offsets_stay_finite():
    # Weights come from LSE differences, so very large LSEs must not overflow.
    O1 = np.ones((1, 1, 1, 2)); O2 = np.full((1, 1, 1, 2), 3.0)
    O, L = merge([(O1, np.full((1, 1, 1), 800.0)), (O2, np.full((1, 1, 1), 800.0))])
    assert np.allclose(O, 2.0) and abs(L.item() - (800 + math.log(2))) < 1e-12
