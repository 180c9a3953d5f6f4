"""Pins for the oracle's tile backward (CPU only): finite differences, closed forms, decompositions."""
import numpy as np
import pytest

from oracle import attn_tile, attn_tile_bwd, attn_bwd_multi, merge, reduce_add
from oracle import layout

RNG = np.random.default_rng(99)


def _loss(q, k, v, do, scale, hm, causal, qp, kp):
    O, _ = attn_tile(q, k, v, scale, hm, causal, qp, kp)
    return float((O * do).sum())


MASKS = [
    (False, None, None),
    (True, layout.contiguous(3), layout.contiguous(0)),
    (True, layout.striped(2, 1), layout.striped(2, 0)),
]


@pytest.mark.parametrize("causal,qseg,kseg", MASKS)
@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2)])
def test_backward_matches_central_differences(causal, qseg, kseg, hq, hkv):
    B, Sq, Sk, d = 1, 5, 6, 3
    q = RNG.standard_normal((B, Sq, hq, d)); k = RNG.standard_normal((B, Sk, hkv, d)); v = RNG.standard_normal((B, Sk, hkv, d))
    do = RNG.standard_normal((B, Sq, hq, d))
    scale = 0.8
    qp = layout.expand_positions(qseg, Sq) if causal else None
    kp = layout.expand_positions(kseg, Sk) if causal else None
    O, L = attn_tile(q, k, v, scale, None, causal, qp, kp)
    dq, dk, dv = attn_tile_bwd(q, k, v, O, do, L, scale, None, causal, qp, kp)
    eps = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            x0 = X[idx]
            X[idx] = x0 + eps; fp = _loss(q, k, v, do, scale, None, causal, qp, kp)
            X[idx] = x0 - eps; fm = _loss(q, k, v, do, scale, None, causal, qp, kp)
            X[idx] = x0
            num[idx] = (fp - fm) / (2 * eps)
        err = np.max(np.abs(num - G)) / max(1.0, np.max(np.abs(G)))
        assert err < 1e-7, err


def test_constant_v_zero_dq_dk():
    # Closed form: constant V makes dP = D, so dS = 0 and dQ = dK = 0.
    q = RNG.standard_normal((1, 7, 2, 4)); k = RNG.standard_normal((1, 9, 1, 4))
    v = np.broadcast_to(RNG.standard_normal(4), (1, 9, 1, 4)).copy(); do = RNG.standard_normal((1, 7, 2, 4))
    O, L = attn_tile(q, k, v, 0.5)
    dq, dk, dv = attn_tile_bwd(q, k, v, O, do, L, 0.5)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    # dV of each key is then its softmax weight times the summed dO of the group
    P = np.exp(0.5 * np.einsum("thd,ud->htu", q[0], k[0, :, 0]) - L[0][:, :, None])
    assert np.max(np.abs(dv[0, :, 0] - np.einsum("htu,thd->ud", P, do[0]))) < 1e-13


def test_single_key_gradients():
    # Closed form: one key -> P = 1, dQ = dK = 0, dV_0 = sum_t dO_t over every head of the group.
    q = RNG.standard_normal((1, 6, 4, 3)); k = RNG.standard_normal((1, 1, 2, 3)); v = RNG.standard_normal((1, 1, 2, 3))
    do = RNG.standard_normal((1, 6, 4, 3))
    O, L = attn_tile(q, k, v, 1.1)
    dq, dk, dv = attn_tile_bwd(q, k, v, O, do, L, 1.1)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    assert np.max(np.abs(dv[0, 0, 0] - do[0, :, 0:2].sum(axis=(0, 1)))) < 1e-13
    assert np.max(np.abs(dv[0, 0, 1] - do[0, :, 2:4].sum(axis=(0, 1)))) < 1e-13


def test_q_split_sums_to_unsplit():
    # Summing dK/dV over any split of the query rows equals the unsplit gradient.
    q = RNG.standard_normal((1, 12, 2, 3)); k = RNG.standard_normal((1, 8, 1, 3)); v = RNG.standard_normal((1, 8, 1, 3))
    do = RNG.standard_normal((1, 12, 2, 3))
    O, L = attn_tile(q, k, v, 0.6)
    dq, dk, dv = attn_tile_bwd(q, k, v, O, do, L, 0.6)
    tiles = [dict(q=q[:, s], o=O[:, s], do=do[:, s], lse=L[:, :, s]) for s in (slice(0, 5), slice(5, 6), slice(6, 12))]
    dqs, dk2, dv2 = attn_bwd_multi(tiles, k, v, 0.6)
    assert np.max(np.abs(np.concatenate(dqs, axis=1) - dq)) < 1e-14
    assert np.max(np.abs(dk2 - dk)) < 1e-13 and np.max(np.abs(dv2 - dv)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_kv_partition_shares_sum_to_full_gradient(causal):
    # [Mesh] section 3.5 decomposition: per-(Q_i, KV_j) backward with the row's final O and LSE
    # gives partial dQ that sum over KV partitions, and dK/dV slices of the full gradient.
    Sq, Sk, n = 10, 12, 3
    q = RNG.standard_normal((1, Sq, 2, 3)); k = RNG.standard_normal((1, Sk, 2, 3)); v = RNG.standard_normal((1, Sk, 2, 3))
    do = RNG.standard_normal((1, Sq, 2, 3))
    qp = layout.expand_positions(layout.contiguous(6), Sq) if causal else None
    kp = layout.expand_positions(layout.contiguous(0), Sk) if causal else None
    O, L = attn_tile(q, k, v, 0.9, None, causal, qp, kp)
    dq, dk, dv = attn_tile_bwd(q, k, v, O, do, L, 0.9, None, causal, qp, kp)
    # the row's final (O, L) is also what merging the per-partition partials gives
    b = Sk // n
    parts = [attn_tile(q, k[:, j*b:(j+1)*b], v[:, j*b:(j+1)*b], 0.9, None, causal, qp, None if kp is None else kp[j*b:(j+1)*b]) for j in range(n)]
    Om, Lm = merge(parts)
    assert np.max(np.abs(Om - O)) < 1e-13
    dq_sum = np.zeros_like(dq)
    for j in range(n):
        sl = slice(j * b, (j + 1) * b)
        dqj, dkj, dvj = attn_tile_bwd(q, k[:, sl], v[:, sl], O, do, L, 0.9, None, causal, qp, None if kp is None else kp[sl])
        dq_sum += dqj
        assert np.max(np.abs(dkj - dk[:, sl])) < 1e-13 and np.max(np.abs(dvj - dv[:, sl])) < 1e-13
    assert np.max(np.abs(dq_sum - dq)) < 1e-13


def test_fully_masked_rows_have_zero_gradient():
    q = RNG.standard_normal((1, 4, 1, 2)); k = RNG.standard_normal((1, 5, 1, 2)); v = RNG.standard_normal((1, 5, 1, 2))
    do = RNG.standard_normal((1, 4, 1, 2))
    qp = layout.expand_positions(layout.contiguous(0), 4); kp = layout.expand_positions(layout.contiguous(2), 5)
    O, L = attn_tile(q, k, v, 1.0, None, True, qp, kp)
    assert np.isinf(L[0, 0, :2]).all()
    dq, dk, dv = attn_tile_bwd(q, k, v, O, do, L, 1.0, None, True, qp, kp)
    assert np.all(dq[0, :2] == 0) and np.isfinite(dk).all() and np.isfinite(dv).all()


def test_reduce_add_is_exact_on_integers():
    # small integers are exact in float64, so the sum must equal Python's integer sum
    parts = [np.arange(12).reshape(3, 4) * (r + 1) - 7 * r for r in range(5)]
    want = [[sum(int(p[i, j]) for p in parts) for j in range(4)] for i in range(3)]
    assert np.array_equal(reduce_add(parts), np.array(want, dtype=np.float64))
    assert np.array_equal(reduce_add(parts[:1]), parts[0].astype(np.float64))


def test_reduce_add_of_kv_partials_gives_unsplit_dq():
    # [Mesh] section 3.5: partial dQ of each (Q_i, KV_j) pair, added, is the gradient of the whole row
    Sq, Sk, n = 9, 12, 4
    q = RNG.standard_normal((1, Sq, 2, 3)); k = RNG.standard_normal((1, Sk, 1, 3)); v = RNG.standard_normal((1, Sk, 1, 3))
    do = RNG.standard_normal((1, Sq, 2, 3))
    O, L = attn_tile(q, k, v, 0.7)
    dq, _, _ = attn_tile_bwd(q, k, v, O, do, L, 0.7)
    b = Sk // n
    parts = [attn_tile_bwd(q, k[:, j*b:(j+1)*b], v[:, j*b:(j+1)*b], O, do, L, 0.7)[0] for j in range(n)]
    assert np.max(np.abs(reduce_add(parts) - dq)) < 1e-13
    # dropping one partial must be visible
    assert np.max(np.abs(reduce_add(parts[1:]) - dq)) > 1e-3
