"""fp64 oracle for the tile forward, the LSE merge and the tile backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Everything is float64,
unblocked and unfused beyond what the definitions state; inputs are upcast
exactly from their stored values (bf16 or fp32 bits -> float64).

Tensor layouts (same meaning as the C ABI, but plain NumPy arrays here):
  q, o, do : [B, Sq, Hq, d]
  k, v     : [B, Sk, Hkv, d]
  lse      : [B, Hq, Sq]          (natural log)
"""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 512  # rows per NumPy call; only bounds memory, changes no arithmetic


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _head_map(hq: int, hkv: int, head_map):
    """GQA head map: query head h reads KV head head_map[h].

    Default follows [Mesh] §4.8 (Evaluation with GQA): each group of g
    consecutive query heads shares one KV head, so kv(h) = floor(h / (Hq/Hkv)).
    """
    if head_map is not None:
        hm = np.asarray(head_map, dtype=np.int64)
        assert hm.shape == (hq,) and hm.min() >= 0 and hm.max() < hkv
        return hm
    assert hq % hkv == 0
    return np.arange(hq, dtype=np.int64) // (hq // hkv)


def _allowed(q_pos_rows, k_pos, causal: bool):
    """Mask on *global* positions: key u is allowed for query t iff pos_k(u) <= pos_q(t).

    [Mesh] §3.7 (causal masking: a token attends to itself and preceding tokens);
    [Ring] "Causal masks and load balancing" (token i attends to tokens <= i) and
    its note that masks must use global positions.  Non-causal: every key allowed.
    """
    if not causal:
        return None
    return np.asarray(k_pos, dtype=np.int64)[None, :] <= np.asarray(q_pos_rows, dtype=np.int64)[:, None]


def attn_tile(q, k, v, scale, head_map=None, causal=False, q_pos=None, k_pos=None, rows=None):
    """Partial attention of one (Q partition, KV partition) pair: returns (O, LSE).

    Definition ([Mesh] §2.1 softmax attention and §2.2, where one pair yields
    O_ij and lse_ij; LSE read as the natural log of the sum of exp of the scaled
    scores over the allowed keys):

      s[t,u]  = scale * sum_c q[t,c] k[u,c]
      LSE[t]  = log sum_{u allowed} exp(s[t,u])         (via the max m for range)
      O[t]    = sum_{u allowed} exp(s[t,u] - LSE[t]) v[u]
      a row with no allowed key: O[t] = 0, LSE[t] = -inf.

    ``rows`` optionally restricts the computation to the given query rows (each
    output row depends only on its own query row), returning arrays whose Sq
    axis has len(rows).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    hm = _head_map(Hq, Hkv, head_map)
    scale = float(scale)
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    if causal:
        q_pos = np.asarray(q_pos, dtype=np.int64)
        k_pos = np.asarray(k_pos, dtype=np.int64)
        assert q_pos.shape == (Sq,) and k_pos.shape == (Sk,)
    O = np.zeros((B, R, Hq, d))
    LSE = np.full((B, Hq, R), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kh = k[b, :, hm[h], :]
            vh = v[b, :, hm[h], :]
            for r0 in range(0, R, _ROW_CHUNK):
                rr = rows[r0:r0 + _ROW_CHUNK]
                s = scale * (q[b, rr, h, :] @ kh.T)                       # [r, Sk]
                allowed = _allowed(q_pos[rr] if causal else None, k_pos, causal)
                if allowed is None:
                    allowed = np.ones(s.shape, dtype=bool)
                n_allowed = allowed.sum(axis=1)
                has = n_allowed > 0
                m = np.where(allowed, s, -np.inf).max(axis=1)
                m = np.where(has, m, 0.0)
                e = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - m[:, None]), 0.0)
                l = e.sum(axis=1)
                lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
                o = (e @ vh) / np.where(has, l, 1.0)[:, None]
                O[b, r0:r0 + len(rr), h, :] = np.where(has[:, None], o, 0.0)
                LSE[b, h, r0:r0 + len(rr)] = lse
    return O, LSE


def merge(parts):
    """Fold partial (O, LSE) pairs over disjoint KV sets into one (O, LSE).

    [Mesh] §2.2 (online softmax rescales partial outputs by their LSE before
    accumulating) and §3.3 (online softmax as the reduce-scatter reducer);
    [Ring] "Ring Attention: Pass KV Blocks Around the Ring" (running max,
    denominator and output; order does not matter).  Closed form of that
    recurrence:

      L* = max_r lse_r;   lse = L* + log sum_r exp(lse_r - L*)
      O  = sum_r exp(lse_r - lse) O_r
      all inputs -inf  ->  O = 0, lse = -inf.

    parts: list of (O [B,S,H,d], LSE [B,H,S]).
    """
    Os = [_f64(o) for o, _ in parts]
    Ls = np.stack([_f64(l) for _, l in parts])                          # [k,B,H,S]
    Lstar = Ls.max(axis=0)
    fin = np.isfinite(Lstar)
    Lb = np.where(fin, Lstar, 0.0)
    tot = np.exp(Ls - Lb[None]).sum(axis=0)
    lse = np.where(fin, Lb + np.log(np.where(fin, tot, 1.0)), -np.inf)
    lse_b = np.where(fin, lse, 0.0)
    O = np.zeros_like(Os[0])
    for r, o in enumerate(Os):
        w = np.where(fin, np.exp(Ls[r] - lse_b), 0.0)                    # [B,H,S]
        O += np.transpose(w, (0, 2, 1))[..., None] * o
    return O, lse


def reduce_add(parts):
    """Element-wise sum of partial gradient buffers, in float64.

    [Mesh] §3.5: the per-pair backward leaves partial dQ_i (one per KV partition
    met) and partial dKV_j (one per Q partition met) that are combined by a
    reduce-scatter whose operation is addition.  parts: list of equal-shape arrays.
    """
    out = np.zeros(np.shape(parts[0]), dtype=np.float64)
    for p in parts:
        out = out + _f64(p)
    return out


def attn_tile_bwd(q, k, v, o, do, lse, scale, head_map=None, causal=False, q_pos=None, k_pos=None):
    """Gradients of one pair's attention given the stored O, LSE and dO.

    [Mesh] §3.5: the backward kernel is invoked per pair with (Q_i, KV_j, O_i,
    dO_i) and yields partial dQ_i and dKV_j that are summed.  The pages print no
    formula; this is the derivative of the forward definition with
    P = exp(s - LSE) on allowed entries:

      D[t]   = sum_c dO[t,c] O[t,c]
      dP     = dO[t] . v[u];      dS = P (dP - D[t])
      dQ[t]  = scale sum_u dS k[u]
      dK[u]  = scale sum_{t, h in group(kv)} dS q[t]
      dV[u]  = sum_{t, h in group(kv)} P dO[t]

    With O and LSE taken over a larger KV set than this tile (a distributed
    row), the same formulas give this KV partition's share of the gradient.
    Returns float64 (dq [B,Sq,Hq,d], dk [B,Sk,Hkv,d], dv [B,Sk,Hkv,d]).
    """
    q, k, v, o, do, lse = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do), _f64(lse)
    B, Sq, Hq, d = q.shape
    _, Sk, Hkv, _ = k.shape
    hm = _head_map(Hq, Hkv, head_map)
    scale = float(scale)
    if causal:
        q_pos = np.asarray(q_pos, dtype=np.int64)
        k_pos = np.asarray(k_pos, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    Dall = (do * o).sum(axis=-1)                                          # [B,Sq,Hq]
    for b in range(B):
        for h in range(Hq):
            kv = hm[h]
            kh, vh = k[b, :, kv, :], v[b, :, kv, :]
            for r0 in range(0, Sq, _ROW_CHUNK):
                rr = np.arange(r0, min(Sq, r0 + _ROW_CHUNK))
                s = scale * (q[b, rr, h, :] @ kh.T)
                allowed = _allowed(q_pos[rr] if causal else None, k_pos, causal)
                if allowed is None:
                    allowed = np.ones(s.shape, dtype=bool)
                L = lse[b, h, rr]
                fin = np.isfinite(L)
                allowed = allowed & fin[:, None]
                P = np.where(allowed, np.exp(np.where(allowed, s - np.where(fin, L, 0.0)[:, None], 0.0)), 0.0)
                dP = do[b, rr, h, :] @ vh.T
                dS = P * (dP - Dall[b, rr, h][:, None])
                dq[b, rr, h, :] = scale * (dS @ kh)
                dk[b, :, kv, :] += scale * (dS.T @ q[b, rr, h, :])
                dv[b, :, kv, :] += P.T @ do[b, rr, h, :]
    return dq, dk, dv


def attn_bwd_multi(tiles, k, v, scale, head_map=None, causal=False, k_pos=None):
    """Backward over several Q partitions against one KV partition.

    tiles: list of dicts with keys q, o, do, lse and (when causal) q_pos.
    dK/dV are summed over the tiles ([Mesh] §3.5: partial gradients are
    accumulated locally, the reducer is addition).  Returns ([dq per tile], dk, dv).
    """
    dks, dvs, dqs = None, None, []
    for t in tiles:
        dq, dk, dv = attn_tile_bwd(t["q"], k, v, t["o"], t["do"], t["lse"], scale, head_map,
                                   causal, t.get("q_pos"), k_pos)
        dqs.append(dq)
        dks = dk if dks is None else dks + dk
        dvs = dv if dvs is None else dvs + dv
    return dqs, dks, dvs
