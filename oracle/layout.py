"""Partition and position mapping, written brute force from the definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Deliberately naive: the
assignment matrix is materialised in full and every set is read off it; tile
classes come from enumerating every (query, key) pair.

Position descriptors here are lists of segments ``(local_begin, global_begin,
stride)``: local index t in [local_begin_s, local_begin_{s+1}) has global
position ``global_begin_s + (t - local_begin_s) * stride_s``.
"""
from __future__ import annotations

import numpy as np

EMPTY, PARTIAL, FULL = 0, 1, 2


# --- token positions -------------------------------------------------------

def expand_positions(segments, length):
    """Global position of every local token, by walking the segments one token at a time."""
    segs = sorted(segments, key=lambda s: s[0])
    assert segs[0][0] == 0
    out = np.empty(length, dtype=np.int64)
    for t in range(length):
        s = max(i for i, seg in enumerate(segs) if seg[0] <= t)
        lb, gb, st = segs[s]
        out[t] = gb + (t - lb) * st
    return out


def contiguous(global_begin):
    """A contiguous partition starting at ``global_begin``."""
    return [(0, int(global_begin), 1)]


def zigzag_chunks(N, r):
    """[Ring] "Causal masks and load balancing": with 2N chunks, rank r holds chunks r and 2N-1-r."""
    return (r, 2 * N - 1 - r)


def zigzag_rank_positions(N, r, chunk_len):
    """Token positions of rank r's zigzag share as one two-segment descriptor."""
    c0, c1 = zigzag_chunks(N, r)
    return [(0, c0 * chunk_len, 1), (chunk_len, c1 * chunk_len, 1)]


def striped(N, r):
    """[Ring] "Causal masks and load balancing": rank r takes tokens r, r+N, r+2N, ...;
    [Mesh] §3.7 uses the same interleaving across the logical mesh."""
    return [(0, int(r), int(N))]


# --- assignment matrix ([Mesh] §3.1-3.3) --------------------------------------

def assignment_matrix(n, a=None, b=None, scheme="kvr"):
    """A[i][j] = GPU that computes (Q_i, KV_j).

    ring : row i to GPU i ([Mesh] §3.1, Ring-Attention).
    basic: GPU g has tile row r=floor(g/a), column c=g mod a; Q partitions
           ra..(r+1)a-1, KV partitions cb..(c+1)b-1 ([Mesh] §3.2).
    kvr  : same tile rows; KV partitions {c + t a : 0 <= t < b} ([Mesh] §3.3).
    """
    A = -np.ones((n, n), dtype=np.int64)
    for g in range(n):
        if scheme == "ring":
            A[g, :] = g
            continue
        assert a * b == n
        r, c = g // a, g % a
        qs = range(r * a, (r + 1) * a)
        if scheme == "basic":
            ks = range(c * b, (c + 1) * b)
        elif scheme == "kvr":
            ks = [c + t * a for t in range(b)]
        else:
            raise ValueError(scheme)
        for i in qs:
            for j in ks:
                assert A[i, j] == -1
                A[i, j] = g
    assert (A >= 0).all()
    return A


def footprint(A, g):
    """I_g^Q, I_g^KV (partitions GPU g touches) and R_g^Q, R_g^KV (the remote ones); [Mesh] §3.1."""
    n = A.shape[0]
    IQ = sorted({i for i in range(n) for j in range(n) if A[i, j] == g})
    IKV = sorted({j for i in range(n) for j in range(n) if A[i, j] == g})
    return IQ, IKV, [i for i in IQ if i != g], [j for j in IKV if j != g]


def comm_units(A, g):
    """Units GPU g communicates, counted as [Mesh] §1 counts them for Figure 1.

    One unit per remote Q partition, two per remote KV partition (K and V), and
    one per partial output sent to another owner (one per remote Q partition).
    """
    _, _, RQ, RKV = footprint(A, g)
    return len(RQ) + 2 * len(RKV) + len(RQ)


def mesh_tile(n, a, b, g, kvr=True):
    """(Q partitions, KV partitions) that GPU g computes, KV in tile order."""
    r, c = g // a, g % a
    qs = list(range(r * a, (r + 1) * a))
    ks = [c + t * a for t in range(b)] if kvr else list(range(c * b, (c + 1) * b))
    A = assignment_matrix(n, a, b, "kvr" if kvr else "basic")
    assert all(A[i, j] == g for i in qs for j in ks)
    return qs, ks


def q_group(n, a, b, g):
    """[Mesh] §3.3 Q group of GPU g: the a GPUs of its tile row, {ra + x}."""
    r = g // a
    return [r * a + x for x in range(a)]


def kv_group(n, a, b, g):
    """[Mesh] §3.3 KV group of GPU g: the b GPUs of its tile column, {c + a x}."""
    c = g % a
    return [c + a * x for x in range(b)]


# --- masks and tile classes ------------------------------------------------------

def allowed_matrix(q_positions, k_positions):
    """allowed[t,u] = pos_k(u) <= pos_q(t), by explicit enumeration."""
    qp = np.asarray(q_positions, dtype=np.int64)
    kp = np.asarray(k_positions, dtype=np.int64)
    return kp[None, :] <= qp[:, None]


def classify(q_positions, k_positions, causal=True):
    """EMPTY (nothing allowed), FULL (everything allowed) or PARTIAL; [Mesh] §3.7 pair classes."""
    if not causal:
        return FULL
    al = allowed_matrix(q_positions, k_positions)
    if not al.any():
        return EMPTY
    if al.all():
        return FULL
    return PARTIAL


def allowed_count(q_positions, k_positions, causal=True):
    """Number of allowed (query, key) pairs (per head)."""
    if not causal:
        return len(q_positions) * len(k_positions)
    return int(allowed_matrix(q_positions, k_positions).sum())


def worklist(q_parts, k_parts, causal=True):
    """Non-EMPTY (qi, kj, class) triples for lists of per-partition position arrays."""
    out = []
    for i, qp in enumerate(q_parts):
        for j, kp in enumerate(k_parts):
            c = classify(qp, kp, causal)
            if c != EMPTY:
                out.append((i, j, c))
    return out
