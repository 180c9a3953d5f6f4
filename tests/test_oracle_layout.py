"""Pins for the oracle's partition/position mapper against values printed on the pages (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import layout

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_figure1_unit_counts():
    g = gold("mesh_n9_figure1.json")
    n, a, b = g["n"], g["a"], g["b"]
    ring = layout.assignment_matrix(n, scheme="ring")
    assert all(layout.comm_units(ring, x) == g["ring_units_per_gpu"] for x in range(n))
    assert sum(layout.comm_units(ring, x) for x in range(n)) == g["ring_total_units"]
    basic = layout.assignment_matrix(n, a, b, "basic")
    for x in range(n):
        _, _, RQ, RKV = layout.footprint(basic, x)
        qkv = len(RQ) + 2 * len(RKV)
        want = g["basic_diagonal_qkv_units"] if x in g["basic_diagonal_gpus"] else g["basic_offdiagonal_qkv_units"]
        assert qkv == want
        assert len(RQ) == g["basic_output_units_per_gpu"]
    assert sum(layout.comm_units(basic, x) for x in range(n)) == g["basic_total_units"]
    kvr = layout.assignment_matrix(n, a, b, "kvr")
    # KV partition order of the rotated matrix, read column by column of tile columns
    order = [j for c in range(a) for j in layout.mesh_tile(n, a, b, c, kvr=True)[1]]
    assert order == g["kvr_kv_order"]
    for x in range(n):
        _, _, RQ, RKV = layout.footprint(kvr, x)
        assert len(RQ) == g["kvr_remote_q_per_gpu"] and len(RKV) == g["kvr_remote_kv_per_gpu"]
    assert sum(layout.comm_units(kvr, x) for x in range(n)) == g["kvr_total_units"]


def test_gpu3_footprint():
    g = gold("mesh_n9_figure1.json")
    IQ, IKV, RQ, RKV = layout.footprint(layout.assignment_matrix(9, 3, 3, "basic"), 3)
    assert IQ == g["gpu3_IQ"] and IKV == g["gpu3_IKV"] and RQ == g["gpu3_RQ"] and RKV == g["gpu3_RKV"]
    assert len(RQ) + len(RKV) == g["gpu3_remote_footprint"]
    _, _, RQr, RKVr = layout.footprint(layout.assignment_matrix(9, scheme="ring"), 3)
    assert len(RQr) + len(RKVr) == g["ring_remote_footprint"]


def test_groups_a3_b5():
    g = gold("mesh_groups_a3_b5.json")
    n, a, b = g["n"], g["a"], g["b"]
    assert layout.q_group(n, a, b, 0) == g["gpu0_q_group"]
    assert layout.kv_group(n, a, b, 0) == g["gpu0_kv_group"]
    qs, ks = layout.mesh_tile(n, a, b, 0)
    assert qs == g["gpu0_q_partitions"] and ks == g["gpu0_kv_partitions"]
    assert layout.mesh_tile(n, a, b, 1)[1] == g["gpu1_kv_partitions"]
    assert layout.mesh_tile(n, a, b, 2)[1] == g["gpu2_kv_partitions"]
    # the three GPUs of the Q group cover all 15 KV partitions exactly once
    cover = sorted(j for x in g["gpu0_q_group"] for j in layout.mesh_tile(n, a, b, x)[1])
    assert cover == list(range(n))


@pytest.mark.parametrize("n", [4, 9, 16, 25, 36, 49, 64])
def test_footprint_bound_square_tiles(n):
    # [Mesh] section 3.2: max_g (|R^Q| + |R^KV|) <= 2 sqrt(n) - 1 for the basic tiling.
    a = b = int(math.isqrt(n))
    A = layout.assignment_matrix(n, a, b, "basic")
    worst = max(len(layout.footprint(A, g)[2]) + len(layout.footprint(A, g)[3]) for g in range(n))
    assert worst <= 2 * math.sqrt(n) - 1


@pytest.mark.parametrize("n,a,b", [(4, 2, 2), (9, 3, 3), (15, 3, 5), (16, 8, 2), (16, 4, 4), (64, 8, 8)])
def test_kvr_groups_are_consistent(n, a, b):
    A = layout.assignment_matrix(n, a, b, "kvr")
    for g in range(n):
        IQ, IKV, _, _ = layout.footprint(A, g)
        # gathered Q partitions are exactly the Q group, gathered KV partitions exactly the KV group
        assert IQ == layout.q_group(n, a, b, g)
        assert IKV == sorted(layout.kv_group(n, a, b, g))
        assert g in IQ and g in IKV


def test_contiguous_causal_imbalance():
    g = gold("causal_balance.json")
    N = g["contiguous_N"]
    units = [sum(layout.classify([r], [j], True) != layout.EMPTY for j in range(N)) for r in range(N)]
    assert sum(units) == g["contiguous_total_block_units"] and max(units) == g["contiguous_critical_path_units"]
    assert abs(sum(units) / (N * max(units)) - g["contiguous_utilisation"]) < 1e-12


@pytest.mark.parametrize("N", [2, 3, 8, 16])
def test_zigzag_balance(N):
    g = gold("causal_balance.json")
    c = 4  # tokens per chunk
    for r in range(N):
        c0, c1 = layout.zigzag_chunks(N, r)
        # block units: a chunk attends to itself and every earlier chunk
        units = (c0 + 1) + (c1 + 1)
        assert units == 2 * N + 1
        qp = layout.expand_positions(layout.zigzag_rank_positions(N, r, c), 2 * c)
        assert list(qp) == list(range(c0 * c, c0 * c + c)) + list(range(c1 * c, c1 * c + c))
    assert layout.zigzag_chunks(N, 0) == (0, 2 * N - 1)
    assert sorted(layout.zigzag_chunks(N, N - 1)) == [N - 1, N]
    assert g["zigzag_rank0_chunks_are_first_and_last"] and g["zigzag_last_rank_holds_two_middle_chunks"]


def test_striped_positions():
    N, r = 16, 5
    assert list(layout.expand_positions(layout.striped(N, r), 6)) == [r + N * t for t in range(6)]


def test_pair_classes_contiguous():
    g = gold("mesh_pair_classes.json")
    P = 6
    name = {layout.EMPTY: "EMPTY", layout.PARTIAL: "PARTIAL", layout.FULL: "FULL"}
    for i in range(4):
        for j in range(4):
            qp = np.arange(i * P, (i + 1) * P); kp = np.arange(j * P, (j + 1) * P)
            key = "i<j" if i < j else ("i=j" if i == j else "i>j")
            assert name[layout.classify(qp, kp)] == g["rule"][key]


def test_zigzag_share_worklist_128k_rank5():
    # Zigzag share of rank 5 of 16 at S = 131072 in 32 chunks of 4096: chunks {5, 26}; against all 32
    # KV chunks, 33 tiles are computed (31 dense + 2 diagonal) and 31 are skipped.
    N, r, C = 16, 5, 4096
    qchunks = layout.zigzag_chunks(N, r)
    assert qchunks == (5, 26)
    # classes from the partition ranges (enumeration on small stand-ins of the same order)
    q_parts = [np.arange(c * C, (c + 1) * C, 64) for c in qchunks]
    k_parts = [np.arange(j * C, (j + 1) * C, 64) for j in range(2 * N)]
    wl = layout.worklist(q_parts, k_parts)
    assert len(wl) == 33 and 64 - len(wl) == 31
    assert sum(c == layout.PARTIAL for _, _, c in wl) == 2
    # exact allowed-pair count per head with full token resolution on the two diagonal tiles
    full = 31 * C * C
    diag = sum(layout.allowed_count(np.arange(c * C, (c + 1) * C), np.arange(c * C, (c + 1) * C)) for c in qchunks)
    assert diag == 2 * (C * (C + 1) // 2)
    assert full + diag == 536_875_008
