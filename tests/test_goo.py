"""GOO step planner ([Mesh] section 3.4): the oracle against the pages' worked example and the
rules every schedule must keep, and the C++ planner behind the C ABI against the oracle (CPU only)."""
import json
import os
import random

import pytest

from oracle import goo, layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "goo_figure4.json")


def _figure4():
    g = json.load(open(GOLDEN))
    c = g["cost"]
    return g, goo.plan(g["k_q"], g["k_kv"], c["AG-Q"], c["AG-KV"], c["RS-Q"], c["C"], g["gamma"])


def test_worked_example_of_figure4():
    g, steps = _figure4()
    comm = [list(c) if c else None for c, _ in steps]
    assert comm[:6] == [list(x) for x in g["comm_steps_1_to_6"]]
    assert [list(t[1:]) for t in steps[2][1]] == g["step3_compute"]
    assert [list(t[1:]) for t in steps[5][1]] == g["step6_compute"]
    assert [s + 1 for s, (c, _) in enumerate(steps) if c is None] == g["compute_only_steps"]
    assert sum(c is not None for c, _ in steps) == 2 * g["k_q"] + g["k_kv"]


def test_gathered_chunk_positions_of_figure4():
    # GPU 4's Q group holds tokens 48..95 in four partitions of 12; with k_Q = 3 the first gathered
    # chunk is tokens 48-51, 60-63, 72-75, 84-87: four segments of four tokens
    g = json.load(open(GOLDEN))
    segs = [(4 * s, 48 + 12 * s, 1) for s in range(4)]
    pos = layout.expand_positions(segs, 16)
    want = [t for a, b in g["gathered_q_chunk0_tokens"] for t in range(a, b + 1)]
    assert list(pos) == want


def check_schedule(steps, kq, kkv, t_agq, t_agkv, t_rsq, tc, gamma):
    """The rules of the step semantics, checked on any schedule."""
    t_comm = {"AG-Q": t_agq, "AG-KV": t_agkv, "RS-Q": t_rsq}
    done = set()
    seen_c = []
    for comm, comp in steps:
        # every compute task of a step was ready when the step began
        for _, i, j in comp:
            assert ("AG-Q", i) in done and ("AG-KV", j) in done
        if comm is None:
            assert len(comp) == 1
        else:
            assert comm not in done
            if comm[0] == "RS-Q":
                assert all(("C", comm[1], j) in done for j in range(kkv))
            # the compute added stays within the target except for the last task
            tot = [tc(i, j) for _, i, j in comp]
            assert sum(tot[:-1]) < gamma * t_comm[comm[0]] or not tot
            done.add(comm)
        for t in comp:
            assert t not in seen_c
            seen_c.append(t)
            done.add(t)
    assert sorted(seen_c) == sorted(("C", i, j) for i in range(kq) for j in range(kkv))
    for kind, n in (("AG-Q", kq), ("AG-KV", kkv), ("RS-Q", kq)):
        assert all((kind, x) in done for x in range(n))
    assert sum(c is not None for c, _ in steps) == 2 * kq + kkv


def _random_cases(n=60):
    rng = random.Random(5)
    out = []
    for _ in range(n):
        kq = rng.randint(1, 4)
        kkv = rng.randint(1, 16 // kq)
        costs = [rng.choice([0.25, 0.5, 1.0, 1.5, 2.0]) for _ in range(3)]
        tcm = [[rng.choice([0.0625, 0.25, 0.5, 0.75]) for _ in range(kkv)] for _ in range(kq)]
        gamma = rng.choice([0.5, 1.0, 1.5, 2.0])
        out.append((kq, kkv, *costs, tcm, gamma))
    return out


@pytest.mark.parametrize("case", _random_cases())
def test_oracle_schedules_keep_the_rules(case):
    kq, kkv, a, b, c, tcm, gamma = case
    steps = goo.plan(kq, kkv, a, b, c, tcm, gamma)
    check_schedule(steps, kq, kkv, a, b, c, lambda i, j: tcm[i][j], gamma)


def test_oracle_rules_catch_a_broken_schedule():
    g, steps = _figure4()
    bad = list(steps)
    bad[2] = (bad[2][0], [("C", 2, 2)])  # C-2-2 is not ready at step 3
    with pytest.raises(AssertionError):
        check_schedule(bad, 3, 3, 0.5, 1.0, 0.5, lambda i, j: 0.5, 1.0)


@pytest.mark.parametrize("case", _random_cases(40) + [(3, 3, 0.5, 1.0, 0.5, [[0.5] * 3] * 3, 1.0)])
def test_library_planner_matches_oracle(case):
    import distributed_long_context_amd as ma
    kq, kkv, a, b, c, tcm, gamma = case
    want = goo.plan(kq, kkv, a, b, c, tcm, gamma)
    got = ma.mesh_attn_goo_plan(kq, kkv, a, b, c, tcm, gamma)
    assert got == want


def test_library_planner_rejects_bad_arguments():
    import distributed_long_context_amd as ma
    for args in [(0, 1), (5, 4), (1, 17)]:
        with pytest.raises(ma.MeshAttnError):
            ma.mesh_attn_goo_plan(args[0], args[1], 1.0, 1.0, 1.0, 1.0, 1.0)
    with pytest.raises(ma.MeshAttnError):
        ma.mesh_attn_goo_plan(2, 2, 0.0, 1.0, 1.0, 1.0, 1.0)  # a communication time must be > 0


def test_library_planner_fills_its_step_array_exactly():
    # k_Q = k_KV = 1: AG-KV-0, AG-Q-0, a compute-only step, RS-Q-0 -- as many steps as the bound
    # 2 k_Q + k_KV + k_Q k_KV, so the planner must not touch the array past them
    import distributed_long_context_amd as ma
    import ctypes as C
    from distributed_long_context_amd import _abi
    steps = (_abi.ma_goo_step * 5)()
    for s in steps:
        s.comm_type = 77
    tc = (C.c_double * 1)(0.5)
    r = ma.lib().mesh_attn_goo_plan(1, 1, 0.5, 1.0, 0.5, tc, 1.0, 4, steps)
    assert r == 4
    assert steps[4].comm_type == 77  # the slot after the last step is untouched
    assert [s.comm_type for s in steps[:4]] == [2, 1, 0, 3]
