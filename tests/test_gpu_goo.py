"""Single-GPU replay of a GOO schedule's compute tasks ([Mesh] section 3.4).

A Q group of four partitions and a KV group of four partitions are cut into k_Q and
k_KV chunks; the gathered chunk i of Q (chunk i of every Q partition, concatenated) is
a tile with a four-segment position map, like tokens 48-51, 60-63, 72-75, 84-87 of
the pages' Figure 4.  The compute tasks C-i-j run in the order of the greedy plan,
each folded into its Q chunk's (O, LSE) with the forward's accumulate mode; at the
end every Q chunk must equal the oracle's attention of those rows over all KV tokens.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import Pos, Tile  # noqa: E402
from oracle import attn_tile  # noqa: E402
from gpu_helpers import BF16_LSE_TOL, BF16_O_TOL, DEV, check_close, gen, host_f64, log  # noqa: E402

import synthetic  # noqa: E402


@pytest.mark.parametrize("kq,kkv,causal", [(3, 3, False), (3, 3, True), (2, 8, True), (4, 4, False)])
def test_goo_replay_equals_unsplit(kq, kkv, causal):
    P, hq, hkv, d, G = 384, 8, 2, 128, 4
    wid = 1400 + 10 * kq + kkv
    log(f"[goo replay] kq={kq} kkv={kkv} causal={causal}")
    cq, ck = P // kq, P // kkv
    q_base = [4 * P + r * P for r in range(G)]      # Q group: four consecutive partitions
    k_base = [r * 4 * P for r in range(G)]          # KV group: every fourth partition
    Qp = [gen(wid, synthetic.T_Q, r, (1, P, hq, d)) for r in range(G)]
    Kp = [gen(wid, synthetic.T_K, r, (1, P, hkv, d)) for r in range(G)]
    Vp = [gen(wid, synthetic.T_V, r, (1, P, hkv, d)) for r in range(G)]
    mode = ma.MA_MASK_STRIPED_ZIGZAG if causal else ma.MA_MASK_NONE
    scale = float(np.float32(1.0 / math.sqrt(d)))
    steps = ma.mesh_attn_goo_plan(kq, kkv, 0.5, 1.0, 0.5, 0.5, 1.0)
    gq, gk, gv, out = {}, {}, {}, {}
    for comm, comp in steps:
        if comm is not None and comm[0] == "AG-Q":       # gathered Q chunk i arrives
            i = comm[1]
            gq[i] = torch.cat([x[0][:, i * cq:(i + 1) * cq] for x in Qp], dim=1)
            out[i] = (torch.zeros((1, G * cq, hq, d), dtype=torch.bfloat16, device=DEV),
                      torch.full((1, hq, G * cq), float("-inf"), dtype=torch.float32, device=DEV))
        elif comm is not None and comm[0] == "AG-KV":    # gathered KV chunk j arrives
            j = comm[1]
            gk[j] = torch.cat([x[0][:, j * ck:(j + 1) * ck] for x in Kp], dim=1)
            gv[j] = torch.cat([x[0][:, j * ck:(j + 1) * ck] for x in Vp], dim=1)
        for _, i, j in comp:
            qpos = Pos([(r * cq, q_base[r] + i * cq, 1) for r in range(G)])
            kpos = Pos([(r * ck, k_base[r] + j * ck, 1) for r in range(G)])
            ma.mesh_attn_tile_fwd([Tile(gq[i], gk[j], gv[j], out[i][0], out[i][1], qpos, kpos)], scale, mode,
                                  accumulate=True)
    torch.cuda.synchronize()
    assert sorted(out) == list(range(kq))
    kall = np.concatenate([x[1] for x in Kp], axis=1)
    vall = np.concatenate([x[1] for x in Vp], axis=1)
    kpos_all = np.concatenate([np.arange(b, b + P) for b in k_base])
    for i in range(kq):
        qv = np.concatenate([x[1][:, i * cq:(i + 1) * cq] for x in Qp], axis=1)
        qpos_i = np.concatenate([np.arange(b + i * cq, b + (i + 1) * cq) for b in q_base])
        Oref, Lref = attn_tile(qv, kall, vall, np.float32(scale), None, causal,
                               qpos_i if causal else None, kpos_all if causal else None)
        check_close(f"O chunk {i}", host_f64(out[i][0]), Oref, BF16_O_TOL, normalised_also=False)
        check_close(f"LSE chunk {i}", host_f64(out[i][1]), Lref, BF16_LSE_TOL)
