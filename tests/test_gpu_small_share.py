"""Full-size parity of the small-tile share the bench times: a 13440 x 13440 non-causal share
(32/8 heads, d = 128, bf16) cut into P x P tiles at [CHARM+]'s partition sizes (its scaling
table: 13440 tokens over 1, 4, 16 and 64 partitions), all (13440 / P)^2 tiles in one forward call,
every output a slice of one long buffer, through mesh_attn_tile_fwd_tabled as in the bench.  Tiles
of 210 keys run the resident-KV kernel from the tile table (and, at 210, the same call through
mesh_attn_tile_fwd must give the same bits), 840 and 3360 the four-wave ring kernel, 13440 the
eight-wave one.  Sampled tiles (the
corners, the diagonal ends and seeded others) are checked on sampled rows, every query head,
against the fp64 oracle over all of the tile's keys."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import distributed_long_context_amd as ma  # noqa: E402
from distributed_long_context_amd import Tile  # noqa: E402
from oracle import attn_tile  # noqa: E402
from gpu_helpers import BF16_LSE_TOL, BF16_O_TOL, DEV, check_close, gen, host_f64, log  # noqa: E402
from test_gpu_workloads import sample_rows  # noqa: E402

import synthetic  # noqa: E402

HQ, HKV, D, S = 32, 8, 128, 13440
SCALE = np.float32(1.0 / math.sqrt(D))
WID = 3100


@pytest.fixture(scope="module")
def share():
    log("[small-tile share] inputs 13440 x 32/8 heads x 128")
    q, qv = gen(WID, synthetic.T_Q, 0, (1, S, HQ, D))
    k, kv = gen(WID, synthetic.T_K, 0, (1, S, HKV, D))
    v, vv = gen(WID, synthetic.T_V, 0, (1, S, HKV, D))
    return q, k, v, qv, kv, vv


@pytest.mark.parametrize("P,ntiles_checked", [(210, 24), (840, 10), (3360, 5), (13440, 1)])
def test_small_tile_share_full_size(share, P, ntiles_checked):
    q, k, v, qv, kv, vv = share
    n = S // P
    log(f"[small-tile share] P={P}: {n * n} tiles in one call")
    o_all = torch.full((n * n * P * HQ * D,), float("nan"), dtype=torch.bfloat16, device=DEV)
    l_all = torch.full((n * n * HQ * P,), float("nan"), dtype=torch.float32, device=DEV)
    tiles = []
    for i in range(n):
        for j in range(n):
            t = i * n + j
            tiles.append(Tile(q[:, i * P:(i + 1) * P], k[:, j * P:(j + 1) * P], v[:, j * P:(j + 1) * P],
                              o_all[t * P * HQ * D:(t + 1) * P * HQ * D].view(1, P, HQ, D),
                              l_all[t * HQ * P:(t + 1) * HQ * P].view(1, HQ, P)))
    ma.mesh_attn_tile_fwd(tiles, float(SCALE), ma.MA_MASK_NONE, table=True)  # the bench's path
    torch.cuda.synchronize()
    if P == 210:  # the same call with the tiles in kernel arguments: bitwise the same
        o2, l2 = torch.full_like(o_all, float("nan")), torch.full_like(l_all, float("nan"))
        tiles2 = [Tile(t.q, t.k, t.v, o2[i * P * HQ * D:(i + 1) * P * HQ * D].view(1, P, HQ, D),
                       l2[i * HQ * P:(i + 1) * HQ * P].view(1, HQ, P)) for i, t in enumerate(tiles)]
        ma.mesh_attn_tile_fwd(tiles2, float(SCALE), ma.MA_MASK_NONE)
        torch.cuda.synchronize()
        assert torch.equal(o_all, o2) and torch.equal(l_all, l2)
        del o2, l2, tiles2
    rng = np.random.default_rng([WID, P])
    fixed = [0, n - 1, n * (n - 1), n * n - 1, (n // 2) * n + n // 2]
    picks = list(dict.fromkeys(fixed))
    for x in rng.permutation(n * n):
        if len(picks) >= ntiles_checked:
            break
        if int(x) not in picks:
            picks.append(int(x))
    picks = picks[:ntiles_checked]
    for t in picks:
        i, j = divmod(t, n)
        rows = sample_rows(P, WID + t, extra=8 if P <= 840 else 4)
        O, L = attn_tile(qv[:, i * P:(i + 1) * P], kv[:, j * P:(j + 1) * P], vv[:, j * P:(j + 1) * P], SCALE,
                         rows=rows)
        got_o = host_f64(tiles[t].o[:, torch.from_numpy(rows).to(DEV)])
        got_l = host_f64(tiles[t].lse[:, :, torch.from_numpy(rows).to(DEV)])
        check_close(f"O tile ({i},{j})", got_o, O, BF16_O_TOL)
        check_close(f"LSE tile ({i},{j})", got_l, L, BF16_LSE_TOL)
    del o_all, l_all, tiles
    torch.cuda.empty_cache()
