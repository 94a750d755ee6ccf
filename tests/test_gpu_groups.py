"""The tile groups and hot experts that moe_fused derives from a sorted layout (large-batch path),
read back from the workspace and compared with the rule written out on the host.

Rule: the tiles of an expert form a maximal run of equal expert ids (the sort writes them in
ascending expert order); a run of L tiles is cut into groups of gs = ceil(L / ceil(L / 8)) tiles
starting at its first tile (the last group shorter).  With fp8 / fp4 activations from 2048
tokens a run of at least ceil(T / 128) tiles is hot, hot indices follow the run order and only
the first MOE_HOT_MAX hot runs keep one; cgroups lists the groups of the runs without a hot
index.  Cases: uniform routing (no hot run), a skewed routing (a few hot runs), more hot
candidates than MOE_HOT_MAX, and a layout of more than 16384 tiles (the tile map read from
global memory instead of LDS)."""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from quantized_moe_expert_sort_amd import inputs as gen

pytestmark = pytest.mark.gpu
GT = 8


def host_rule(eids, n, hot_min):
    runs, t = [], 0
    while t < n:
        s = t
        while t < n and eids[t] == eids[s]:
            t += 1
        runs.append((s, t - s, int(eids[s])))
    groups, cgroups, hot_e, tile_hot = [], [], [], np.full(n, -1, dtype=np.int64)
    nhot = 0
    for rs, L, e in runs:
        gs = -(-L // -(-L // GT))
        hot = L >= hot_min
        h = nhot if hot and nhot < qm.HOT_MAX else -1
        nhot += hot
        if h >= 0:
            hot_e.append(e)
            tile_hot[rs:rs + L] = h
        for j in range(-(-L // gs)):
            g = (rs + j * gs, min(gs, L - j * gs))
            groups.append(g)
            if h < 0:
                cgroups.append(g)
    return groups, cgroups, hot_e, min(nhot, qm.HOT_MAX), tile_hot


def routing(kind, T, E, K, seed):
    rng = np.random.default_rng(seed)
    if kind == "uniform":
        return gen.make_routing(seed, T, E, K, 0.0)
    if kind == "skewed":
        return gen.make_routing(seed, T, E, K, 1.1)
    # many hot candidates: every token picks K distinct experts among the first 20
    ids = np.stack([rng.permutation(20)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    return ids, w / w.sum(1, keepdims=True)


CASES = [("uniform", 4096, 64, 8, "fp8"),
         ("skewed", 4096, 128, 16, "fp4"),
         ("many_hot", 2048, 32, 16, "fp8"),
         ("skewed", 36000, 256, 16, "fp4")]     # > 16384 tiles


@pytest.mark.parametrize("kind,T,E,K,a_dtype", CASES)
def test_groups_match_rule(kind, T, E, K, a_dtype):
    print(f"groups {kind} T={T} E={E} K={K} {a_dtype}", flush=True)
    D, I, bm = 512, 256, 32
    ids, w = routing(kind, T, E, K, seed=T + E)
    ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    lay = qm.moe_sort(ids_d, w_d, 0, E, bm)
    x = torch.from_numpy(gen.make_x(T, T, D).view(np.int16)).cuda()
    xa, xs = qm.moe_quant_act(x, a_dtype)
    wd = qm.device_weights(*gen.make_weights(E, E, D, I))
    act = qm.ACTS["situv2"]
    ws = torch.zeros(qm.fused_ws_bytes(T, D, I, lay.cap, bm, qm.DTYPES[a_dtype], act), dtype=torch.uint8,
                     device="cuda")
    qm.moe_fused(xa, xs, a_dtype, *wd, w_d, lay, E, "situv2", gen.BETA, gen.LINEAR_BETA, ws=ws, stages=qm.STAGE_1)
    torch.cuda.synchronize()
    n = int(lay.num_tiles.item())
    eids = lay.expert_ids.cpu().numpy()
    hot_min = -(-T // 128)
    groups, cgroups, hot_e, nh, tile_hot = host_rule(eids, n, hot_min)
    print(f"  tiles {n}, groups {len(groups)}, hot runs {nh}", flush=True)
    W = qm.fused_ws_parts(T, D, I, lay.cap, bm, qm.DTYPES[a_dtype], act)
    gb = (lay.cap * 8 + 255) // 256 * 256

    def i32(off, count):
        return ws[off:off + 4 * count].cpu().numpy().view(np.int32)

    assert i32(W["groups"] + gb, 1)[0] == len(groups)
    assert [tuple(g) for g in i32(W["groups"], 2 * len(groups)).reshape(-1, 2).tolist()] == groups
    assert i32(W["cgroups"] + gb, 1)[0] == len(cgroups)
    assert [tuple(g) for g in i32(W["cgroups"], 2 * len(cgroups)).reshape(-1, 2).tolist()] == cgroups
    he = i32(W["hot_e"], qm.HOT_MAX + 1)
    assert he[qm.HOT_MAX] == nh and he[:nh].tolist() == hot_e
    assert np.array_equal(i32(W["tile_hot"], n), tile_hot)
    if kind == "many_hot":
        assert nh == qm.HOT_MAX and len(cgroups) < len(groups)
    if kind == "uniform":
        assert nh == 0 and cgroups == groups
    if T > 30000:
        assert n > 16384
