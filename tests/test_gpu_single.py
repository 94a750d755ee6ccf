"""The single-launch path of moe_fused (a layout with sync words, batches below
SINGLE_LAUNCH_MAX_TOKENS; opt-in) against the default per-stage launches on the same inputs: the
same output bits, since both run the same Stage1 / Stage2 / combine arithmetic, and every token's
output row within the bar against the oracle.  Also: the sort zeroes the sync words, every call
leaves them zero (so a layout can be reused), and no wait timed out."""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from oracle import moe as om
from quantized_moe_expert_sort_amd import inputs as gen
from _parity import RequantExplainer, assert_rows_close

pytestmark = pytest.mark.gpu
BETA, LBETA = gen.BETA, gen.LINEAR_BETA


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def problem(T, Er, K, D, I, eb, E, a_dtype, zipf=0.0, seed=None):
    seed = T * 7 + D + I + eb if seed is None else seed
    ids, w = gen.make_routing(seed, T, Er, K, zipf)
    x = gen.make_x(seed, T, D)
    host_w = gen.make_weights(seed, E, D, I, experts=range(eb, eb + E))
    x_d = dev(x)
    if a_dtype == "bf16":
        xa, xs = x_d, None
    else:
        xa, xs = qm.moe_quant_act(x_d, a_dtype)
    return dict(ids=ids, w=w, x=x, host_w=host_w, ids_d=dev(ids), w_d=dev(w), xa=xa, xs=xs,
                wd=qm.device_weights(*host_w))


def fused(pb, lay, eb, E, a_dtype, act="situv2"):
    out = qm.moe_fused(pb["xa"], pb["xs"], a_dtype, *pb["wd"], pb["w_d"], lay, E, act, BETA, LBETA)
    torch.cuda.synchronize()
    return out


CASES = [  # (T, E_router, K, D, I, eb, E_local, bm, a_dtype, act)
    (1, 128, 16, 3584, 384, 0, 128, 16, "bf16", "situv2"),     # decode-sized rows
    (4, 64, 8, 512, 256, 0, 64, 16, "bf16", "situv2"),
    (37, 16, 4, 512, 256, 0, 16, 16, "fp8", "situv2"),
    (37, 16, 4, 512, 256, 0, 16, 32, "fp4", "situv2"),
    (100, 24, 6, 384, 384, 0, 24, 32, "bf16", "silu"),
    (61, 20, 3, 256, 128, 0, 20, 16, "fp4", "silu"),
    (50, 32, 4, 256, 256, 8, 8, 16, "fp8", "situv2"),            # expert-parallel: tokens w/o rows
    (300, 40, 5, 640, 256, 0, 40, 32, "bf16", "situv2"),
    (2047, 64, 8, 256, 128, 0, 64, 32, "fp8", "situv2"),        # largest single-launch batch
    # at most 32 routed rows: the per-stage path's fused Stage2 + combine kernel
    (8, 32, 4, 512, 256, 0, 32, 16, "fp8", "situv2"),            # exactly 32 rows
    (2, 32, 16, 256, 128, 0, 32, 32, "fp4", "silu"),
    (6, 32, 4, 256, 256, 8, 8, 16, "fp4", "situv2"),            # expert-parallel: tokens w/o rows
    # 33..64 routed rows at block_m 16 (per-tile Stage2 + combine)
    (4, 64, 16, 512, 256, 0, 64, 16, "bf16", "situv2"),          # exactly 64 rows
    (3, 40, 16, 256, 512, 0, 40, 16, "fp8", "situv2"),           # inter_dim 512
    (4, 32, 12, 256, 128, 8, 16, 16, "fp4", "silu"),             # expert-parallel: tokens w/o rows
]


@pytest.mark.parametrize("T,Er,K,D,I,eb,E,bm,a_dtype,act", CASES)
def test_single_launch_matches_per_stage_bits(T, Er, K, D, I, eb, E, bm, a_dtype, act):
    print(f"single T={T} E={E} D={D} I={I} bm={bm} {a_dtype} {act}", flush=True)
    pb = problem(T, Er, K, D, I, eb, E, a_dtype)
    lay_s = qm.moe_sort(pb["ids_d"], pb["w_d"], eb, E, bm, single_launch=True)
    lay_m = qm.moe_sort(pb["ids_d"], pb["w_d"], eb, E, bm, single_launch=False)
    assert lay_s.sync is not None and lay_m.sync is None
    out_s = fused(pb, lay_s, eb, E, a_dtype, act)
    out_m = fused(pb, lay_m, eb, E, a_dtype, act)
    assert int(lay_s.sync[0].item()) == 0, "a wait of the single-launch kernel timed out"
    assert torch.equal(out_s.view(torch.int16), out_m.view(torch.int16))
    # every counter was set back to zero by its last user
    assert int(torch.count_nonzero(lay_s.sync).item()) == 0
    # and the outputs are the operator's: every token's row against the oracle
    ids = pb["ids"]
    local = ((ids >= eb) & (ids < eb + E)).any(axis=1)
    got = out_s.float().cpu().numpy().astype(np.float64)
    ref, inter = om.moe_fused(pb["x"], a_dtype, *pb["host_w"], ids, pb["w"], eb, E, act, BETA, LBETA,
                              return_intermediate=True)
    tol = 5e-3 if a_dtype == "bf16" else 2e-2
    ex = None
    if a_dtype != "bf16":
        # the per-stage call's workspace holds its intermediate (the same bits as the single launch)
        ws = torch.empty(qm.fused_ws_bytes(T, D, I, lay_m.cap, bm, qm.DTYPES[a_dtype], qm.ACTS[act]),
                         dtype=torch.uint8, device="cuda")
        qm.moe_fused(pb["xa"], pb["xs"], a_dtype, *pb["wd"], pb["w_d"], lay_m, E, act, BETA, LBETA, ws=ws)
        torch.cuda.synchronize()
        parts = qm.fused_ws_parts(T, D, I, lay_m.cap, bm, qm.DTYPES[a_dtype], qm.ACTS[act])
        ex = RequantExplainer(got, ws.cpu().numpy(), lay_m.row_of.cpu().numpy(), inter, None, a_dtype, act, BETA,
                              LBETA, pb["host_w"][2], pb["host_w"][3], ids, pb["w"], eb, D, I, lay_m.cap * bm, tol,
                              parts["inter"], parts["iscale"])
    assert_rows_close(got, ref, local, tol, f"{a_dtype} {act}", explain=ex)


def test_single_launch_reuses_layout_without_sorting_again():
    T, Er, K, D, I, E, bm = 16, 256, 16, 1024, 384, 256, 16
    pb = problem(T, Er, K, D, I, 0, E, "bf16")
    lay = qm.moe_sort(pb["ids_d"], pb["w_d"], 0, E, bm, single_launch=True)
    first = fused(pb, lay, 0, E, "bf16")
    for _ in range(3):
        again = fused(pb, lay, 0, E, "bf16")
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
    assert int(torch.count_nonzero(lay.sync).item()) == 0


def test_sort_zeroes_sync_words():
    T, K, E, bm = 40, 4, 32, 16
    ids, w = gen.make_routing(5, T, E, K, 0.0)
    lay = qm.MoeLayout(T, K, E, bm, single_launch=True)
    lay.sync.fill_(7)
    qm.moe_sort(dev(ids), dev(w), 0, E, bm, layout=lay)
    torch.cuda.synchronize()
    assert lay.sync.numel() == qm.sync_words(T, lay.cap)
    assert int(torch.count_nonzero(lay.sync).item()) == 0


def test_single_launch_nothing_local():
    T, Er, K, D, I, eb, E, bm = 24, 64, 4, 256, 128, 60, 4, 16
    pb = problem(T, Er, K, D, I, eb, E, "fp8", seed=3)
    ids = np.full((T, K), 2, np.int32)                       # every id outside [60, 64)
    pb["ids_d"] = dev(ids)
    lay = qm.moe_sort(pb["ids_d"], pb["w_d"], eb, E, bm, single_launch=True)
    out = fused(pb, lay, eb, E, "fp8")
    assert int(lay.num_tiles.item()) == 0
    assert int(torch.count_nonzero(out.view(torch.int16)).item()) == 0
