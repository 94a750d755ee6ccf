"""moe_fused on the GPU vs the oracle.

* Small problems (several tiles per expert, ragged tails, every a_dtype, SiTUv2 and SiLU,
  an expert-parallel shard): every output element, relL2 <= 5e-3 for bf16 activations and
  <= 2e-2 for fp8 / fp4 (the oracle applies the same quantization), ||out|| > 0, and rows of
  tokens without a local expert exactly zero.
* Exact case: small-integer activations and e2m1 weights at scale 2^0 make every stage1 sum
  exact, so the raw gate/up sums written by the NONE_TEST hook must match bit for bit.
* Full workload sizes in the benchmark's launch configuration: sampled tokens recomputed one
  by one by the oracle, plus whole-output properties.
"""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from oracle import moe as om
from oracle import mx_formats as mx
from quantized_moe_expert_sort_amd import inputs as gen

pytestmark = pytest.mark.gpu
BETA, LBETA = gen.BETA, gen.LINEAR_BETA
TOL = {"bf16": 5e-3, "fp8": 2e-2, "fp4": 2e-2}


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def run_gpu(x, ids, w, weights_d, eb, E, bm, a_dtype, act="situv2", beta=BETA, lb=LBETA):
    ids_d, w_d = dev(ids), dev(w)
    lay = qm.moe_sort(ids_d, w_d, eb, E, bm)
    x_d = dev(x)
    if a_dtype == "bf16":
        xa, xs = x_d, None
    else:
        xa, xs = qm.moe_quant_act(x_d, a_dtype)
    res = qm.moe_fused(xa, xs, a_dtype, *weights_d, w_d, lay, E, act, beta, lb)
    torch.cuda.synchronize()
    return res, lay


SMALL = [  # (T, E_router, K, D, I, eb, E_local, bm, a_dtype, act, zipf)
    (4, 8, 2, 256, 128, 0, 8, 16, "bf16", "situv2", 0.0),       # the tiny workload's shape
    (1, 64, 8, 512, 256, 0, 64, 16, "bf16", "situv2", 0.0),
    (37, 16, 4, 512, 256, 0, 16, 16, "bf16", "situv2", 0.0),
    (37, 16, 4, 512, 256, 0, 16, 16, "fp8", "situv2", 0.0),
    (37, 16, 4, 512, 256, 0, 16, 16, "fp4", "situv2", 0.0),
    (100, 24, 6, 384, 384, 0, 24, 32, "bf16", "situv2", 1.1),
    (100, 24, 6, 384, 384, 0, 24, 32, "fp8", "situv2", 1.1),
    (100, 24, 6, 384, 384, 0, 24, 32, "fp4", "situv2", 1.1),
    (61, 20, 3, 256, 128, 0, 20, 16, "bf16", "silu", 0.0),
    (61, 20, 3, 256, 128, 0, 20, 32, "fp8", "silu", 0.0),
    (50, 32, 4, 256, 256, 8, 8, 16, "fp8", "situv2", 0.0),       # expert-parallel shard
    (50, 32, 4, 256, 256, 8, 8, 32, "bf16", "situv2", 0.0),
    # at most 32 routed rows (Stage2 and the combine in one kernel), every a_dtype and block_m
    (2, 64, 16, 512, 256, 0, 64, 16, "fp8", "situv2", 0.0),
    (2, 64, 16, 512, 256, 0, 64, 32, "fp4", "situv2", 0.0),
    (4, 40, 8, 256, 384, 0, 40, 32, "bf16", "silu", 0.0),
    (8, 32, 4, 256, 256, 8, 8, 16, "fp8", "situv2", 0.0),        # expert-parallel shard
    # >= 2048 tokens with model_dim % 512 == 0: the tiled large-batch
    # stages (Stage1 scale chunks span 4 K steps: 7 chunks at 3584, 2 at 1024, 1 at 512)
    (2048, 16, 4, 512, 256, 0, 16, 32, "fp8", "situv2", 1.1),
    (2048, 16, 4, 512, 256, 0, 16, 32, "fp4", "situv2", 1.1),
    (2048, 24, 4, 1024, 512, 0, 24, 32, "fp8", "silu", 0.5),      # four Stage1 column blocks
    (2500, 40, 6, 1024, 128, 0, 40, 32, "fp4", "silu", 0.0),
    (3000, 64, 8, 1024, 384, 16, 24, 32, "fp8", "situv2", 0.0),
    # bf16 activations from 2048 tokens: grouped Stage1 (128-row groups), per-tile Stage2
    (2048, 16, 4, 512, 256, 0, 16, 32, "bf16", "situv2", 1.1),
    (2500, 40, 6, 1024, 128, 0, 40, 32, "bf16", "silu", 0.0),
    (3000, 64, 8, 1024, 384, 16, 24, 32, "bf16", "situv2", 0.0),
    (2048, 64, 5, 512, 256, 0, 64, 32, "bf16", "situv2", 0.0),    # ~5-tile groups: parts of 3 + 2 tiles
    # the same batch sizes with model_dim % 512 != 0 take the per-tile stages
    (2500, 40, 6, 256, 128, 0, 40, 32, "fp4", "silu", 0.0),
    (3000, 64, 8, 768, 384, 16, 24, 32, "fp8", "situv2", 0.0),
]


@pytest.mark.parametrize("T,Er,K,D,I,eb,E,bm,a_dtype,act,zipf", SMALL)
def test_fused_small_full_output(T, Er, K, D, I, eb, E, bm, a_dtype, act, zipf):
    seed = T * 31 + D + I
    ids, w = gen.make_routing(seed, T, Er, K, zipf)
    x = gen.make_x(seed, T, D)
    w1, w1s, w2, w2s = gen.make_weights(seed, E, D, I, experts=range(eb, eb + E))
    wd = qm.device_weights(w1, w1s, w2, w2s)
    print(f"fused small T={T} E={E} D={D} I={I} bm={bm} {a_dtype} {act}", flush=True)
    out, _ = run_gpu(x, ids, w, wd, eb, E, bm, a_dtype, act)
    got = out.float().cpu().numpy().astype(np.float64)
    ref = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, eb, E, act, BETA, LBETA)
    local = ((ids >= eb) & (ids < eb + E)).any(axis=1)
    assert np.all(got[~local] == 0)
    assert np.linalg.norm(got) > 0
    err = om.rel_l2(got, ref)
    print(f"  relL2 {err:.3e}", flush=True)
    assert err <= TOL[a_dtype]


@pytest.mark.parametrize("a_dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("bm", [16, 32])
def test_stage1_exact_integer_sums(a_dtype, bm):
    rng = np.random.default_rng(17)
    T, E, K, D, I = 40, 6, 3, 256, 128
    xi = rng.integers(-4, 5, size=(T, D)).astype(np.float32)
    x = torch.from_numpy(xi).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w1 = mx.pack_fp4(rng.integers(0, 16, size=(E, 2 * I, D)))
    w2 = mx.pack_fp4(rng.integers(0, 16, size=(E, D, I)))
    w1s = np.full((E, 2 * I, D // 32), 127, np.uint8)
    w2s = np.full((E, D, I // 32), 127, np.uint8)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = np.ones((T, K), np.float32)
    wd = qm.device_weights(w1, w1s, w2, w2s)
    ws, lay = run_gpu(x, ids, w, wd, 0, E, bm, a_dtype, act="none_test")
    off = qm.fused_debug_offset(T, D, I, lay.cap, bm, qm.DTYPES[a_dtype])
    rows = lay.cap * bm
    dbg = ws[off:off + rows * 2 * I * 4].view(torch.float32).reshape(rows, 2 * I).cpu().numpy()
    sid = lay.sorted_token_ids.cpu().numpy()
    _, inter = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, E, "situv2", BETA, LBETA,
                            return_intermediate=True)
    checked = 0
    for e, (vs, g, u, _) in inter.items():
        for r, v in enumerate(vs):
            R = int(np.nonzero(sid == v)[0][0])
            assert np.array_equal(dbg[R, :I], g[r].astype(np.float32)), (e, v)
            assert np.array_equal(dbg[R, I:], u[r].astype(np.float32)), (e, v)
            checked += 1
    assert checked == T * K


# ------------------------------------------------------------------ full workload sizes

_WEIGHTS = {}


def weights_for(wl):
    key = (wl.seed, wl.experts, wl.model_dim, wl.inter_dim)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        host = gen.make_weights(wl.seed, wl.experts, wl.model_dim, wl.inter_dim)
        _WEIGHTS[key] = (host, qm.device_weights(*host))
    return _WEIGHTS[key]


FULL = ["dec-1", "dec-4", "dec-16", "mid-64", "mid-256", "mid-1024", "pre-16384", "ep-8192", "pre-a16-8192",
        "pre-a8-8192"]


@pytest.mark.parametrize("name", FULL)
def test_fused_full_size_sampled_tokens(name):
    wl = gen.WORKLOADS[name]
    print(f"full {name}: generating inputs", flush=True)
    host, wd = weights_for(wl)
    p = gen.make_problem(wl, with_weights=False)
    print(f"full {name}: T={wl.tokens} E={wl.experts} I={wl.inter_dim} {wl.a_dtype} bm={wl.block_m}", flush=True)
    out, lay = run_gpu(p["x"], p["topk_ids"], p["topk_w"], wd, 0, wl.experts, wl.block_m, wl.a_dtype)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    ids = p["topk_ids"]
    local = ((ids >= 0) & (ids < wl.experts)).any(axis=1)
    assert np.all(got[~local] == 0)
    assert np.all(np.abs(got[local]).sum(axis=1) > 0)
    rng = np.random.default_rng(1)
    cand = np.nonzero(local)[0]
    toks = sorted({int(cand[0]), int(cand[-1])} | set(int(t) for t in rng.choice(cand, size=min(2, len(cand)), replace=False)))
    ref = om.moe_tokens(toks, p["x"], wl.a_dtype, *host, ids, p["topk_w"], 0, wl.experts, "situv2", BETA, LBETA)
    err = om.rel_l2(got[toks], ref)
    print(f"  tokens {toks} relL2 {err:.3e}", flush=True)
    assert err <= TOL[wl.a_dtype]
