"""moe_fused on the GPU vs the oracle.

* Small problems (several tiles per expert, ragged tails, every a_dtype, SiTUv2 and SiLU,
  an expert-parallel shard): every output row of a token with a local expert within the bar
  (relL2 <= 5e-3 for bf16 activations, <= 2e-2 for fp8 / fp4, the oracle applying the same
  quantization) and nonzero, the whole output within the bar, and rows of tokens without a
  local expert exactly zero.
* Exact case: small-integer activations and e2m1 weights at scale 2^0 make every stage1 sum
  exact, so the raw gate/up sums written by the NONE_TEST hook must match bit for bit.
* Tile-geometry invariance (github ROCm/aiter PR 5118 "Accuracy": a change of N-tile that
  keeps the K-reduction order gives bitwise identical results): the per-tile path at block_m
  16 and 32 (different column blocks per workgroup, the same K split) gives the same bits, and
  changing the weight rows of other output columns leaves a column block's results unchanged.
* Full workload sizes in the benchmark's launch configuration: the tokens of the first routed
  row of every other tile of every expert (so every touched expert and every tile group of the
  large-batch path), each token's row checked against the oracle, plus whole-output properties.
"""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from oracle import moe as om
from oracle import mx_formats as mx
from quantized_moe_expert_sort_amd import inputs as gen
from _parity import RequantExplainer, assert_rows_close, coverage_tokens, oracle_tokens

pytestmark = pytest.mark.gpu
BETA, LBETA = gen.BETA, gen.LINEAR_BETA
TOL = {"bf16": 5e-3, "fp8": 2e-2, "fp4": 2e-2}


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def run_gpu(x, ids, w, weights_d, eb, E, bm, a_dtype, act="situv2", beta=BETA, lb=LBETA, keep_ws=False):
    ids_d, w_d = dev(ids), dev(w)
    lay = qm.moe_sort(ids_d, w_d, eb, E, bm)
    x_d = dev(x)
    if a_dtype == "bf16":
        xa, xs = x_d, None
    else:
        xa, xs = qm.moe_quant_act(x_d, a_dtype)
    T, D, I = x.shape[0], weights_d[2].shape[1], weights_d[2].shape[2] * 2
    ws = torch.empty(qm.fused_ws_bytes(T, D, I, lay.cap, bm, qm.DTYPES[a_dtype], qm.ACTS[act]), dtype=torch.uint8,
                     device="cuda")
    res = qm.moe_fused(xa, xs, a_dtype, *weights_d, w_d, lay, E, act, beta, lb, ws=ws)
    torch.cuda.synchronize()
    if keep_ws:
        return res, lay, ws
    return res, lay


def explainer(got, ws, lay, inter, tokens, a_dtype, act, host_w, ids, w, eb, D, I):
    """Near-tie requantization explainer of fp8 / fp4 rows (None for bf16)."""
    if a_dtype == "bf16":
        return None
    T = np.asarray(ids).shape[0]
    parts = qm.fused_ws_parts(T, D, I, lay.cap, lay.block_m, qm.DTYPES[a_dtype], qm.ACTS[act])
    return RequantExplainer(got, ws.cpu().numpy(), lay.row_of.cpu().numpy(), inter, tokens, a_dtype, act, BETA, LBETA,
                            host_w[2], host_w[3], ids, w, eb, D, I, lay.cap * lay.block_m, TOL[a_dtype],
                            parts["inter"], parts["iscale"])


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
    # 33..64 routed rows (per-tile Stage2 + combine); inter_dim 128 and 512
    (4, 64, 16, 512, 256, 0, 64, 16, "bf16", "situv2", 0.0),
    (3, 48, 16, 512, 384, 0, 48, 16, "fp8", "situv2", 0.0),
    (5, 40, 12, 256, 128, 0, 40, 16, "fp4", "silu", 0.0),
    (4, 32, 16, 256, 512, 8, 16, 16, "bf16", "situv2", 0.0),     # expert-parallel shard
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
    # ~1000 skewed items: several per workgroup, so the next-item prefetch and (fp8 / fp4) the
    # per-XCD work claims run, next to hot experts and the resident-row Stage2
    (4096, 512, 8, 512, 256, 0, 512, 32, "fp8", "situv2", 0.7),
    (4096, 512, 8, 512, 256, 0, 512, 32, "fp4", "silu", 0.7),
    (4096, 512, 8, 512, 256, 0, 512, 32, "bf16", "situv2", 0.7),
    # experts with at least a quarter of the tokens' rows: token-major Stage2 for up to 16 of them
    (2048, 24, 16, 512, 256, 0, 24, 32, "fp4", "silu", 0.3),      # all 24 qualify: 16 token-major
    (2100, 24, 16, 512, 256, 0, 24, 32, "fp8", "situv2", 0.0),    # partial last 128-token tile
    (2600, 32, 16, 512, 256, 4, 16, 32, "fp4", "situv2", 0.0),    # expert-parallel shard, all local hot
    # the same batch sizes with model_dim % 512 != 0 take the per-tile stages
    (2500, 40, 6, 256, 128, 0, 40, 32, "fp4", "silu", 0.0),
    (3000, 64, 8, 768, 384, 16, 24, 32, "fp8", "situv2", 0.0),
    # the smallest shape (one K step each way, a Stage2 column block wider than model_dim) at
    # the decode kernel's limit and one row past it, and top-1 routing
    (3, 40, 11, 128, 128, 0, 40, 16, "fp8", "situv2", 0.0),      # 33 routed rows: per-tile Stage2
    (1, 8, 8, 128, 128, 0, 8, 32, "fp4", "silu", 0.0),           # one token, 32-row tiles
    (32, 16, 1, 128, 256, 0, 16, 16, "bf16", "situv2", 0.0),     # top-1: exactly 32 routed rows
]


@pytest.mark.parametrize("T,Er,K,D,I,eb,E,bm,a_dtype,act,zipf", SMALL)
def test_fused_small_full_output(T, Er, K, D, I, eb, E, bm, a_dtype, act, zipf):
    seed = T * 31 + D + I
    ids, w = gen.make_routing(seed, T, Er, K, zipf)
    x = gen.make_x(seed, T, D)
    w1, w1s, w2, w2s = gen.make_weights(seed, E, D, I, experts=range(eb, eb + E))
    wd = qm.device_weights(w1, w1s, w2, w2s)
    print(f"fused small T={T} E={E} D={D} I={I} bm={bm} {a_dtype} {act}", flush=True)
    out, lay, ws = run_gpu(x, ids, w, wd, eb, E, bm, a_dtype, act, keep_ws=True)
    got = out.float().cpu().numpy().astype(np.float64)
    ref, inter = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, eb, E, act, BETA, LBETA, return_intermediate=True)
    local = ((ids >= eb) & (ids < eb + E)).any(axis=1)
    ex = explainer(got, ws, lay, inter, None, a_dtype, act, (w1, w1s, w2, w2s), ids, w, eb, D, I)
    assert_rows_close(got, ref, local, TOL[a_dtype], f"{a_dtype} {act}", explain=ex)


@pytest.mark.parametrize("T,a_dtype", [(2048, "fp4"), (2100, "fp8"), (2048, "bf16"), (300, "fp8")])
def test_fused_repeated_expert_ids(T, a_dtype):
    # a token that names one expert twice: two identical intermediate rows, both weighted into
    # its sum (with fp8 / fp4 at 2048+ tokens every expert here is hot: the token-major Stage2
    # adds the two router weights)
    E, K, D, I = 24, 16, 512, 256
    seed = 4242 + T
    ids, w = gen.make_routing(seed, T, E, K, 0.3)
    ids = ids.copy()
    rep = np.arange(T) % 3 == 0
    ids[rep, 1] = ids[rep, 0]
    ids[np.arange(T) % 5 == 0, K - 1] = ids[np.arange(T) % 5 == 0, 2]
    x = gen.make_x(seed, T, D)
    w1, w1s, w2, w2s = gen.make_weights(seed, E, D, I)
    wd = qm.device_weights(w1, w1s, w2, w2s)
    print(f"repeated ids T={T} {a_dtype}", flush=True)
    out, lay, ws = run_gpu(x, ids, w, wd, 0, E, 32, a_dtype, "situv2", keep_ws=True)
    got = out.float().cpu().numpy().astype(np.float64)
    ref, inter = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, E, "situv2", BETA, LBETA,
                              return_intermediate=True)
    local = np.ones(T, bool)
    ex = explainer(got, ws, lay, inter, None, a_dtype, "situv2", (w1, w1s, w2, w2s), ids, w, 0, D, I)
    assert_rows_close(got, ref, local, TOL[a_dtype], f"repeated ids {a_dtype}", explain=ex)


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


# ------------------------------------------------------------------ tile-geometry invariance

def _problem(T, Er, K, D, I, seed, E=None, zipf=0.0):
    E = Er if E is None else E
    ids, w = gen.make_routing(seed, T, Er, K, zipf)
    x = gen.make_x(seed, T, D)
    return x, ids, w, gen.make_weights(seed, E, D, I)


@pytest.mark.parametrize("a_dtype", ["bf16", "fp8", "fp4"])
def test_block_m_16_and_32_give_the_same_bits(a_dtype):
    # per-tile path (T < 2048): the column blocks per workgroup differ between the two tile
    # heights, the K split of Stage1 (4 waves, reduced in wave order) and the Stage2 K order do
    # not, so every sum is formed in the same order and the outputs agree bit for bit
    T, E, K, D, I = 150, 24, 6, 512, 256
    x, ids, w, host = _problem(T, E, K, D, I, seed=21, zipf=0.8)
    wd = qm.device_weights(*host)
    print(f"block_m invariance {a_dtype} T={T}", flush=True)
    o16, _ = run_gpu(x, ids, w, wd, 0, E, 16, a_dtype)
    o32, _ = run_gpu(x, ids, w, wd, 0, E, 32, a_dtype)
    assert torch.equal(o16.view(torch.int16), o32.view(torch.int16))
    ref = om.moe_fused(x, a_dtype, *host, ids, w, 0, E, "situv2", BETA, LBETA)
    assert_rows_close(o16.float().cpu().numpy(), ref, np.ones(T, bool), TOL[a_dtype], a_dtype)


@pytest.mark.parametrize("T,a_dtype", [(60, "fp8"), (60, "bf16"), (2048, "fp4"), (2048, "bf16"), (2048, "fp8")])
def test_column_block_results_ignore_other_columns_weights(T, a_dtype):
    # per-tile path (T = 60) and large-batch path (T = 2048).
    # Stage1: with the w2 codes of intermediate columns [128, I) zero (they add exact zeros to
    # every Stage2 sum), replacing the w1 gate and up rows of those columns leaves every output
    # bit identical: intermediate columns [0, 128) depend on their own w1 rows only.
    # Stage2: replacing the w2 rows of output columns [256, D) leaves columns [0, 256) unchanged.
    E, K, D, I = 16, 4, 512, 256
    x, ids, w, (w1, w1s, w2, w2s) = _problem(T, E, K, D, I, seed=23)
    rng = np.random.default_rng(5)
    w1b = w1.copy()
    for half in (0, I):
        w1b[:, half + 128:half + I] = rng.integers(0, 256, size=w1b[:, half + 128:half + I].shape, dtype=np.uint8)
    w2z = w2.copy()
    w2z[:, :, 64:] = 0                                    # K columns [128, I) of every w2 row
    w2b = w2.copy()
    w2b[:, 256:] = rng.integers(0, 256, size=w2b[:, 256:].shape, dtype=np.uint8)
    bm = gen.Workload("t", T, E, K, D, I, a_dtype).block_m
    print(f"column invariance {a_dtype} T={T} bm={bm}", flush=True)
    run = lambda a1, a2: run_gpu(x, ids, w, qm.device_weights(a1, w1s, a2, w2s), 0, E, bm, a_dtype)[0]
    oz, ozb = run(w1, w2z), run(w1b, w2z)
    assert torch.equal(oz.view(torch.int16), ozb.view(torch.int16))
    oa, ob = run(w1, w2), run(w1b, w2)
    assert not torch.equal(oa.view(torch.int16), ob.view(torch.int16))   # the changed rows are used
    oc = run(w1, w2b)
    assert torch.equal(oa[:, :256].view(torch.int16), oc[:, :256].view(torch.int16))
    assert not torch.equal(oa[:, 256:].view(torch.int16), oc[:, 256:].view(torch.int16))


# ------------------------------------------------------------------ full workload sizes

_WEIGHTS = {}


def weights_for(wl):
    key = (wl.seed, wl.experts, wl.model_dim, wl.inter_dim)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        host = gen.make_weights(wl.seed, wl.experts, wl.model_dim, wl.inter_dim)
        _WEIGHTS[key] = (host, qm.device_weights(*host))
    return _WEIGHTS[key]


# workloads of the 896-expert weight set first, the 112-expert set last (generated once each)
FULL = ["dec-1", "dec-4", "dec-16", "mid-64", "mid-256", "mid-1024", "pre-16384", "pre-a16-2048", "pre-a16-4096",
        "pre-a16-8192", "pre-a16-16384", "pre-a8-8192", "ep-8192"]


@pytest.mark.parametrize("name", FULL)
def test_fused_full_size_covering_every_tile_group(name):
    wl = gen.WORKLOADS[name]
    print(f"full {name}: generating inputs", flush=True)
    host, wd = weights_for(wl)
    p = gen.make_problem(wl, with_weights=False)
    print(f"full {name}: T={wl.tokens} E={wl.experts} I={wl.inter_dim} {wl.a_dtype} bm={wl.block_m}", flush=True)
    out, lay, ws = run_gpu(p["x"], p["topk_ids"], p["topk_w"], wd, 0, wl.experts, wl.block_m, wl.a_dtype,
                           keep_ws=True)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    ids = p["topk_ids"]
    local = ((ids >= 0) & (ids < wl.experts)).any(axis=1)
    assert np.all(got[~local] == 0)
    assert np.all(np.abs(got[local]).sum(axis=1) > 0)
    toks, covered, olay = coverage_tokens(ids, wl.experts, wl.block_m, tile_step=2)
    touched = set(np.unique(ids[(ids >= 0) & (ids < wl.experts)]).tolist())
    # the GPU layout is the oracle's (bit-exact sort), so the sample reaches the GPU's tiles
    assert int(lay.num_tiles.item()) == olay["num_tiles"]
    print(f"  coverage: {len(toks)} tokens, touched experts covered {len(covered)} of {len(touched)}, "
          f"tiles {olay['num_tiles']}", flush=True)
    assert covered == touched
    ref, inter = oracle_tokens(toks, p["x"], wl.a_dtype, *host, ids, p["topk_w"], wl.experts, "situv2", BETA, LBETA,
                               with_intermediate=True)
    ex = explainer(got[toks], ws, lay, inter, toks, wl.a_dtype, "situv2", host, ids, p["topk_w"], 0,
                   wl.model_dim, wl.inter_dim)
    assert_rows_close(got[toks], ref, local[toks], TOL[wl.a_dtype], name, explain=ex)
