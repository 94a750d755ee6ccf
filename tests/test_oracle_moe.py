"""Pins of the MoE oracle (routing sort, SiTUv2, the fused operator) against closed forms,
brute force, a library routine and the statistics printed on the source pages."""
import os

import numpy as np
import pytest
import torch

from oracle import moe as om
from oracle import mx_formats as mx
from quantized_moe_expert_sort_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BETA, LBETA = 4.0, 25.0


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------- SiTUv2

def test_situv2_betas_from_page_module_names():
    # the tags on github ROCm/aiter PR 4471 spell beta and linear_beta as hex floats
    for label, tb, tl, b, lb in _golden("situv2_betas.txt"):
        dec = [float.fromhex(t.replace("d", ".", 1).replace("pp", "p+")) for t in (tb, tl)]
        assert dec == [float(b), float(lb)], label
    assert (float(_golden("situv2_betas.txt")[0][3]), float(_golden("situv2_betas.txt")[0][4])) == (BETA, LBETA)


def test_situv2_gate_saturation_limit():
    # g -> +inf: sigmoid -> 1 and beta*tanh(g/beta) -> beta, so y -> beta*lb*tanh(u/lb)
    u = np.linspace(-300, 300, 1001)
    y = om.situv2(np.full_like(u, 1e4), u, BETA, LBETA)
    assert np.allclose(y, BETA * LBETA * np.tanh(u / LBETA), rtol=1e-15, atol=0)


def test_situv2_up_term_is_odd():
    rng = np.random.default_rng(0)
    g, u = rng.standard_normal(1000) * 5, rng.standard_normal(1000) * 50
    assert np.array_equal(om.situv2(g, -u, BETA, LBETA), -om.situv2(g, u, BETA, LBETA))


def test_situv2_recovers_silu_for_large_betas():
    # beta, lb -> inf: beta*tanh(g/beta) -> g and lb*tanh(u/lb) -> u, so y -> silu(g)*u, and the
    # gap shrinks like 1/beta^2 (tanh(z) = z - z^3/3 + ...)
    rng = np.random.default_rng(1)
    g, u = rng.standard_normal(4000) * 3, rng.standard_normal(4000) * 3
    ref = g / (1 + np.exp(-g)) * u
    errs = [np.max(np.abs(om.situv2(g, u, b, b) - ref)) for b in (1e2, 1e3)]
    assert errs[1] < 1e-2 and 90 < errs[0] / errs[1] < 110


def test_situv2_gate_difference_identity():
    # sigmoid(-g) = 1 - sigmoid(g)  =>  situ(g) - situ(-g) = beta*tanh(g/beta)
    g = np.linspace(-40, 40, 2001)
    up = LBETA * np.tanh(1.0 / LBETA)
    situ = lambda z: om.situv2(z, np.ones_like(z), BETA, LBETA) / up
    assert np.allclose(situ(g) - situ(-g), BETA * np.tanh(g / BETA), rtol=1e-12, atol=1e-12)


def test_situv2_bounds_zeros_and_saturation():
    big = np.array([-1e30, -1e5, -100.0, 0.0, 100.0, 1e5, 1e30])
    G, U = np.meshgrid(big, big)
    y = om.situv2(G, U, BETA, LBETA)
    assert np.all(np.isfinite(y)) and np.all(np.abs(y) <= BETA * LBETA)
    assert np.all(om.situv2(0.0 * big, big, BETA, LBETA) == 0)
    assert np.all(om.situv2(big, 0.0 * big, BETA, LBETA) == 0)


# ----------------------------------------------------------------------------- SiLU epilogue
#
# silu(g) * u (github ROCm/aiter PR 4471, "Motivation": the SiLU path stays next to SiTUv2).
# Pinned by points where the logistic function is rational, by its symmetry, by its limits and
# by the pinned SiTUv2, whose large-beta limit it is.

def test_silu_rational_sigmoid_points():
    # sigmoid(ln k) = k / (k + 1) and sigmoid(-ln k) = 1 / (k + 1)
    for k in (3.0, 7.0, 0.25):
        g = np.log(k)
        for u in (1.0, -2.5, 40.0):
            assert om.silu_mul(g, u) == pytest.approx(g * k / (k + 1) * u, rel=1e-15)
            assert om.silu_mul(-g, u) == pytest.approx(-g / (k + 1) * u, rel=1e-15)


def test_silu_odd_part_and_even_part():
    # silu(g) - silu(-g) = g (sigmoid(g) + sigmoid(-g) = 1); silu(g) + silu(-g) = g tanh(g / 2)
    g = np.linspace(-30, 30, 601)
    one = np.ones_like(g)
    assert np.allclose(om.silu_mul(g, one) - om.silu_mul(-g, one), g, rtol=1e-14, atol=1e-14)
    assert np.allclose(om.silu_mul(g, one) + om.silu_mul(-g, one), g * np.tanh(g / 2), rtol=1e-12, atol=1e-14)


def test_silu_limits_zero_and_linearity_in_up():
    assert om.silu_mul(60.0, 3.0) == pytest.approx(180.0, rel=1e-15)      # g -> +inf: g * u
    assert abs(om.silu_mul(-60.0, 3.0)) < 1e-20                            # g -> -inf: 0
    assert om.silu_mul(0.0, 123.0) == 0.0 and om.silu_mul(1.7, 0.0) == 0.0
    rng = np.random.default_rng(4)
    g, u = rng.standard_normal(100) * 4, rng.standard_normal(100) * 4
    assert np.allclose(om.silu_mul(g, 3 * u), 3 * om.silu_mul(g, u), rtol=1e-14, atol=0)


def test_silu_is_the_large_beta_limit_of_situv2():
    # the SiTUv2 pins above fix situv2; beta = linear_beta -> inf reduces it to silu(g) * u
    # with a gap of order 1/beta^2
    rng = np.random.default_rng(2)
    g, u = rng.standard_normal(4000) * 3, rng.standard_normal(4000) * 3
    errs = [np.max(np.abs(om.situv2(g, u, b, b) - om.silu_mul(g, u))) for b in (1e2, 1e3)]
    assert errs[1] < 1e-2 and 90 < errs[0] / errs[1] < 110


def test_activation_dispatch_selects_silu():
    g, u = np.array([np.log(3.0)]), np.array([2.0])
    assert om.activation(g, u, "silu")[0] == pytest.approx(np.log(3.0) * 0.75 * 2.0, rel=1e-15)


# ----------------------------------------------------------------------------- relL2
#
# relL2 = ||got - ref||_2 / ||ref||_2 over every element (the parity measure of the tests).

def test_rel_l2_hand_computed_values():
    assert om.rel_l2([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert om.rel_l2([0.0, 0.0], [3.0, 4.0]) == 1.0                        # 5 / 5
    assert om.rel_l2([6.0, 8.0], [3.0, 4.0]) == 1.0                        # 5 / 5: normalised by ref
    assert om.rel_l2([3.0, 4.0], [6.0, 8.0]) == 0.5                        # 5 / 10
    assert om.rel_l2([1.0, 2.0, 2.5], [1.0, 2.0, 2.0]) == pytest.approx(0.5 / 3.0, rel=1e-15)
    # every element of a 2-D array counts: ||ref|| = 3, ||diff|| = 0.6
    assert om.rel_l2([[1.0, 2.0], [2.0, 0.6]], [[1.0, 2.0], [2.0, 0.0]]) == pytest.approx(0.2, rel=1e-15)
    # a zero reference: the norm of got itself
    assert om.rel_l2([3.0, 4.0], [0.0, 0.0]) == 5.0


def test_rel_l2_scale_invariance_and_float32_inputs():
    rng = np.random.default_rng(8)
    ref = rng.standard_normal(1000)
    got = ref + 1e-3 * rng.standard_normal(1000)
    r = om.rel_l2(got, ref)
    assert om.rel_l2(1024.0 * got, 1024.0 * ref) == pytest.approx(r, rel=1e-14)
    # float32 inputs are widened before the sums (no float32 accumulation)
    assert om.rel_l2(got.astype(np.float32), ref.astype(np.float32)) == pytest.approx(
        om.rel_l2(got.astype(np.float32).astype(np.float64), ref.astype(np.float32).astype(np.float64)), rel=0)


def test_activation_rejects_unknown_and_missing_betas():
    with pytest.raises(ValueError):
        om.activation(np.zeros(2), np.zeros(2), "swiglu")
    with pytest.raises(ValueError):
        om.activation(np.zeros(2), np.zeros(2), "situv2")


# ----------------------------------------------------------------------------- routing sort

def _brute_layout(ids, eb, E, bm):
    T, K = ids.shape
    keys = sorted((int(ids[t, k]) - eb, t * K + k) for t in range(T) for k in range(K)
                  if 0 <= ids[t, k] - eb < E)
    out, eids = [], []
    for e in range(E):
        vs = [v for (ee, v) in keys if ee == e]
        if not vs:
            continue
        n = -(-len(vs) // bm)
        out += vs + [T * K] * (n * bm - len(vs))
        eids += [e] * n
    return out, eids


@pytest.mark.parametrize("T,K,E,eb,nloc,bm", [(1, 16, 896, 0, 896, 16), (5, 2, 8, 0, 8, 16),
                                               (37, 4, 20, 5, 9, 16), (64, 8, 33, 0, 33, 32),
                                               (300, 6, 40, 0, 40, 32)])
def test_sort_layout_brute_force(T, K, E, eb, nloc, bm):
    rng = np.random.default_rng(T * 7 + K)
    ids = rng.integers(-1, E + 3, size=(T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    lay = om.sort_layout(ids, eb, nloc, bm, topk_w=w)
    want_ids, want_e = _brute_layout(ids, eb, nloc, bm)
    nt = lay["num_tiles"]
    assert nt == len(want_e)
    assert list(lay["sorted_token_ids"][:nt * bm]) == want_ids
    assert list(lay["expert_ids"][:nt]) == want_e
    assert np.all(lay["expert_ids"][nt:] == -1)
    assert np.all(lay["sorted_token_ids"][nt * bm:] == T * K)
    # invariants: each local v once, weights follow ids, padding count, monotone experts
    s = lay["sorted_token_ids"]
    loc = [(t * K + k) for t in range(T) for k in range(K) if eb <= ids[t, k] < eb + nloc]
    assert sorted(s[s < T * K].tolist()) == loc
    assert np.all(lay["sorted_weights"][s < T * K] == w.reshape(-1)[s[s < T * K]])
    assert np.all(lay["sorted_weights"][s == T * K] == 0)
    c = lay["counts"]
    assert int(np.sum(-(-c // bm) * bm - c)) == int(np.sum(s[:nt * bm] == T * K))
    assert np.all(np.diff(lay["expert_ids"][:nt]) >= 0)
    assert lay["cap"] >= nt
    # row_of inverts the layout on local rows and marks the others -1
    ro = lay["row_of"]
    flat = ids.reshape(-1)
    loc_mask = (flat >= eb) & (flat < eb + nloc)
    assert np.all(ro[~loc_mask] == -1)
    assert np.array_equal(s[ro[loc_mask]], np.nonzero(loc_mask)[0])


def test_sort_assignment_count_invariant():
    # sum over experts of routed rows == tokens * topk when every expert is local
    ids, _ = gen.make_routing(3, 50, 64, 6)
    lay = om.sort_layout(ids, 0, 64, 16)
    assert int(lay["counts"].sum()) == 50 * 6


def test_decode_padding_statistic_from_page():
    g = {r[0]: [float(x) for x in r[1:]] for r in _golden("decode_padding.txt")}
    T, E, K, bm = (int(g[k][0]) for k in ("tokens", "experts", "topk", "block_m"))
    ids, _ = gen.make_routing(0, T, E, K)
    lay = om.sort_layout(ids, 0, E, bm)
    c = lay["counts"]
    routed, distinct = int(c.sum()), int(np.count_nonzero(c))
    padded = lay["num_tiles"] * bm
    assert routed == g["routed_rows"][0]
    assert abs(distinct - g["distinct_experts"][0]) <= g["distinct_experts"][1]
    assert abs(routed / distinct - g["rows_per_expert"][0]) <= g["rows_per_expert"][1]
    assert abs((padded - routed) / padded - g["padding_fraction"][0]) <= g["padding_fraction"][1]


# ----------------------------------------------------------------------------- fused operator

def _small_problem(T, E, K, D, I, seed=0, zipf=0.0):
    ids, w = gen.make_routing(seed, T, E, K, zipf)
    x = gen.make_x(seed, T, D)
    w1, w1s, w2, w2s = gen.make_weights(seed, E, D, I)
    return x, ids, w, w1, w1s, w2, w2s


def _per_token_loops(x, a_dtype, w1, w1s, w2, w2s, ids, w, eb, E, act):
    """Pure-Python brute force: for t, for k, explicit dot products."""
    T, D = x.shape
    I = w2.shape[2] * 2
    X = om.activation_values(x, a_dtype)
    out = np.zeros((T, D))
    for t in range(T):
        for k in range(ids.shape[1]):
            e = int(ids[t, k]) - eb
            if not 0 <= e < E:
                continue
            W1 = mx.dequant_mxfp4(w1[e], w1s[e])
            W2 = mx.dequant_mxfp4(w2[e], w2s[e])
            xr = X[t].tolist()
            h = [sum(a * b for a, b in zip(xr, W1[n].tolist())) for n in range(2 * I)]
            y = om.activation(np.array(h[:I]), np.array(h[I:]), act, BETA, LBETA)
            yq = om.requantize_intermediate(y[None, :], a_dtype)[0].tolist()
            for n in range(D):
                out[t, n] += float(w[t, k]) * sum(a * b for a, b in zip(yq, W2[n].tolist()))
    return out


@pytest.mark.parametrize("a_dtype,act", [("bf16", "situv2"), ("fp8", "situv2"),
                                         ("fp4", "situv2"), ("bf16", "silu")])
def test_fused_matches_per_token_brute_force(a_dtype, act):
    T, E, K, D, I = 4, 8, 2, 64, 32
    x, ids, w, w1, w1s, w2, w2s = _small_problem(T, E, K, D, I, seed=11)
    ref = _per_token_loops(x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, E, act)
    got = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, E, act, BETA, LBETA)
    assert np.linalg.norm(ref) > 0
    assert om.rel_l2(got, ref) < 1e-6


def test_tiny_workload_matches_per_token_brute_force():
    wl = gen.WORKLOADS["tiny"]
    p = gen.make_problem(wl)
    ref = _per_token_loops(p["x"], "bf16", p["w1"], p["w1s"], p["w2"], p["w2s"], p["topk_ids"],
                           p["topk_w"], 0, wl.experts, "situv2")
    got = om.moe_fused(p["x"], "bf16", p["w1"], p["w1s"], p["w2"], p["w2s"], p["topk_ids"],
                       p["topk_w"], 0, wl.experts, "situv2", BETA, LBETA)
    assert om.rel_l2(got, ref) < 1e-6


@pytest.mark.parametrize("a_dtype", ["bf16", "fp8", "fp4"])
def test_dense_ffn_special_case_against_torch(a_dtype):
    # one expert, top-1, weight 1: the MoE is a dense gated FFN
    T, D, I = 9, 128, 64
    x, _, _, w1, w1s, w2, w2s = _small_problem(T, 1, 1, D, I, seed=5)
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    got = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, 1, "situv2", BETA, LBETA)
    X = torch.from_numpy(om.activation_values(x, a_dtype))
    W1 = torch.from_numpy(mx.dequant_mxfp4(w1[0], w1s[0]))
    W2 = torch.from_numpy(mx.dequant_mxfp4(w2[0], w2s[0]))
    h = torch.nn.functional.linear(X, W1)
    g, u = h[:, :I], h[:, I:]
    y = BETA * torch.tanh(g / BETA) * torch.sigmoid(g) * LBETA * torch.tanh(u / LBETA)
    y32 = y.to(torch.float32)
    if a_dtype == "bf16":
        yq = y32.to(torch.bfloat16).to(torch.float64)
    else:
        fmt = {"fp8": "e4m3", "fp4": "e2m1"}[a_dtype]
        c, s = mx.quantize_1x32(y32.double().numpy(), fmt)
        yq = torch.from_numpy(mx.dequantize_1x32(c, s, fmt))
    ref = torch.nn.functional.linear(yq, W2).numpy()
    assert om.rel_l2(got, ref) < 1e-12


def test_exact_small_integer_gemm():
    # integer activations and e2m1 weights at scale 2^0: every product and sum is exact,
    # so the oracle's gate/up values equal exact integer arithmetic (in units of 1/2)
    rng = np.random.default_rng(7)
    T, E, K, D, I = 6, 3, 2, 64, 32
    xi = rng.integers(-4, 5, size=(T, D))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes1 = rng.integers(0, 16, size=(E, 2 * I, D))
    codes2 = rng.integers(0, 16, size=(E, D, I))
    w1, w2 = mx.pack_fp4(codes1), mx.pack_fp4(codes2)
    w1s = np.full((E, 2 * I, D // 32), 127, np.uint8)
    w2s = np.full((E, D, I // 32), 127, np.uint8)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = np.ones((T, K), np.float32)
    _, inter = om.moe_fused(x, "bf16", w1, w1s, w2, w2s, ids, w, 0, E, "situv2", BETA, LBETA,
                            return_intermediate=True)
    half = (2 * mx.e2m1_value(np.arange(16))).astype(np.int64)   # e2m1 values times 2
    for e, (vs, g, u, _) in inter.items():
        for r, v in enumerate(vs):
            t = v // K
            h2 = [sum(int(xi[t, k]) * int(half[codes1[e, n, k]]) for k in range(D)) for n in range(2 * I)]
            assert np.array_equal(np.concatenate([g[r], u[r]]) * 2, np.array(h2, dtype=np.float64))


def test_router_weight_linearity_and_unrouted_tokens():
    T, E, K, D, I = 12, 16, 3, 64, 32
    x, ids, w, w1, w1s, w2, w2s = _small_problem(T, E, K, D, I, seed=9)
    # expert-parallel shard: experts 4..7 local; tokens with no local expert output zero
    eb, nloc = 4, 4
    out = om.moe_fused(x, "bf16", w1[eb:eb + nloc], w1s[eb:eb + nloc], w2[eb:eb + nloc],
                       w2s[eb:eb + nloc], ids, w, eb, nloc, "situv2", BETA, LBETA)
    out2 = om.moe_fused(x, "bf16", w1[eb:eb + nloc], w1s[eb:eb + nloc], w2[eb:eb + nloc],
                        w2s[eb:eb + nloc], ids, 2 * w, eb, nloc, "situv2", BETA, LBETA)
    assert np.array_equal(out2, 2 * out)
    local = ((ids >= eb) & (ids < eb + nloc)).any(axis=1)
    assert not local.all() and local.any()
    assert np.all(out[~local] == 0) and np.all(np.abs(out[local]).sum(axis=1) > 0)
    # the shard's output equals the full model's output restricted to local slots
    wmask = np.where((ids >= eb) & (ids < eb + nloc), w, 0).astype(np.float32)
    full = om.moe_fused(x, "bf16", w1, w1s, w2, w2s, ids, wmask, 0, E, "situv2", BETA, LBETA)
    assert om.rel_l2(out, full) < 1e-12


@pytest.mark.parametrize("a_dtype", ["bf16", "fp8", "fp4"])
def test_sampled_tokens_match_expert_major(a_dtype):
    T, E, K, D, I = 20, 12, 4, 128, 64
    x, ids, w, w1, w1s, w2, w2s = _small_problem(T, E, K, D, I, seed=13, zipf=1.1)
    full = om.moe_fused(x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, E, "situv2", BETA, LBETA)
    toks = [0, 7, 19]
    part = om.moe_tokens(toks, x, a_dtype, w1, w1s, w2, w2s, ids, w, 0, E, "situv2", BETA, LBETA)
    assert om.rel_l2(part, full[toks]) < 1e-12
