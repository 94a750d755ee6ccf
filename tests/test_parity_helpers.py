"""The GPU parity tests' helpers (tests/_parity.py) on the CPU: the token sample reaches every
expert and tile it claims to, and the sharded oracle equals the oracle on the whole problem."""
import numpy as np
import pytest

from oracle import moe as om
from quantized_moe_expert_sort_amd import inputs as gen
from _parity import assert_rows_close, coverage_tokens, oracle_tokens

BETA, LBETA = gen.BETA, gen.LINEAR_BETA


@pytest.mark.parametrize("T,E,K,bm,zipf,step", [(300, 24, 6, 16, 1.1, 2), (2000, 40, 4, 32, 0.0, 2),
                                                 (2000, 40, 4, 32, 1.1, 4)])
def test_coverage_tokens_reach_every_expert_and_every_step_of_tiles(T, E, K, bm, zipf, step):
    ids, _ = gen.make_routing(T + E, T, E, K, zipf)
    toks, experts, lay = coverage_tokens(ids, E, bm, tile_step=step)
    assert experts == set(np.unique(ids).tolist())
    tset = set(toks)
    nt, sid, eid = lay["num_tiles"], lay["sorted_token_ids"], lay["expert_ids"]
    for e in experts:
        tiles = np.nonzero(eid[:nt] == e)[0]
        for j, tl in enumerate(tiles):
            rows = sid[tl * bm:(tl + 1) * bm]
            hit = any(int(v) // K in tset for v in rows if v < T * K)
            if j % step == 0 or j == len(tiles) - 1:
                assert hit, (e, j)
    # any cut of an expert's tiles into runs of >= step tiles has a sampled token in each run
    for e in experts:
        tiles = np.nonzero(eid[:nt] == e)[0]
        for s0 in range(0, len(tiles) - step + 1):
            run = tiles[s0:s0 + step]
            assert any(int(v) // K in tset for tl in run for v in sid[tl * bm:(tl + 1) * bm] if v < T * K)


@pytest.mark.parametrize("a_dtype,shard", [("bf16", 3), ("fp8", 32), ("fp4", 5)])
def test_sharded_oracle_equals_whole_oracle(a_dtype, shard):
    T, E, K, D, I = 40, 12, 4, 128, 64
    ids, w = gen.make_routing(9, T, E, K, 1.1)
    x = gen.make_x(9, T, D)
    host = gen.make_weights(9, E, D, I)
    whole = om.moe_fused(x, a_dtype, *host, ids, w, 0, E, "situv2", BETA, LBETA)
    toks = [0, 3, 17, 39]
    part = oracle_tokens(toks, x, a_dtype, *host, ids, w, E, "situv2", BETA, LBETA, shard=shard, threads=4)
    assert om.rel_l2(part, whole[toks]) < 1e-12


def test_assert_rows_close_catches_one_bad_row():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3000, 64))
    local = np.ones(3000, bool)
    local[7] = False
    ref[7] = 0
    got = ref * (1 + 1e-3 * rng.standard_normal(ref.shape))
    assert_rows_close(got, ref, local, 2e-2)
    bad = got.copy()
    bad[1234] = 0                                        # one zeroed row of 3000: whole relL2 ~ 0.018
    assert om.rel_l2(bad, ref) < 2e-2
    with pytest.raises(AssertionError):
        assert_rows_close(bad, ref, local, 2e-2)
    bad = got.copy()
    bad[7, 3] = 1.0                                      # a token without a local expert
    with pytest.raises(AssertionError):
        assert_rows_close(bad, ref, local, 2e-2)


def _fake_workspace(a_dtype, inter, lay, D, I):
    """A moe_fused workspace holding the oracle's own intermediate codes at each row's layout
    position (what a GPU that decided exactly as the oracle would have written)."""
    from oracle import mx_formats as mx
    import quantized_moe_expert_sort_amd as qm
    fmt = {"fp8": "e4m3", "fp4": "e2m1"}[a_dtype]
    rows = lay["cap"] * 16
    rb = I if a_dtype == "fp8" else I // 2
    parts = qm.fused_ws_parts(len(lay["row_of"]) // 2, D, I, lay["cap"], 16, qm.DTYPES[a_dtype], qm.ACT_SITUV2)
    off_c, off_s = parts["inter"], parts["iscale"]
    ws = np.zeros(parts["total"], np.uint8)
    for e, (vs, g, u, _) in inter.items():
        for r, v in enumerate(vs):
            y32 = np.asarray(om.activation(g[r], u[r], "situv2", BETA, LBETA), np.float32).astype(np.float64)
            c, sc = mx.quantize_1x32(y32, fmt)
            R = lay["row_of"][v]
            ws[off_c + R * rb:off_c + (R + 1) * rb] = mx.pack_fp4(c) if fmt == "e2m1" else c.astype(np.uint8)
            ws[off_s + R * (I // 32):off_s + (R + 1) * (I // 32)] = sc
    return ws, off_c, off_s, rb


@pytest.mark.parametrize("a_dtype", ["fp8", "fp4"])
def test_requant_explainer_accepts_near_ties_only(a_dtype):
    from _parity import RequantExplainer
    from oracle import mx_formats as mx
    T, E, K, D, I = 12, 6, 2, 64, 64
    ids, w = gen.make_routing(4, T, E, K)
    x = gen.make_x(4, T, D)
    host = gen.make_weights(4, E, D, I)
    ref, inter = om.moe_fused(x, a_dtype, *host, ids, w, 0, E, "situv2", BETA, LBETA, return_intermediate=True)
    lay = om.sort_layout(ids, 0, E, 16)
    ws, off_c, off_s, rb = _fake_workspace(a_dtype, inter, lay, D, I)
    mk = lambda got, ws_, eps: RequantExplainer(got, ws_, lay["row_of"], inter, None, a_dtype, "situv2", BETA, LBETA,
                                                host[2], host[3], ids, w, 0, D, I, lay["cap"] * 16, 2e-2, off_c, off_s,
                                                rel_eps=eps)
    assert all(mk(ref, ws, 1e-5)(t) for t in range(T))          # the oracle's own codes: nothing to explain
    # change one element code of token 0's first slot where the value is far from a grid midpoint
    e, (vs, g, u, _) = next((e, it) for e, it in inter.items() if 0 in it[0].tolist())
    r = vs.tolist().index(0)
    y32 = np.asarray(om.activation(g[r], u[r], "situv2", BETA, LBETA), np.float32).astype(np.float64)
    codes, sc = mx.quantize_1x32(y32, {"fp8": "e4m3", "fp4": "e2m1"}[a_dtype])
    i = int(np.argmax(np.abs(y32)))
    bad = codes.copy()
    bad[i] = bad[i] - 1 if (bad[i] & 0x7) else bad[i] + 1       # a neighbouring code
    ws2 = ws.copy()
    R = lay["row_of"][0]
    ws2[off_c + R * rb:off_c + (R + 1) * rb] = mx.pack_fp4(bad) if a_dtype == "fp4" else bad.astype(np.uint8)
    # far from a tie: not explained, whatever the output row
    assert not mk(ref, ws2, 1e-5)(0)
    # taken as a tie (a loose eps): explained only when the row matches the operator on those codes
    fmt = {"fp8": "e4m3", "fp4": "e2m1"}[a_dtype]
    W2 = mx.dequant_mxfp4(host[2][e], host[3][e])
    delta = float(w[0, 0]) * (W2 @ (mx.dequantize_1x32(bad, sc, fmt) - mx.dequantize_1x32(codes, sc, fmt)))
    assert mk(ref + np.vstack([delta, np.zeros((T - 1, D))]), ws2, 1.0)(0)
    assert not mk(ref + np.vstack([delta + 0.5 * np.abs(ref[0]).max(), np.zeros((T - 1, D))]), ws2, 1.0)(0)
