"""Helpers of the GPU parity tests: per-token comparison with the oracle, a token sample that
reaches every tile of the layout, and the oracle evaluated over expert shards in threads.

The oracle is not changed here: a token's output depends only on its own activation row,
routing and router weights, so the oracle run on a subset of tokens gives exactly those
tokens' outputs, and the outputs of disjoint expert ranges (each run as an expert-parallel
shard) add up to the whole operator's output (pinned by the shard-restriction case of
tests/test_oracle_moe.py)."""
import concurrent.futures
import os

import numpy as np
import threadpoolctl

from oracle import moe as om


def assert_rows_close(got, ref, local, tol, what="", explain=None, tokens=None):
    """Every output row of a token with a local expert: relL2 <= tol and nonzero; every other
    row exactly zero; and the whole output within tol.  Returns (worst row relL2, whole relL2).

    explain(i) (fp8 / fp4 intermediates): a row above tol passes only if explain(i) shows that
    the row's Stage1 requantization took, at a near-tie, a decision other than the oracle's and
    that the row is within tol of the operator evaluated on the GPU's own codes (see
    RequantExplainer); row i is token tokens[i] (default: i)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    local = np.asarray(local, dtype=bool)
    assert np.all(got[~local] == 0), f"{what}: a token without a local expert has a nonzero row"
    rows = np.nonzero(local)[0]
    errs = np.array([om.rel_l2(got[t], ref[t]) for t in rows]) if len(rows) else np.zeros(0)
    zero = [int(t) for t in rows if not np.any(got[t] != 0)]
    assert not zero, f"{what}: zero output rows for local tokens {zero[:8]}"
    worst = float(errs.max()) if len(errs) else 0.0
    bad = rows[errs > tol] if len(errs) else rows[:0]
    whole = om.rel_l2(got, ref)
    print(f"  {what} rows {len(rows)}: worst row relL2 {worst:.3e}, whole relL2 {whole:.3e}", flush=True)
    if len(bad) and explain is not None:
        explained = [int(i) for i in bad if explain(int(i))]
        print(f"  {what}: {len(bad)} rows above {tol}; {len(explained)} explained by near-tie requantization "
              f"decisions (rows {explained[:8]})", flush=True)
        bad = np.array([i for i in bad if int(i) not in set(explained)], dtype=np.int64)
        for i in bad[:8]:
            print(f"  {what}: row {int(i)} (relL2 {errs[np.searchsorted(rows, i)]:.3e}) not explained: "
                  f"{getattr(explain, 'reasons', {}).get(int(i), '?')}", flush=True)
    assert len(bad) == 0, f"{what}: {len(bad)} token rows above {tol} (worst {worst:.3e}, tokens {bad[:8].tolist()})"
    assert whole <= tol
    return worst, whole


def coverage_tokens(topk_ids, num_local_experts, block_m, tile_step=2):
    """Tokens whose routed rows reach every expert that has rows, every tile_step-th tile of
    each expert and each expert's last tile, from the oracle's layout.  Any grouping of an
    expert's consecutive tiles into parts of at least tile_step tiles (plus a possibly shorter
    last part) then has a routed row in every part.  Tokens are chosen greedily (those reaching
    the most required tiles first), so the sample stays small.
    Returns (sorted tokens, experts reached, oracle layout)."""
    topk_ids = np.asarray(topk_ids)
    lay = om.sort_layout(topk_ids, 0, num_local_experts, block_m)
    nt, eids, row_of = lay["num_tiles"], lay["expert_ids"], lay["row_of"]
    T, K = topk_ids.shape
    need = set()
    start = 0
    while start < nt:
        end = start
        while end < nt and eids[end] == eids[start]:
            end += 1
        need.update(range(start, end, tile_step))
        need.add(end - 1)
        start = end
    tiles_of = np.where(row_of >= 0, row_of // block_m, -1).reshape(T, K)
    toks = []
    for m in range(K, 0, -1):                             # tokens reaching >= m uncovered tiles
        if not need:
            break
        for t in range(T):
            hit = {int(x) for x in tiles_of[t] if x in need}
            if len(hit) >= m:
                toks.append(t)
                need -= hit
    assert not need
    reached = {int(eids[x]) for t in toks for x in tiles_of[t] if x >= 0}
    return sorted(toks), reached, lay


def oracle_tokens(tokens, x, a_dtype, w1, w1s, w2, w2s, topk_ids, topk_w, num_local_experts, act,
                  beta, linear_beta, shard=32, threads=None, with_intermediate=False):
    """The oracle's output rows of `tokens` ([len(tokens), D] float64): the expert-major oracle
    on those tokens, run as expert shards [a, a + shard) in a thread pool and summed.  With
    with_intermediate, also the oracle's per-expert (flat indices v = t*topk + k of the whole
    problem, g, u, requantized y), keyed by local expert."""
    tokens = np.asarray(tokens, dtype=np.int64)
    xs, ids, w = np.asarray(x)[tokens], np.asarray(topk_ids)[tokens], np.asarray(topk_w)[tokens]
    E, K = num_local_experts, ids.shape[1]
    shards = [(a, min(E, a + shard)) for a in range(0, E, shard)]

    def one(ab):
        a, b = ab
        if not np.any((ids >= a) & (ids < b)):
            return None
        return a, om.moe_fused(xs, a_dtype, w1[a:b], w1s[a:b], w2[a:b], w2s[a:b], ids, w, a, b - a, act,
                               beta, linear_beta, return_intermediate=True)

    n = threads or min(16, os.cpu_count() or 1)
    # one BLAS thread per shard thread: the pool itself uses the cores
    with threadpoolctl.threadpool_limits(1), concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
        parts = [r for r in ex.map(one, shards) if r is not None]
    out = np.zeros((len(tokens), np.asarray(x).shape[1]), dtype=np.float64)
    inter = {}
    for a, (r, it) in parts:
        out += r
        for e, (vs, g, u, yq) in it.items():
            inter[a + e] = (tokens[vs // K] * K + vs % K, g, u, yq)
    return (out, inter) if with_intermediate else out


class RequantExplainer:
    """For fp8 / fp4 intermediates: explains a token row that differs from the oracle by more
    than the bar through Stage1 requantization decisions taken at near-ties.

    Both sides decide the intermediate's 1x32 codes in float32, but from values that differ in
    the last bits (fp32 sums in another order and the GPU's exp2 / reciprocal against float64
    libm), so where a value sits within a hair of a rounding boundary the two sides may pick
    neighbouring codes, or neighbouring block scales where a block maximum sits at a power of
    two.  For a row with one or two local experts such a decision can move the row by a few
    percent.  explain(i) holds when, for every local slot (t, k) of token t = tokens[i]:
      * every block scale byte the GPU wrote differs from the oracle's only where the oracle's
        block maximum lies within rel_eps (relative) of a power of two, and every element code
        differs only where the oracle's scaled value lies within rel_eps x the block's largest
        scaled value of a midpoint of the code grid (the two sides' values differ by fp32
        rounding of sums whose size is that of the block's large values, not of the element);
    and the GPU row is within tol of sum_k w[t,k] * W2[e] . dequant(GPU codes), the operator
    evaluated on the GPU's own intermediate.  Everything is decoded with the oracle's codecs."""

    def __init__(self, got, ws_host, row_of, inter, tokens, a_dtype, act, beta, linear_beta, w2, w2s, topk_ids,
                 topk_w, expert_begin, model_dim, inter_dim, layout_rows, tol, off_c, off_s, rel_eps=1e-5):
        """off_c, off_s: byte offsets of the intermediate codes and scales in the workspace."""
        from oracle import mx_formats as mx
        self.mx = mx
        self.fmt = {"fp8": "e4m3", "fp4": "e2m1"}[a_dtype]
        I, D = inter_dim, model_dim
        rb = I if a_dtype == "fp8" else I // 2
        ws_host = np.asarray(ws_host, dtype=np.uint8)
        self.codes = ws_host[off_c:off_c + layout_rows * rb].reshape(layout_rows, rb)
        self.scales = ws_host[off_s:off_s + layout_rows * (I // 32)].reshape(layout_rows, I // 32)
        self.where = {}
        for e, (vs, g, u, _) in inter.items():
            for r, v in enumerate(vs):
                self.where[int(v)] = (e, g[r], u[r])
        self.got, self.row_of, self.tokens = got, row_of, tokens
        self.a_dtype, self.act, self.beta, self.lb = a_dtype, act, beta, linear_beta
        self.w2, self.w2s, self.ids, self.w = w2, w2s, np.asarray(topk_ids), np.asarray(topk_w)
        self.eb, self.tol, self.eps = expert_begin, tol, rel_eps
        grid = mx.e4m3_value(np.arange(127)) if self.fmt == "e4m3" else mx.e2m1_value(np.arange(8))
        self.mids = (grid[1:] + grid[:-1]) / 2
        self.reasons = {}

    def _gpu_codes(self, R):
        c = self.codes[R]
        return self.mx.unpack_fp4(c).astype(np.int64) if self.fmt == "e2m1" else c.astype(np.int64)

    def near_tie(self, y32, gc, gs):
        """(True, n differences) if every difference is at a near-tie, else (False, why)."""
        oc, os_ = self.mx.quantize_1x32(y32, self.fmt)
        n = 0
        for b in range(len(gs)):
            blk = slice(32 * b, 32 * b + 32)
            if gs[b] != os_[b]:
                amax = float(np.max(np.abs(y32[blk])))
                m, _ = np.frexp(amax)                    # amax = m * 2^e, m in [0.5, 1)
                d = min(abs(2 * m - 1), abs(1 - m)) if amax else np.inf
                if d > self.eps:
                    return False, f"block {b}: scale {int(gs[b])} vs {int(os_[b])}, amax {amax:.6g} at {d:.2e} from 2^n"
                n += 1
                continue
            diff = np.nonzero(gc[blk] != oc[blk])[0]
            if len(diff) == 0:
                continue
            unit = np.ldexp(1.0, int(os_[b]) - 127)
            top = float(np.max(np.abs(y32[blk]))) / unit
            for j in diff:
                v = abs(float(y32[blk][j])) / unit
                d = np.min(np.abs(self.mids - v)) / top
                if d > self.eps:
                    return False, (f"block {b} element {int(j)}: code {int(gc[blk][j])} vs {int(oc[blk][j])}, "
                                   f"scaled value {v:.6g} at {d:.2e} of the block maximum from a midpoint")
                n += 1
        return True, n

    def __call__(self, i):
        from oracle import moe as om
        t = int(self.tokens[i]) if self.tokens is not None else int(i)
        K = self.ids.shape[1]
        ref = np.zeros(self.got.shape[1])
        for k in range(K):
            v = t * K + k
            if v not in self.where:
                continue                                   # not a local slot
            e, g, u = self.where[v]
            y32 = np.asarray(om.activation(g, u, self.act, self.beta, self.lb), dtype=np.float32).astype(np.float64)
            R = int(self.row_of[v])
            gc, gs = self._gpu_codes(R), self.scales[R]
            ok, why = self.near_tie(y32, gc, gs)
            if not ok:
                self.reasons[i] = f"slot k={k} (expert {e}, layout row {R}): {why}"
                return False
            self.reasons.setdefault(i, "")
            self.reasons[i] += f"k={k}: {why} near-tie differences; "
            yg = self.mx.dequantize_1x32(gc, gs, self.fmt)
            W2 = self.mx.dequant_mxfp4(self.w2[e], self.w2s[e])
            ref += float(self.w[t, k]) * (W2 @ yg)
        err = om.rel_l2(self.got[i], ref)
        self.reasons[i] = self.reasons.get(i, "") + f"relL2 on the GPU's codes {err:.3e}"
        return err <= self.tol
