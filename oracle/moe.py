"""Fused two-stage MoE FFN, as a plain float64 CPU definition (test infrastructure only).

What is computed (github ROCm/aiter PR 6259 "Motivation" and "Technical Details";
PR 5118 "Summary"; PR 4463 "What"; PR 4471 "Technical Details"):

  1. Routing sort: routed rows (t, k) are grouped by local expert, each expert padded to a
     whole block_m with a sentinel (PR 5118, "Summary": moe_sorting pads every expert up to a
     full block_m).
  2. Stage1: for every routed row, h = W1[e] . X[t] over K = model_dim; the first inter_dim
     rows of W1 are the gate, the next inter_dim rows the up projection; y = act(g, u) with
     SiTUv2: beta*tanh(g/beta)*sigmoid(g) * linear_beta*tanh(u/linear_beta)
     (PR 6259, "Motivation"), or SiLU: silu(g) * u (PR 4471, "Motivation").
  3. The stage1 output is re-encoded in the activation dtype before Stage2: bf16 for a16,
     fp8 1x32 for a8, fp4x2 1x32 for a4 (PR 4463, "Three tuner defects", item 2: the fused
     fp4 stage1 writes an fp4x2 intermediate).
  4. Stage2: o = W2[e] . y over K = inter_dim, scaled by the router weight topk_w[t, k] and
     summed into out[t] (PR 5118 review, item 10 and the commit notes: atomic scatter into
     the token rows).

Readings where the pages are silent: gate rows first in W1 ("[gate|up]"); the router weight
multiplies the Stage2 result; a16 intermediates are rounded to bf16 (the a16 stage2 consumes
bf16 activations); a token with no local expert gets a zero output row; within an expert,
routed rows are ordered by ascending flat index v = t*topk + k; the padding sentinel is T*topk;
experts with no rows get no tile; unused tail tiles carry expert id -1.

Precision: float64 accumulation and activation.  Where floating point decides a code (the
requantization of the stage1 output), the value is first rounded to float32, the precision
in which the GPU takes the same decision.

Parity pins: see tests/test_oracle_moe.py -- SiTUv2 closed forms and limits; SiLU at points
where the logistic function is rational (g = +-ln k), its odd and even parts, its limits, and
as the large-beta limit of the pinned SiTUv2; relL2 against hand-computed values (normalised
by the reference, every element counted); a brute-force sort via Python's sorted(), sort
invariants and the decode padding statistic printed on PR 5118; a pure-Python per-token loop
on tiny inputs; the dense-FFN special case against torch's linear algebra; and an exact
small-integer GEMM case.  Every function here is pinned.
"""
import numpy as np
import scipy.special
import torch

from . import mx_formats as mx

ACT_SITUV2 = "situv2"
ACT_SILU = "silu"


# ---------------------------------------------------------------- bf16 helpers (torch casts)

def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def round_to_bf16(v):
    """float64 -> float32 -> nearest bf16 (ties to even), returned as float64."""
    t = torch.from_numpy(np.asarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- activations

def situv2(g, u, beta, linear_beta):
    """SiTUv2 (PR 6259, "Motivation"): beta*tanh(g/beta)*sigmoid(g) * lb*tanh(u/lb)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return beta * np.tanh(g / beta) * scipy.special.expit(g) * (linear_beta * np.tanh(u / linear_beta))


def silu_mul(g, u):
    """SiLU epilogue (PR 4471, "Motivation"): silu(g) * u."""
    g = np.asarray(g, dtype=np.float64)
    return g * scipy.special.expit(g) * np.asarray(u, dtype=np.float64)


def activation(g, u, act, beta=None, linear_beta=None):
    if act == ACT_SITUV2:
        if beta is None or linear_beta is None:
            raise ValueError("SiTUv2 needs both betas; there are no defaults")
        return situv2(g, u, beta, linear_beta)
    if act == ACT_SILU:
        return silu_mul(g, u)
    raise ValueError(f"act must be 'silu' or 'situv2', got {act!r}")


# ---------------------------------------------------------------- routing sort

def cap_tiles(T, topk, num_local_experts, block_m):
    """Upper bound on sum_e ceil(c_e / block_m): ceil(T*topk/bm) + min(E, T*topk)."""
    n = T * topk
    return -(-n // block_m) + min(num_local_experts, n)


def sort_layout(topk_ids, expert_begin, num_local_experts, block_m, topk_w=None, cap=None):
    """Padded expert-major layout of the routed rows.

    Returns dict with sorted_token_ids [cap*bm] int32 (flat index v = t*topk + k, sentinel
    T*topk), sorted_weights [cap*bm] float32 (0 on padding), expert_ids [cap] int32 (local
    expert index, -1 past num_tiles), row_of [T*topk] int32 (position of row v in
    sorted_token_ids, -1 if its expert is not local), num_tiles int, counts [E] int."""
    topk_ids = np.asarray(topk_ids)
    T, K = topk_ids.shape
    flat = topk_ids.reshape(-1)
    sentinel = T * K
    if cap is None:
        cap = cap_tiles(T, K, num_local_experts, block_m)
    ids = np.full(cap * block_m, sentinel, dtype=np.int32)
    wts = np.zeros(cap * block_m, dtype=np.float32)
    eids = np.full(cap, -1, dtype=np.int32)
    counts = np.zeros(num_local_experts, dtype=np.int64)
    wflat = None if topk_w is None else np.asarray(topk_w, dtype=np.float32).reshape(-1)
    tile = 0
    for e in range(num_local_experts):
        vs = np.nonzero(flat == expert_begin + e)[0]          # ascending v
        counts[e] = len(vs)
        if len(vs) == 0:
            continue
        ntile = -(-len(vs) // block_m)
        if tile + ntile > cap:
            raise ValueError("capacity too small")
        start = tile * block_m
        ids[start:start + len(vs)] = vs
        if wflat is not None:
            wts[start:start + len(vs)] = wflat[vs]
        eids[tile:tile + ntile] = e
        tile += ntile
    row_of = np.full(T * K, -1, dtype=np.int32)
    for pos in range(tile * block_m):
        if ids[pos] != sentinel:
            row_of[ids[pos]] = pos
    return {"sorted_token_ids": ids, "sorted_weights": wts, "expert_ids": eids, "row_of": row_of,
            "num_tiles": tile, "counts": counts, "cap": cap}


# ---------------------------------------------------------------- activations in a_dtype

def activation_values(x_bf16_bits, a_dtype):
    """The values Stage1 multiplies: bf16 as is, or rule-Q fp8 / fp4 codes times scales."""
    X = bf16_bits_to_f64(x_bf16_bits)
    if a_dtype == "bf16":
        return X
    if a_dtype == "fp8":
        c, s = mx.quantize_1x32(X, "e4m3")
        return mx.dequantize_1x32(c, s, "e4m3")
    if a_dtype == "fp4":
        c, s = mx.quantize_1x32(X, "e2m1")
        return mx.dequantize_1x32(c, s, "e2m1")
    raise ValueError(f"unknown a_dtype {a_dtype!r}")


def requantize_intermediate(y, a_dtype):
    """Re-encode the stage1 output in the activation dtype (decision taken on float32 y)."""
    y32 = np.asarray(y, dtype=np.float32).astype(np.float64)
    if a_dtype == "bf16":
        return round_to_bf16(y32)
    fmt = {"fp8": "e4m3", "fp4": "e2m1"}[a_dtype]
    c, s = mx.quantize_1x32(y32, fmt)
    return mx.dequantize_1x32(c, s, fmt)


# ---------------------------------------------------------------- the fused operator

def expert_weights(w1, w1s, w2, w2s, e):
    """Dequantized W1[e] [2I, D] and W2[e] [D, I] in float64."""
    return mx.dequant_mxfp4(w1[e], w1s[e]), mx.dequant_mxfp4(w2[e], w2s[e])


def stage1_rows(Xrows, W1, act, beta, linear_beta):
    """Gate/up GEMM and activation for a block of rows: returns (g, u, y) float64."""
    I = W1.shape[0] // 2
    h = Xrows @ W1.T
    g, u = h[:, :I], h[:, I:]
    return g, u, activation(g, u, act, beta, linear_beta)


def moe_fused(x_bf16_bits, a_dtype, w1, w1s, w2, w2s, topk_ids, topk_w,
              expert_begin, num_local_experts, act, beta=None, linear_beta=None,
              return_intermediate=False):
    """Expert-major evaluation of the whole operator.  Returns out [T, D] float64
    (and, on request, a dict of per-expert (rows, g, u, y_requantized))."""
    topk_ids = np.asarray(topk_ids)
    topk_w = np.asarray(topk_w, dtype=np.float32)
    T, D = np.asarray(x_bf16_bits).shape
    X = activation_values(x_bf16_bits, a_dtype)
    out = np.zeros((T, D), dtype=np.float64)
    inter = {}
    for e in range(num_local_experts):
        t_idx, k_idx = np.nonzero(topk_ids == expert_begin + e)   # ascending v = t*K + k
        if len(t_idx) == 0:
            continue
        W1, W2 = expert_weights(w1, w1s, w2, w2s, e)
        g, u, y = stage1_rows(X[t_idx], W1, act, beta, linear_beta)
        yq = requantize_intermediate(y, a_dtype)
        o = (yq @ W2.T) * topk_w[t_idx, k_idx].astype(np.float64)[:, None]
        np.add.at(out, t_idx, o)
        if return_intermediate:
            inter[e] = (t_idx * topk_ids.shape[1] + k_idx, g, u, yq)
    return (out, inter) if return_intermediate else out


def moe_tokens(token_list, x_bf16_bits, a_dtype, w1, w1s, w2, w2s, topk_ids, topk_w,
               expert_begin, num_local_experts, act, beta=None, linear_beta=None):
    """Outputs of selected tokens only, one token at a time (for sampled checks at full
    size): out[i] = sum_k topk_w[t,k] * W2[e] . requant(act(W1[e] . X[t]))."""
    topk_ids = np.asarray(topk_ids)
    topk_w = np.asarray(topk_w, dtype=np.float32)
    D = np.asarray(x_bf16_bits).shape[1]
    res = np.zeros((len(token_list), D), dtype=np.float64)
    cache = {}
    for i, t in enumerate(token_list):
        X = activation_values(np.asarray(x_bf16_bits)[t:t + 1], a_dtype)
        for k in range(topk_ids.shape[1]):
            e = int(topk_ids[t, k]) - expert_begin
            if not 0 <= e < num_local_experts:
                continue
            if e not in cache:
                cache[e] = expert_weights(w1, w1s, w2, w2s, e)
            W1, W2 = cache[e]
            _, _, y = stage1_rows(X, W1, act, beta, linear_beta)
            yq = requantize_intermediate(y, a_dtype)
            res[i] += float(topk_w[t, k]) * (yq @ W2.T)[0]
    return res


def rel_l2(got, ref):
    """||got - ref||_2 / ||ref||_2 accumulated in float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.sqrt(np.sum(ref * ref))
    return float(np.sqrt(np.sum((got - ref) ** 2)) / den) if den > 0 else float(np.sqrt(np.sum(got * got)))
