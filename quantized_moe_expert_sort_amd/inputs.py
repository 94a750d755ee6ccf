"""Seeded synthetic inputs for the fused MXFP4 MoE (shared by the tests and the benchmark).

Holds no arithmetic of the operator itself: it only draws random data.

* x: bf16 activations ~ N(0, 1).
* Routing: router logits ~ N(0, 1) (optionally plus a Zipf prior -s*ln(rank) per expert),
  softmax in float64, stable top-k (lower expert id wins a tie), renormalized, cast to fp32.
* MXFP4 weights ~ N(0, 0.02) as they look after 1x32 e8m0 block quantization, drawn directly
  in code space: each 32-element block draws its scale byte from the distribution of the
  binade of the largest of 32 |N(0, 0.02^2)| samples (shifted by the e2m1 exponent range),
  and each element draws a sign and an e2m1 magnitude code from the distribution that
  N(0, (0.02 / scale)^2) places on the cells of the e2m1 value grid.  Each expert has its
  own seed stream, so a shard of experts 0..E_local-1 equals the same experts of the full set.

Workload shapes follow the tuned wide-MoE shape of the source pages (896 experts, top-16,
model_dim 3584, inter_dim 384 per tensor-parallel shard, or 112 local experts with inter_dim
3072 per expert-parallel rank).
"""
import concurrent.futures
import math
import os
from dataclasses import dataclass

import numpy as np
import torch

# ----------------------------------------------------------------------------- workloads


@dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    experts: int            # local experts held on this GPU
    topk: int
    model_dim: int
    inter_dim: int
    a_dtype: str            # "bf16" | "fp8" | "fp4"
    global_experts: int = 0  # experts the router chooses from (0: same as experts)
    zipf_s: float = 0.0
    seed: int = 0

    @property
    def router_experts(self):
        return self.global_experts or self.experts

    @property
    def block_m(self):
        # decode/mid batches at 16 rows per tile, larger batches at 32
        return 16 if self.tokens <= 512 else 32


BETA, LINEAR_BETA = 4.0, 25.0

WORKLOADS = {
    "tiny": Workload("tiny", 4, 8, 2, 256, 128, "bf16"),
    "dec-1": Workload("dec-1", 1, 896, 16, 3584, 384, "bf16"),
    "dec-4": Workload("dec-4", 4, 896, 16, 3584, 384, "bf16"),
    "dec-16": Workload("dec-16", 16, 896, 16, 3584, 384, "bf16"),
    "mid-64": Workload("mid-64", 64, 896, 16, 3584, 384, "fp8"),
    "mid-256": Workload("mid-256", 256, 896, 16, 3584, 384, "fp8"),
    "mid-1024": Workload("mid-1024", 1024, 896, 16, 3584, 384, "fp8"),
    "ep-8192": Workload("ep-8192", 8192, 112, 16, 3584, 3072, "fp8", global_experts=896),
    "pre-16384": Workload("pre-16384", 16384, 896, 16, 3584, 384, "fp4", zipf_s=1.1),
    # the pages' own large-batch timing shape (uniform routing over all 896 experts)
    "pre-a16-2048": Workload("pre-a16-2048", 2048, 896, 16, 3584, 384, "bf16"),
    "pre-a16-4096": Workload("pre-a16-4096", 4096, 896, 16, 3584, 384, "bf16"),
    "pre-a16-8192": Workload("pre-a16-8192", 8192, 896, 16, 3584, 384, "bf16"),
    "pre-a16-16384": Workload("pre-a16-16384", 16384, 896, 16, 3584, 384, "bf16"),
    "pre-a8-8192": Workload("pre-a8-8192", 8192, 896, 16, 3584, 384, "fp8"),
}

# ----------------------------------------------------------------------------- generators

_X, _ROUTE, _W1, _W2 = 1, 2, 3, 4


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def make_x(seed, T, D):
    """bf16 bit patterns (uint16 [T, D]) of N(0, 1) samples."""
    v = _rng(seed, _X).standard_normal((T, D), dtype=np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_routing(seed, T, E, K, zipf_s=0.0):
    """(topk_ids int32 [T, K], topk_w float32 [T, K]) over E router experts."""
    logits = _rng(seed, _ROUTE).standard_normal((T, E), dtype=np.float32).astype(np.float64)
    if zipf_s:
        logits = logits - zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))[None, :]
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :K]
    w = np.take_along_axis(p, ids, axis=1)
    w /= w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


# e2m1 value-grid cell edges (midpoints between 0, .5, 1, 1.5, 2, 3, 4, 6)
_E2M1_EDGES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_SIGMA_W = 0.02


def _phi_abs(a, sigma):
    """P(|N(0, sigma^2)| < a)."""
    return math.erf(a / (sigma * math.sqrt(2.0)))


def _scale_byte_table():
    """Scale bytes and probabilities: the largest of 32 |N(0, 0.02^2)| lies in binade
    [2^b, 2^(b+1)); the block scale byte is b - 2 + 127."""
    out = []
    for b in range(-9, 0):
        lo, hi = 2.0 ** b, 2.0 ** (b + 1)
        p = _phi_abs(hi, _SIGMA_W) ** 32 - _phi_abs(lo, _SIGMA_W) ** 32
        if p > 1e-7:
            out.append((b - 2 + 127, p))
    tot = sum(p for _, p in out)
    return [(s, p / tot) for s, p in out]


def _element_lut(scale_byte):
    """256-entry table: uniform byte -> e2m1 code (bit 0 of the byte is the sign)."""
    sigma = _SIGMA_W / 2.0 ** (scale_byte - 127)
    cdf = [_phi_abs(m, sigma) for m in _E2M1_EDGES] + [1.0]
    lut = np.zeros(256, dtype=np.uint8)
    for u in range(256):
        q = ((u >> 1) + 0.5) / 128.0
        mag = next(i for i, c in enumerate(cdf) if q <= c)
        lut[u] = mag | ((u & 1) << 3)
    return lut


def _top_code6_prob(scale_byte):
    """P(magnitude code 6 | the block's largest value in the top binade [4, 8) x 2^sexp): the
    share of [4, 8) that rounds to 4.0 rather than 6.0, under N(0, (0.02 / 2^sexp)^2)."""
    sigma = _SIGMA_W / 2.0 ** (scale_byte - 127)
    p6 = _phi_abs(5.0, sigma) - _phi_abs(4.0, sigma)
    p7 = _phi_abs(8.0, sigma) - _phi_abs(5.0, sigma)
    return p6 / (p6 + p7)


_SCALES = _scale_byte_table()
_SCALE_BYTES = np.array([s for s, _ in _SCALES], dtype=np.uint8)
_SCALE_CDF = np.cumsum([p for _, p in _SCALES])
_ELEM_LUTS = np.stack([_element_lut(int(s)) for s in _SCALE_BYTES])   # [nscale, 256]
_TOP6 = np.array([_top_code6_prob(int(s)) for s in _SCALE_BYTES])


def make_mxfp4_expert(seed, tensor_id, e, N, K):
    """One expert's MXFP4 weight: (packed uint8 [N, K/2], scales uint8 [N, K/32])."""
    rng = _rng(seed, tensor_id, e)
    sidx = np.searchsorted(_SCALE_CDF, rng.random((N, K // 32)), side="right")
    sidx = np.minimum(sidx, len(_SCALE_BYTES) - 1).astype(np.intp)
    u = rng.integers(0, 256, size=(N, K // 32, 32), dtype=np.uint8)
    main = int(np.argmax(np.bincount(sidx.ravel(), minlength=len(_SCALE_BYTES))))
    codes = _ELEM_LUTS[main][u]
    for j in range(len(_SCALE_BYTES)):
        if j != main:
            sel = sidx == j
            codes[sel] = _ELEM_LUTS[j][u[sel]]
    # A block's scale byte stands for the binade of its largest |value|, so (as in any block
    # the 1x32 encoding produces) its largest magnitude code is 6 (4.0) or 7 (6.0): where the
    # independent draws left every code below 6, one element, chosen at random, keeps its sign
    # and takes magnitude 6 or 7.
    low = (codes & 7).max(axis=-1) < 6
    pick = rng.integers(0, 32, size=(N, K // 32))
    top = np.where(rng.random((N, K // 32)) < _TOP6[sidx], 6, 7).astype(np.uint8)
    r, c = np.nonzero(low)
    el = pick[r, c]
    codes[r, c, el] = (codes[r, c, el] & 8) | top[r, c]
    codes = codes.reshape(N, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.astype(np.uint8), _SCALE_BYTES[sidx]


def make_mxfp4(seed, tensor_id, E, N, K, experts=None):
    """Experts 0..E-1 (or the listed ones, in that order) of one MXFP4 weight tensor."""
    ids = list(range(E)) if experts is None else list(experts)
    packed = np.empty((len(ids), N, K // 2), dtype=np.uint8)
    scales = np.empty((len(ids), N, K // 32), dtype=np.uint8)

    def one(i):
        packed[i], scales[i] = make_mxfp4_expert(seed, tensor_id, ids[i], N, K)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(one, range(len(ids))))
    return packed, scales


def make_weights(seed, E, D, I, experts=None):
    """w1 [E, 2I, D/2] + [E, 2I, D/32] (gate rows 0..I-1, up rows I..2I-1) and
    w2 [E, D, I/2] + [E, D, I/32]; with `experts`, only those experts, in that order."""
    w1, w1s = make_mxfp4(seed, _W1, E, 2 * I, D, experts)
    w2, w2s = make_mxfp4(seed, _W2, E, D, I, experts)
    return w1, w1s, w2, w2s


def make_problem(wl, routing_seed=None, with_weights=True):
    """All host inputs of one workload as a dict of numpy arrays."""
    rs = wl.seed if routing_seed is None else routing_seed
    ids, w = make_routing(rs, wl.tokens, wl.router_experts, wl.topk, wl.zipf_s)
    prob = {"x": make_x(rs, wl.tokens, wl.model_dim), "topk_ids": ids, "topk_w": w}
    if with_weights:
        prob["w1"], prob["w1s"], prob["w2"], prob["w2s"] = make_weights(
            wl.seed, wl.experts, wl.model_dim, wl.inter_dim)
    return prob
