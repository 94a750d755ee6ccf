"""The debug build of the library (libmoe_mi355x_debug.so, compiled with MOE_DEBUG_CHECKS).

* Valid inputs: every call returns MOE_OK and the sorted layout and the output are
  bit-identical to the normal library's (the checks only read), on the decode kernel, the
  per-tile stages at block_m 16 and 32, an expert-parallel shard, the large-batch grouped stages
  (with a few hot experts, and with every expert hot: the token-major Stage2), and the
  single-launch path.
* Corrupted layouts, each chosen so that the corrupted access stays inside allocated memory even
  if its check were missing: a row_of entry one row past the layout (the combine's read of that
  row would land in the workspace part after the per-row outputs), a sorted row id past
  T*topk (every stage reads it as padding) and a tile's expert id equal to num_local_experts
  (the per-tile stages skip such a tile).  The debug build must answer MOE_ERR_DEBUG_CHECK, and
  the next valid call MOE_OK again (the violation words are cleared when read).
"""
import os

import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from quantized_moe_expert_sort_amd import inputs as gen

pytestmark = pytest.mark.gpu
BETA, LBETA = gen.BETA, gen.LINEAR_BETA
DEBUG_CHECK = 6


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def problem(T, Er, K, D, I, eb, E, zipf):
    seed = 7 * T + D + I + eb
    ids, w = gen.make_routing(seed, T, Er, K, zipf)
    x = gen.make_x(seed, T, D)
    host_w = gen.make_weights(seed, E, D, I, experts=range(eb, eb + E))
    return ids, w, x, host_w


def run(lib_path, ids, w, x, wd, eb, E, bm, a_dtype, single=False, corrupt=None):
    prev = qm.select_library(lib_path)
    try:
        ids_d, w_d, x_d = dev(ids), dev(w), dev(x)
        lay = qm.moe_sort(ids_d, w_d, eb, E, bm, single_launch=single)
        if corrupt is not None:
            torch.cuda.synchronize()
            corrupt(lay)
            torch.cuda.synchronize()
        xa, xs = (x_d, None) if a_dtype == "bf16" else qm.moe_quant_act(x_d, a_dtype)
        out = qm.moe_fused(xa, xs, a_dtype, *wd, w_d, lay, E, "situv2", BETA, LBETA)
        torch.cuda.synchronize()
        return out, lay
    finally:
        qm.select_library(prev)


@pytest.fixture(scope="module")
def debug_lib():
    if not os.path.exists(qm.DEBUG_LIB_PATH):
        pytest.fail(f"{qm.DEBUG_LIB_PATH} is not built; run: python -m quantized_moe_expert_sort_amd.build")
    return qm.DEBUG_LIB_PATH


VALID = [  # (T, E_router, K, D, I, eb, E_local, bm, a_dtype, zipf, single_launch)
    (4, 8, 2, 256, 128, 0, 8, 16, "bf16", 0.0, False),          # decode Stage2 + combine kernel
    (37, 16, 4, 512, 256, 0, 16, 16, "fp8", 0.0, False),        # per-tile stages, block_m 16
    (100, 24, 6, 384, 384, 0, 24, 32, "fp4", 1.1, False),       # per-tile stages, block_m 32
    (50, 32, 4, 256, 256, 8, 8, 16, "bf16", 0.0, False),        # expert-parallel shard
    (4096, 512, 8, 512, 256, 0, 512, 32, "fp8", 0.7, False),    # grouped stages, hot experts
    (2048, 16, 4, 512, 256, 0, 16, 32, "bf16", 1.1, False),     # grouped bf16 Stage1
    (6, 32, 8, 256, 128, 0, 32, 16, "fp8", 0.0, True),          # single-launch path
    (2048, 24, 16, 512, 256, 0, 24, 32, "fp4", 0.3, False),     # token-major Stage2 of hot experts
]


@pytest.mark.parametrize("T,Er,K,D,I,eb,E,bm,a_dtype,zipf,single", VALID)
def test_debug_build_matches_normal_build(debug_lib, T, Er, K, D, I, eb, E, bm, a_dtype, zipf, single):
    ids, w, x, host_w = problem(T, Er, K, D, I, eb, E, zipf)
    wd = qm.device_weights(*host_w)
    print(f"debug build T={T} E={E} D={D} I={I} bm={bm} {a_dtype} single={single}", flush=True)
    ref, ref_lay = run(qm.LIB_PATH, ids, w, x, wd, eb, E, bm, a_dtype, single)
    got, lay = run(debug_lib, ids, w, x, wd, eb, E, bm, a_dtype, single)
    for name in ("sorted_token_ids", "expert_ids", "num_tiles", "row_of"):
        assert torch.equal(getattr(lay, name), getattr(ref_lay, name)), name
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def _row_past_layout(lay):
    r = lay.row_of
    i = int(torch.nonzero(r >= 0)[0, 0])
    r[i] = lay.cap * lay.block_m


def _row_id_past_tokens(T, K):
    def f(lay):
        lay.sorted_token_ids[0] = T * K + 5
    return f


def _expert_past_local(E):
    def f(lay):
        lay.expert_ids[0] = E
    return f


@pytest.mark.parametrize("what", ["row_of", "row_id", "expert"])
def test_debug_build_reports_corrupted_layouts(debug_lib, what):
    T, Er, K, D, I, eb, E, bm, a_dtype = 37, 16, 4, 512, 256, 0, 16, 16, "fp8"
    ids, w, x, host_w = problem(T, Er, K, D, I, eb, E, 0.0)
    wd = qm.device_weights(*host_w)
    corrupt = {"row_of": _row_past_layout, "row_id": _row_id_past_tokens(T, K), "expert": _expert_past_local(E)}[what]
    print(f"debug build: corrupted {what}", flush=True)
    with pytest.raises(qm.MoeError) as exc:
        run(debug_lib, ids, w, x, wd, eb, E, bm, a_dtype, corrupt=corrupt)
    assert exc.value.status == DEBUG_CHECK
    # the violation words were cleared: the same problem uncorrupted passes
    run(debug_lib, ids, w, x, wd, eb, E, bm, a_dtype)
