"""moe_fused_noalloc (the library's fixed per-device scratch as the workspace) against moe_fused
(a caller workspace) through the C ABI: the same kernels on the same inputs, so the outputs agree
bit for bit, on calls in a row of decreasing size (the scratch keeps the previous call's
contents), on the large-batch grouped path and the per-tile and decode paths; a batch whose
workspace exceeds the scratch is refused with MOE_ERR_WORKSPACE before any launch, and the
next call still works.  The no-alloc call itself allocates nothing through torch either."""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from quantized_moe_expert_sort_amd import inputs as gen

pytestmark = pytest.mark.gpu
BETA, LBETA = gen.BETA, gen.LINEAR_BETA


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


_W = {}


def weights(E, D, I):
    if (E, D, I) not in _W:
        _W[(E, D, I)] = qm.device_weights(*gen.make_weights(7, E, D, I))
    return _W[(E, D, I)]


def both(T, E, K, D, I, a_dtype, seed):
    """(noalloc output, moe_fused output) of one problem."""
    ids, w = gen.make_routing(seed, T, E, K, 0.7)
    ids_d, w_d = dev(ids), dev(w)
    x = dev(gen.make_x(seed, T, D))
    xa, xs = (x, None) if a_dtype == "bf16" else qm.moe_quant_act(x, a_dtype)
    wd = weights(E, D, I)
    lay = qm.moe_sort(ids_d, w_d, 0, E, qm.block_m(T))
    out_n = torch.full((T, D), 7.0, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    qm.moe_fused_noalloc(xa, xs, a_dtype, *wd, w_d, lay, E, "situv2", BETA, LBETA, out=out_n)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    out_r = qm.moe_fused(xa, xs, a_dtype, *wd, w_d, lay, E, "situv2", BETA, LBETA)
    torch.cuda.synchronize()
    return out_n, out_r


# calls in a row, each smaller than the one before: grouped path, per-tile path at full model
# width, decode (Stage2 + combine in one kernel)
SEQUENCE = [(2048, 16, 4, 512, 256, "fp4"), (64, 128, 16, 3584, 384, "fp8"), (4, 128, 16, 3584, 384, "bf16"),
            (1, 128, 16, 3584, 384, "fp8")]


def test_noalloc_matches_moe_fused_on_calls_in_a_row():
    for i, (T, E, K, D, I, a_dtype) in enumerate(SEQUENCE):
        print(f"noalloc call {i}: T={T} E={E} D={D} I={I} {a_dtype}", flush=True)
        got, want = both(T, E, K, D, I, a_dtype, seed=40 + i)
        assert torch.count_nonzero(want.view(torch.int16)) > 0
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {i}"


def test_noalloc_refuses_more_than_the_scratch_then_still_works():
    T, E, K, D, I = 1024, 128, 16, 3584, 384
    cap = qm.cap_tiles(T, K, E, qm.block_m(T))
    assert qm.fused_ws_bytes(T, D, I, cap, qm.block_m(T), qm.DT_FP8, qm.ACT_SITUV2) > qm.NOALLOC_SCRATCH_BYTES
    ids, w = gen.make_routing(3, T, E, K)
    x = dev(gen.make_x(3, T, D))
    xa, xs = qm.moe_quant_act(x, "fp8")
    lay = qm.moe_sort(dev(ids), dev(w), 0, E, qm.block_m(T))
    out = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_fused_noalloc(xa, xs, "fp8", *weights(E, D, I), dev(w), lay, E, "situv2", BETA, LBETA, out=out)
    assert ei.value.status == 5                       # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0   # nothing was launched
    got, want = both(16, E, K, D, I, "bf16", seed=5)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
