"""moe_pack_w1 and moe_pack_w2 on the GPU: the packed weight layouts are pure reorderings of the
bytes, checked byte for byte against the layout the ABI header states, written out with numpy."""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm

pytestmark = pytest.mark.gpu


def packed_reference(w1):
    # block (e, f, s): rows 16f..16f+15, bytes [64s, 64s+64) of each; byte 16*(16g + r) + b of
    # the block is byte 64s + 16g + b of row 16f + r
    E, R, H = w1.shape
    S = H * 2 // 128
    x = w1.reshape(E, R // 16, 16, S, 4, 16)               # e, f, r, s, g, b
    return np.ascontiguousarray(x.transpose(0, 1, 3, 4, 2, 5)).reshape(E, R, H)


@pytest.mark.parametrize("E,D,I", [(1, 128, 128), (3, 512, 256), (5, 1024, 384)])
def test_pack_w1_matches_stated_layout(E, D, I):
    rng = np.random.default_rng(E * 1000 + D + I)
    w1 = rng.integers(0, 256, size=(E, 2 * I, D // 2), dtype=np.uint8)
    got = qm.moe_pack_w1(torch.from_numpy(w1).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), packed_reference(w1))


@pytest.mark.parametrize("E,D,I", [(1, 128, 128), (3, 512, 256), (5, 384, 384), (2, 3584, 384)])
def test_pack_w2_matches_stated_layout(E, D, I):
    rng = np.random.default_rng(E * 7000 + D + I)
    w2 = rng.integers(0, 256, size=(E, D, I // 2), dtype=np.uint8)
    got = qm.moe_pack_w2(torch.from_numpy(w2).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), packed_reference(w2))


def test_pack_w2_into_the_bytes_right_after_it():
    # w2 holds E*D*I/2 bytes (half of w1's E*2I*D/2): a packed buffer that starts right after it
    # does not overlap and must be accepted
    E, D, I = 2, 256, 128
    rng = np.random.default_rng(5)
    w2 = rng.integers(0, 256, size=(E, D, I // 2), dtype=np.uint8)
    buf = torch.empty(2 * w2.size, dtype=torch.uint8, device="cuda")
    src, dst = buf[:w2.size], buf[w2.size:]
    src.copy_(torch.from_numpy(w2.reshape(-1)).cuda())
    qm.moe_pack_w2(src.view(E, D, I // 2), out=dst.view(E, D, I // 2))
    torch.cuda.synchronize()
    assert np.array_equal(dst.view(E, D, I // 2).cpu().numpy(), packed_reference(w2))
