"""moe_quant_act on the GPU vs the oracle's 1x32 rule: bit-exact codes and scales (fp4 codes
compared nibble by nibble), on random rows and on the rule's edge cases."""
import numpy as np
import pytest
import torch

import quantized_moe_expert_sort_amd as qm
from oracle import mx_formats as mx
from oracle import moe as om
from quantized_moe_expert_sort_amd import inputs as gen

pytestmark = pytest.mark.gpu


def f32_to_bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gpu_quant(xbits, dt):
    x = torch.from_numpy(xbits.view(np.int16)).cuda()
    q, s = qm.moe_quant_act(x, dt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check_quant(xbits, dt):
    fmt = {"fp8": "e4m3", "fp4": "e2m1"}[dt]
    codes, scales = mx.quantize_1x32(om.bf16_bits_to_f64(xbits), fmt)
    q, s = gpu_quant(xbits, dt)
    assert np.array_equal(s, scales)
    got = q.astype(np.int64) if dt == "fp8" else mx.unpack_fp4(q).astype(np.int64)
    assert np.array_equal(got, codes)


@pytest.mark.parametrize("dt", ["fp8", "fp4"])
@pytest.mark.parametrize("rows,cols,mag", [(1, 32, 1.0), (7, 3584, 1.0), (129, 256, 1e-30),
                                           (33, 512, 1e30), (1024, 3584, 1.0)])
def test_quant_random(dt, rows, cols, mag):
    rng = np.random.default_rng(rows + cols)
    v = rng.standard_normal((rows, cols)) * mag * np.exp(rng.uniform(-3, 3, (rows, 1)))
    check_quant(f32_to_bf16_bits(v), dt)


@pytest.mark.parametrize("dt", ["fp8", "fp4"])
def test_quant_edge_cases(dt):
    emax = 8 if dt == "fp8" else 2
    top = 448.0 if dt == "fp8" else 6.0
    grid = np.abs(mx.e4m3_value(np.arange(127)) if dt == "fp8" else mx.e2m1_value(np.arange(8)))
    mids = (grid[1:] + grid[:-1]) / 2
    blocks = []
    blocks.append(np.zeros(32))                                          # zero block
    blocks.append(-np.zeros(32))                                         # negative zeros
    b = np.zeros(32); b[0] = 2.0 ** emax * 1.0; b[1:1 + len(mids[:31])] = mids[:31]
    blocks.append(b)                                                     # exact ties, scale 2^0
    b = np.full(32, 2.0 ** (emax + 1) - 2.0 ** (emax - 7)); b[1::2] *= -1  # saturation at +-top
    blocks.append(b)
    b = np.zeros(32); b[0] = top; b[1:] = np.linspace(-top, top, 31)
    blocks.append(b)
    b = np.ones(32) * 2.0 ** -130; b[3] = -2.0 ** -133                   # bf16 subnormals
    blocks.append(b)
    b = np.zeros(32); b[5] = 3.3e38; b[6] = -1.0                          # near the bf16 maximum
    blocks.append(b)
    b = np.zeros(32); b[7] = 1e-3                                        # lone small value
    blocks.append(b)
    v = np.stack(blocks).reshape(1, -1)
    check_quant(f32_to_bf16_bits(v), dt)
    # every bf16 bit pattern that is finite, in blocks of 32
    allbits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = (allbits & 0x7F80) != 0x7F80
    pats = allbits[finite][: (int(finite.sum()) // 32) * 32].reshape(-1, 32)
    check_quant(pats, dt)


@pytest.mark.parametrize("dt", ["fp8", "fp4"])
def test_quant_nonfinite_block_gets_nan_scale(dt):
    v = np.ones((2, 64), np.float32)
    v[0, 40] = np.inf
    x = f32_to_bf16_bits(v)
    q, s = gpu_quant(x, dt)
    assert s[0, 1] == 255 and np.all(s[[0, 1, 1], [0, 0, 1]] != 255)
    codes = q if dt == "fp8" else mx.unpack_fp4(q)
    assert np.all(codes[0, 32:64] == 0)


def test_quant_workload_activations():
    wl = gen.WORKLOADS["mid-1024"]
    x = gen.make_x(wl.seed, wl.tokens, wl.model_dim)
    check_quant(x, "fp8")
    check_quant(x, "fp4")
