"""Pins of the oracle's MX format codecs and block quantization rule against references that
are not the oracle: closed-form tables, torch's own float8 decoders and casts, brute-force
nearest-value search, and hand-worked rounding cases."""
import math

import numpy as np
import pytest
import torch

from oracle import mx_formats as mx

# e2m1 values by code, from the OCP Microscaling v1.0 element table (sign in bit 3)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_exhaustive_table():
    got = mx.e2m1_value(np.arange(16))
    want = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    assert np.array_equal(got, want)
    assert np.signbit(got[8])            # code 8 is -0


def test_e4m3_matches_torch_decoder():
    codes = np.arange(256)
    got = mx.e4m3_value(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.sum(np.isnan(got)) == 2


def test_e8m0_matches_torch_decoder():
    got = mx.e8m0_value(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0


def _brute_encode(v, fmt):
    """Nearest code by exhaustive search over all finite codes; ties -> even code;
    beyond the largest finite value -> the largest; sign bit copied."""
    if fmt == "e2m1":
        vals = [abs(x) for x in mx.e2m1_value(np.arange(8))]
        sign = 8
    else:
        vals = [abs(x) for x in mx.e4m3_value(np.arange(127))]
        sign = 0x80
    out = []
    for x in np.asarray(v, dtype=np.float64).ravel():
        a = abs(x)
        best, bestd = None, None
        for c, val in enumerate(vals):
            d = abs(a - val)
            if best is None or d < bestd or (d == bestd and c % 2 == 0):
                best, bestd = c, d
        if a >= vals[-1]:
            best = len(vals) - 1
        out.append(best | (sign if math.copysign(1.0, x) < 0 else 0))
    return np.array(out)


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_encode_matches_brute_force(fmt):
    rng = np.random.default_rng(1)
    top = 6.0 if fmt == "e2m1" else 448.0
    grid = np.abs(mx.e2m1_value(np.arange(8)) if fmt == "e2m1" else mx.e4m3_value(np.arange(127)))
    mids = (grid[1:] + grid[:-1]) / 2                      # every exact tie
    v = np.concatenate([rng.uniform(-top * 1.2, top * 1.2, 3000),
                        rng.standard_normal(2000) * (1 if fmt == "e2m1" else 16),
                        mids, -mids, grid, -grid, [0.0, -0.0, top * 3, -top * 3]])
    assert np.array_equal(mx.encode_rne_sat(v, fmt), _brute_encode(v, fmt))


def test_e4m3_encoder_matches_torch_cast_below_saturation():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-463.9, 463.9, 20000), rng.standard_normal(20000) * 2.0 ** -6,
                        (mx.e4m3_value(np.arange(126))[1:] + mx.e4m3_value(np.arange(126))[:-1]) / 2])
    v = v.astype(np.float32)                        # torch casts from float32 values
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    assert np.array_equal(mx.encode_rne_sat(v.astype(np.float64), "e4m3"), ref)


def test_e2m1_hand_worked_ties_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.01, 7.0, 100.0, -0.1, -2.9, 0.26])
    want_vals = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 6.0, -0.0, -3.0, 0.5]
    codes = mx.encode_rne_sat(v, "e2m1")
    assert np.array_equal(mx.e2m1_value(codes), np.array(want_vals))
    assert codes[10] == 8                          # -0.1 keeps its sign: -0


def test_rule_q_scale_exponent():
    # zero block: scale code 0 (2^-127), elements +-0
    c, s = mx.quantize_1x32(np.zeros(32), "e2m1")
    assert s[0] == 0 and np.all(c == 0)
    # amax = 1.0: floor(log2) = 0, e2m1 emax 2 -> 2^-2 -> code 125; e4m3 emax 8 -> code 119
    blk = np.zeros(32); blk[3] = 1.0
    assert mx.quantize_1x32(blk, "e2m1")[1][0] == 125
    assert mx.quantize_1x32(blk, "e4m3")[1][0] == 119
    # just below a power of two stays in the lower binade
    blk[3] = np.nextafter(1.0, 0)
    assert mx.quantize_1x32(blk, "e2m1")[1][0] == 124
    # floor(log2) from the binary exponent agrees with math.log2 away from powers of two
    rng = np.random.default_rng(3)
    a = np.exp(rng.uniform(-60, 60, 5000))
    ref = np.array([math.floor(math.log2(x)) for x in a]) - 2
    assert np.array_equal(mx.block_scale_exponent(a, "e2m1"), np.clip(ref, -127, 127))
    # clamping at both ends
    assert mx.block_scale_exponent(np.array([2.0 ** -140]), "e4m3")[0] == -127
    assert mx.block_scale_exponent(np.array([2.0 ** 200]), "e2m1")[0] == 127


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_rule_q_roundtrip_of_representable_blocks(fmt):
    rng = np.random.default_rng(4)
    n_codes = 8 if fmt == "e2m1" else 127
    dec = mx.e2m1_value if fmt == "e2m1" else mx.e4m3_value
    top = n_codes - 1
    for sexp in (-20, -7, 0, 5):
        codes = rng.integers(0, n_codes, size=(50, 32))
        codes[:, 0] = top                           # the block maximum fixes the scale
        v = dec(codes) * (2.0 ** sexp) * rng.choice([-1.0, 1.0], size=codes.shape)
        c, s = mx.quantize_1x32(v, fmt)
        assert np.all(s == sexp + 127)
        assert np.array_equal(mx.dequantize_1x32(c, s, fmt), v)


def test_rule_q_error_bound_e4m3():
    # unsaturated e4m3 normals: relative error at most 2^-4 (3 mantissa bits, round to nearest)
    rng = np.random.default_rng(5)
    v = rng.standard_normal((400, 64))
    c, s = mx.quantize_1x32(v, "e4m3")
    r = mx.dequantize_1x32(c, s, "e4m3")
    scale = np.repeat(mx.e8m0_value(s), 32, axis=-1)
    scaled = np.abs(v) / scale
    # the shared exponent maps the block maximum into [256, 512): above the largest finite
    # value's rounding boundary (464) elements saturate to +-448
    sat = scaled >= 464.0
    assert np.all(np.abs(r[sat]) == 448.0 * scale[sat])
    normal = (scaled >= 2.0 ** -6) & ~sat
    assert np.all(np.abs(r - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    sub = scaled < 2.0 ** -6
    assert np.all(np.abs(r - v)[sub] <= 2.0 ** -10 * scale[sub])


def test_fp4x2_nibble_order():
    # github ROCm/aiter PR 4463, "Three tuner defects" item 2: fp4x2 packs two e2m1 codes per
    # byte; a low-nibble difference moves the byte by 1, a high-nibble one by 16.
    assert mx.pack_fp4(np.array([1, 0]))[0] == 1
    assert mx.pack_fp4(np.array([0, 1]))[0] == 16
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 16, size=(7, 64))
    assert np.array_equal(mx.unpack_fp4(mx.pack_fp4(codes)), codes)
