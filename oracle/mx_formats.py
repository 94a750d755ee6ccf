"""MX block formats, written from their definitions (test infrastructure only).

The pages use three element/scale encodings without defining them:
* MXFP4 weights and fp4x2 activations: e2m1 codes, two per byte
  (github ROCm/aiter PR 4463, "Three tuner defects", item 2: a low-nibble difference moves
  the byte by 1 and a high-nibble one by 16);
* fp8 activations with per-1x32 scales, "fp8_blockwise_1x32"
  (github ROCm/aiter PR 6259, "Test Result");
* e8m0 shared scales, one per 32 elements along K (the "1x32" of both pages).

Readings taken where the pages are silent (each listed in the design notes):
* e2m1 = sign, 2 exponent bits (bias 1), 1 mantissa bit; values 0, .5, 1, 1.5, 2, 3, 4, 6.
* fp8 = OCP E4M3FN: bias 7, max 448, only S.1111.111 is NaN, no infinities.
* e8m0 = 2^(code - 127); code 255 is NaN.
* fp4x2 packing: the element with the even index sits in the low nibble.
* Block quantization (rule Q), the OCP MX shared-scale rule: for a block of 32 values,
  amax = max|v|; if amax == 0 the scale code is 0 and all elements encode +-0; otherwise
  E = floor(log2(amax)) read exactly from the binary exponent, sexp = clamp(E - emax, -127,
  127) with emax = 2 (e2m1) or 8 (e4m3), the scale code is sexp + 127, and every element is
  rounded to nearest, ties to the even code, saturating at +-6 (e2m1) or +-448 (e4m3), on
  v / 2^sexp.  The sign bit of v is kept, so a negative value that rounds to zero gives -0.

Parity pins (tests that fix these functions to something other than themselves):
  decoders   exhaustive closed-form tables, torch's float8_e4m3fn / float8_e8m0fnu decoders;
  encoders   brute-force nearest-value search over every code, torch's float8_e4m3fn RNE
             cast for non-saturating values, hand-worked ties and saturation cases.
"""
import numpy as np

E2M1_EMAX = 2       # 6 = 1.5 * 2^2
E4M3_EMAX = 8       # 448 = 1.75 * 2^8
E2M1_SIGN = 0x8
E4M3_SIGN = 0x80
BLOCK = 32


def e2m1_value(code):
    """Decode e2m1 codes (ints 0..15) to float64: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent field 0 is subnormal (0 or 0.5)."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & E2M1_SIGN, -1.0, 1.0)
    e = (code >> 1) & 3
    m = (code & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def e4m3_value(code):
    """Decode OCP E4M3FN codes (ints 0..255) to float64: sign bit 7, exponent bits 6..3
    (bias 7), mantissa bits 2..0; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & E4M3_SIGN, -1.0, 1.0)
    e = (code >> 3) & 15
    m = (code & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((code & 7) == 7), np.nan, mag)
    return sign * mag


def e8m0_value(code):
    """Decode e8m0 scale codes: 2^(code - 127); 255 is NaN."""
    code = np.asarray(code, dtype=np.int64)
    return np.where(code == 255, np.nan, np.ldexp(1.0, code - 127))


def _grid(fmt):
    """Non-negative finite values of a format in code order (code i has value grid[i])."""
    if fmt == "e2m1":
        return e2m1_value(np.arange(8)), E2M1_EMAX, E2M1_SIGN
    if fmt == "e4m3":
        return e4m3_value(np.arange(127)), E4M3_EMAX, E4M3_SIGN
    raise ValueError(f"unknown element format {fmt!r}")


def encode_rne_sat(v, fmt):
    """Round each float64 in v to the nearest value of fmt (ties to the even code) with
    saturation at the largest finite value; the sign bit of v is kept.  Returns int codes."""
    grid, _, signbit = _grid(fmt)
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)       # saturate
    return idx.astype(np.int64) | np.where(np.signbit(v), signbit, 0)


def block_scale_exponent(amax, fmt):
    """Shared exponent of rule Q for block maxima amax (float64, finite, >= 0)."""
    _, emax, _ = _grid(fmt)
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)              # amax = m * 2^e with m in [0.5, 1): floor(log2) = e - 1
    sexp = np.clip((e - 1) - emax, -127, 127)
    return np.where(amax == 0, -127, sexp).astype(np.int64)


def quantize_1x32(v, fmt):
    """Rule Q along the last axis (length a multiple of 32).

    Returns (codes, scale_codes): codes is an int array shaped like v holding one element code
    each (not packed), scale_codes is uint8 [..., n/32]."""
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    if not np.all(np.isfinite(v)):
        raise ValueError("rule Q is defined here for finite inputs only")
    blocks = v.reshape(*v.shape[:-1], v.shape[-1] // BLOCK, BLOCK)
    sexp = block_scale_exponent(np.max(np.abs(blocks), axis=-1), fmt)
    scaled = blocks / np.ldexp(1.0, sexp)[..., None]
    codes = encode_rne_sat(scaled, fmt).reshape(v.shape)
    return codes, (sexp + 127).astype(np.uint8)


_E2M1_TABLE = None
_E4M3_TABLE = None


def _value_table(fmt):
    """Decoded value of every code (the closed forms above, evaluated once per code)."""
    global _E2M1_TABLE, _E4M3_TABLE
    if fmt == "e2m1":
        if _E2M1_TABLE is None:
            _E2M1_TABLE = e2m1_value(np.arange(16))
        return _E2M1_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = e4m3_value(np.arange(256))
    return _E4M3_TABLE


def dequantize_1x32(codes, scale_codes, fmt):
    """Inverse of quantize_1x32: element value times 2^(scale - 127), per 32-element block."""
    codes = np.asarray(codes)
    vals = _value_table(fmt)[codes]
    s = e8m0_value(scale_codes)
    blocks = vals.reshape(*vals.shape[:-1], vals.shape[-1] // BLOCK, BLOCK)
    return (blocks * s[..., None]).reshape(vals.shape)


def pack_fp4(codes):
    """Pack e2m1 codes pairwise along the last axis: element 2i -> low nibble of byte i."""
    codes = np.asarray(codes, dtype=np.int64)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed):
    """Split fp4x2 bytes into e2m1 codes: byte i -> elements 2i (low) and 2i + 1 (high)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequant_mxfp4(packed, scale_codes):
    """MXFP4 tensor [..., N, K/2] bytes + [..., N, K/32] e8m0 -> float64 [..., N, K]."""
    return dequantize_1x32(unpack_fp4(packed), scale_codes, "e2m1")


def dequant_fp8_1x32(codes, scale_codes):
    """fp8 e4m3 bytes [..., K] + [..., K/32] e8m0 -> float64 [..., K]."""
    return dequantize_1x32(np.asarray(codes, dtype=np.int64), scale_codes, "e4m3")
