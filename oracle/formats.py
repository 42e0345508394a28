"""Number formats of the MX layer, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats -- MXFP4 weights ("MxE2m1"), MXFP8 activations
with a per-token block-scale tensor, bf16 activations ("TokenSpeed SiTU",
"Supported contract" and the bundle list naming MxE4m3_MxE2m1MxE4m3 and
Bfloat16_MxE2m1MxE4m3) -- but never print their bit layouts.  Those come from
the OCP Microscaling Formats (MX) v1.0 specification, sections "Scale data
type" (E8M0) and "Element data types" (FP8 E4M3, FP4 E2M1), and from the
bfloat16 definition (the upper 16 bits of an IEEE binary32).

Every decode here is exact in float64.  Encoders return integer codes; their
rounding is round-to-nearest, ties-to-even, saturating, found by a nearest
search over the format's own value list, so a reader can check it without
knowing any bit trick.

Pins (tests/test_oracle_formats.py): exhaustive decode of every code against
an independent bit-field reading and, for E4M3/E8M0/bf16, against torch's
library dtypes; the encoders against brute-force nearest search over all
bf16 inputs; the block-scale rule against hand-built blocks at, just below
and just above powers of two.
"""

import numpy as np

# --------------------------------------------------------------------------
# E2M1 (FP4): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
# OCP MX v1.0, "Element data types": the eight magnitudes of FP4 E2M1.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E2M1_EMAX = 2  # exponent of the largest normal, 6 = 1.5 * 2**2

# E4M3 (FP8, the "FN" variant used by MX): bias 7, no infinities, the
# all-ones exponent+mantissa pattern (0x7F / 0xFF) is NaN.
E4M3_MAX = 448.0
E4M3_EMAX = 8  # 448 = 1.75 * 2**8

SCALE_BLOCK = 32  # one E8M0 scale per 32 consecutive elements along K


def decode_e2m1(codes):
    """Value of each 4-bit E2M1 code (0..15) as float64."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag)


def unpack_fp4(packed, n):
    """Split packed MXFP4 bytes into codes along the last axis.

    Two E2M1 codes per byte, the LOW nibble holding the even element.  The
    pages do not fix the nibble order; this is the layout of this library's
    weights, shared by the HIP path only through the documented format.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    assert packed.shape[-1] * 2 == n, (packed.shape, n)
    lo = packed & 0x0F
    hi = packed >> 4
    out = np.empty(packed.shape[:-1] + (n,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_fp4(codes):
    """Inverse of unpack_fp4: codes (..., n) -> bytes (..., n/2)."""
    codes = np.asarray(codes, dtype=np.uint8)
    assert codes.shape[-1] % 2 == 0
    return (codes[..., 0::2] & 0x0F) | ((codes[..., 1::2] & 0x0F) << 4)


def decode_e8m0(codes):
    """E8M0 scale: 2**(c - 127); the code 0xFF is NaN."""
    codes = np.asarray(codes).astype(np.int64)
    val = np.ldexp(1.0, codes - 127)
    return np.where(codes == 255, np.nan, val)


def decode_e4m3(codes):
    """Value of each 8-bit E4M3 code as float64.

    exponent field 0: subnormal, m * 2**-9 (m = 3-bit mantissa);
    otherwise (1 + m/8) * 2**(e - 7); 0x7F and 0xFF are NaN.
    """
    codes = np.asarray(codes).astype(np.int64)
    sign = np.where((codes & 0x80) != 0, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    val = sign * mag
    return np.where((codes & 0x7F) == 0x7F, np.nan, val)


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_to_f32(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x):
    """Round float32 values to the nearest bf16, ties to even mantissa.

    Written as the definition: among the two bf16 values that bracket x (x
    truncated to 16 bits, and that plus one bf16 ulp), take the nearer, and
    on an exact tie the one whose last mantissa bit is 0.  NaN stays NaN
    (quiet), infinities stay infinities.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.uint64)
    lower = bits & 0xFFFF0000            # truncation toward zero in magnitude
    rem = bits & 0x0000FFFF              # what truncation dropped
    half = 0x8000
    lsb = (lower >> 16) & 1
    round_up = (rem > half) | ((rem == half) & (lsb == 1))
    out = (lower + np.where(round_up, np.uint64(0x10000), np.uint64(0))) >> np.uint64(16)
    nan = np.isnan(x)
    out = np.where(nan, ((bits >> np.uint64(16)) | np.uint64(0x40)) & np.uint64(0xFFFF), out)
    return out.astype(np.uint16)


# --------------------------------------------------------------------------
# Encoders: nearest representable value, ties to the even code, saturating.

def _positive_grid(decode, codes):
    vals = decode(np.asarray(codes))
    order = np.argsort(vals, kind="stable")
    return vals[order], np.asarray(codes)[order]


_E4M3_POS_VALS, _E4M3_POS_CODES = _positive_grid(decode_e4m3, np.arange(0, 0x7F))
_E2M1_POS_VALS, _E2M1_POS_CODES = _positive_grid(decode_e2m1, np.arange(0, 8))


def _encode_nearest_even(v, grid_vals, grid_codes, sign_bit):
    """Encode float64 values by nearest search over a sorted magnitude grid.

    Magnitudes above the grid's maximum saturate to it.  On an exact tie
    between two neighbours the code with an even last bit wins.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), grid_vals[-1])
    hi = np.searchsorted(grid_vals, a, side="left")      # first grid >= a
    hi = np.clip(hi, 0, len(grid_vals) - 1)
    lo = np.clip(hi - 1, 0, len(grid_vals) - 1)
    d_lo = a - grid_vals[lo]
    d_hi = grid_vals[hi] - a
    c_lo = grid_codes[lo]
    c_hi = grid_codes[hi]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((c_hi & 1) == 0))
    code = np.where(pick_hi, c_hi, c_lo).astype(np.int64)
    neg = np.signbit(v) & (code != 0)
    return (code | np.where(neg, sign_bit, 0)).astype(np.uint8)


def encode_e4m3(v):
    """float64 -> E4M3 code, RNE, saturating to +-448.  -0 maps to +0."""
    return _encode_nearest_even(v, _E4M3_POS_VALS, _E4M3_POS_CODES, 0x80)


def encode_e2m1(v):
    """float64 -> E2M1 code, RNE, saturating to +-6.  -0 maps to +0."""
    return _encode_nearest_even(v, _E2M1_POS_VALS, _E2M1_POS_CODES, 0x8)


def floor_log2(a):
    """floor(log2(a)) for positive finite a, exactly, from frexp's exponent.

    frexp returns a = m * 2**ex with m in [0.5, 1), so floor(log2 a) = ex - 1.
    A floating log2 would round up just below powers of two.
    """
    _, ex = np.frexp(np.asarray(a, dtype=np.float64))
    return ex.astype(np.int64) - 1


def mx_block_scale_codes(v, emax_elem, block=SCALE_BLOCK):
    """E8M0 code of each block of `block` values along the last axis.

    OCP MX v1.0 conversion rule: shared exponent = floor(log2(amax)) - emax_elem,
    clamped to the E8M0 range [-127, 127]; the code is that exponent + 127.
    A block whose amax is 0 gets the smallest scale (code 0).
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    assert n % block == 0, (n, block)
    blocks = v.reshape(v.shape[:-1] + (n // block, block))
    amax = np.max(np.abs(blocks), axis=-1)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.where(amax > 0, floor_log2(safe) - emax_elem, -127)
    e = np.clip(e, -127, 127)
    return (e + 127).astype(np.uint8)


def mx_quantize(v, elem, block=SCALE_BLOCK):
    """Quantize along the last axis to MX: returns (element codes, scale codes).

    elem is "e4m3" (MXFP8) or "e2m1" (MXFP4; codes returned unpacked).
    Each element is v / 2**e rounded to the element format (RNE, saturating).
    Dividing by a power of two is exact in float64 for every value here.
    """
    v = np.asarray(v, dtype=np.float64)
    if elem == "e4m3":
        emax, enc = E4M3_EMAX, encode_e4m3
    elif elem == "e2m1":
        emax, enc = E2M1_EMAX, encode_e2m1
    else:
        raise ValueError(elem)
    sc = mx_block_scale_codes(v, emax, block)
    n = v.shape[-1]
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), block, axis=-1)
    codes = enc(v / scale)
    assert codes.shape[-1] == n
    return codes, sc


def mx_dequantize(codes, scale_codes, elem, block=SCALE_BLOCK):
    """Element codes (unpacked) and E8M0 codes -> float64 values."""
    dec = decode_e4m3 if elem == "e4m3" else decode_e2m1
    vals = dec(codes)
    return vals * np.repeat(decode_e8m0(scale_codes), block, axis=-1)


# The two E2M1 values of every byte value, [256, 2] (low nibble first), built
# from unpack_fp4 and decode_e2m1 above; decoding a packed matrix is then one
# table lookup per byte.
_FP4_BYTE_VALUES = decode_e2m1(unpack_fp4(np.arange(256, dtype=np.uint8)[:, None], 2))


def _dequant_fp4_blocks(packed, block_scales, block):
    """Packed E2M1 matrix (..., K/2 bytes) times one float64 scale per `block`
    consecutive elements along K (block_scales (..., K/block)) -> float64."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    n = packed.shape[-1] * 2
    vals = _FP4_BYTE_VALUES[packed].reshape(lead + (n // block, block))
    return (vals * np.asarray(block_scales, np.float64)[..., None]).reshape(lead + (n,))


def dequant_mxfp4(packed, scale_codes):
    """Packed MXFP4 matrix (..., K/2 bytes) + E8M0 scales (..., K/32) -> float64
    (the same values as mx_dequantize of the unpacked codes)."""
    return _dequant_fp4_blocks(packed, decode_e8m0(scale_codes), SCALE_BLOCK)


# NVFP4: E2M1 elements with one E4M3 scale per 16 consecutive elements along
# K (NVIDIA's NVFP4 layout; the pages name the format -- the Kimi-K3 NVFP4
# checkpoint, the NVFP4 MoE-LoRA op -- without printing it).  A per-tensor
# fp32 scale completes the format; in this layer it is the per-expert alpha
# of each GEMM, applied outside the weight decode.
NVFP4_BLOCK = 16


def dequant_nvfp4(packed, scale_codes):
    """Packed NVFP4 matrix (..., K/2 bytes) + E4M3 scales (..., K/16) -> float64."""
    return _dequant_fp4_blocks(packed, decode_e4m3(scale_codes), NVFP4_BLOCK)
