"""Pins of the oracle's number formats against things other than itself.

Each test checks an oracle function against an independent source: the OCP
MX v1.0 value table (tests/golden), a bit-field reading of the format, a
library dtype (torch's float8_e4m3fn / float8_e8m0fnu / bfloat16), or a
brute-force nearest search.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F


def _read_table(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e2m1_decode_matches_ocp_table(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "e2m1_values.txt"))
    assert len(rows) == 16
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    got = F.decode_e2m1(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_e2m1_decode_matches_bitfields():
    # value = (-1)^s * 2^(e-1) * (1 + m/2) for e > 0, (-1)^s * m/2 for e = 0
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1 + m / 2)
        v = -v if s else v
        assert F.decode_e2m1(np.array([c]))[0] == v, c


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.decode_e4m3(codes)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], lib[~nan])
    assert np.nanmax(got) == 448.0 and F.E4M3_MAX == 448.0
    assert got[1] == 2.0 ** -9  # smallest subnormal


def test_e8m0_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(lib[255])
    assert np.array_equal(got[:255], lib[:255])
    assert got[127] == 1.0


def test_fp4_nibble_order_roundtrip():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    packed = F.pack_fp4(codes)
    assert np.array_equal(packed[:, 0] & 0xF, codes[:, 0])   # low nibble = element 0
    assert np.array_equal(packed[:, 0] >> 4, codes[:, 1])
    assert np.array_equal(F.unpack_fp4(packed, 64), codes)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10.0),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-39),   # subnormals
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38, 1e-45], dtype=np.float32),
    ])
    # exact ties: bf16 value + half a bf16 ulp, both parities of the kept lsb
    base = rng.integers(0x3000, 0x5000, size=2000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.f32_to_bf16_rne(x)
    assert np.array_equal(got, want)


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)].astype(np.float64)


def _brute_nearest_even(v, magnitudes, codes, sign_bit, vmax):
    """Nearest magnitude by exhaustive distance table; ties to the even code."""
    a = np.minimum(np.abs(v), vmax)
    d = np.abs(a[:, None] - magnitudes[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates take the even code (there are at most two)
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    code = codes[pick]
    neg = (v < 0) & (code != 0)
    return (code | np.where(neg, sign_bit, 0)).astype(np.uint8)


def test_e4m3_encode_bruteforce_all_bf16():
    v = _all_bf16_values()
    codes = np.arange(0x7F)
    mags = np.array([(1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15) - 7) if (c >> 3) & 15
                     else (c & 7) * 2.0 ** -9 for c in codes])
    want = _brute_nearest_even(v, mags, codes, 0x80, 448.0)
    got = F.encode_e4m3(v)
    assert np.array_equal(got, want)


def test_e4m3_encode_matches_torch_in_range():
    v = _all_bf16_values()
    v = v[np.abs(v) <= 448.0]
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.encode_e4m3(v)
    # torch keeps the sign of a value that rounds to zero; the oracle maps it to +0
    lib = np.where((lib & 0x7F) == 0, 0, lib)
    assert np.array_equal(got, lib)


def test_e4m3_encode_saturates():
    v = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e6, -1e30])
    assert F.encode_e4m3(v).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e2m1_encode_bruteforce():
    v = _all_bf16_values()
    v = v[np.abs(v) < 64]
    codes = np.arange(8)
    mags = F.decode_e2m1(codes)
    want = _brute_nearest_even(v, mags, codes, 0x8, 6.0)
    assert np.array_equal(F.encode_e2m1(v), want)
    # ties: 0.25 -> 0 (even), 0.75 -> 1.0 (code 2), 2.5 -> 2.0 (code 4), 5 -> 4 (code 6)
    assert F.encode_e2m1(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])).tolist() == [0, 2, 2, 4, 4, 6, 6]


def test_floor_log2_exact_near_powers_of_two():
    for p in range(-140, 130):
        x = math.ldexp(1.0, p)
        assert F.floor_log2(x) == p
        assert F.floor_log2(np.nextafter(x, 0.0)) == p - 1
        assert F.floor_log2(np.nextafter(x, np.inf)) == p


def test_mx_scale_rule_at_powers_of_two():
    for emax, elem in ((8, "e4m3"), (2, "e2m1")):
        for p in (-20, -7, -1, 0, 3, 10):
            for amax, fl in ((math.ldexp(1.0, p), p),
                             (np.nextafter(math.ldexp(1.0, p), 0.0), p - 1),
                             (np.nextafter(math.ldexp(1.0, p), np.inf), p)):
                blk = np.zeros(32)
                blk[5] = -amax
                blk[9] = amax / 3
                _, sc = F.mx_quantize(blk, elem)
                assert int(sc[0]) == fl - emax + 127, (elem, p, amax)
    # all-zero block -> code 0; clamp at both ends of the E8M0 range
    assert F.mx_block_scale_codes(np.zeros(32), 8)[0] == 0
    assert F.mx_block_scale_codes(np.full(32, 2.0 ** -140), 8)[0] == 0
    assert F.mx_block_scale_codes(np.full(32, 2.0 ** 200), 8)[0] == 254


def test_mxfp8_hand_worked_block(golden_dir):
    rows = _read_table(os.path.join(golden_dir, "mxfp8_block_example.txt"))
    assert rows[0][0] == "scale"
    scale = int(rows[0][1])
    vals = [float(r[0]) for r in rows[1:]]
    codes = [int(r[1], 16) for r in rows[1:]]
    blk = np.zeros(32)
    blk[:len(vals)] = vals
    c, s = F.mx_quantize(blk, "e4m3")
    assert int(s[0]) == scale
    assert c[:len(vals)].tolist() == codes
    assert np.all(c[len(vals):] == 0)


def test_mx_quantize_error_bound_and_top_binade():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((400, 64)) * np.exp(rng.uniform(-10, 10, size=(400, 1)))
    for elem, mbits, emax in (("e4m3", 3, 8), ("e2m1", 1, 2)):
        c, s = F.mx_quantize(v, elem)
        d = F.mx_dequantize(c, s, elem)
        scale = np.repeat(F.decode_e8m0(s), 32, axis=-1)
        blocks = np.abs(v).reshape(400, 2, 32).max(-1)
        ratio = blocks / F.decode_e8m0(s)
        assert np.all((ratio >= 2.0 ** emax) & (ratio < 2.0 ** (emax + 1)))
        # saturation only affects the top of the binade: |err| <= max(half ulp, clip)
        vmax = 448.0 if elem == "e4m3" else 6.0
        err = np.abs(d - v)
        clip = np.maximum(np.abs(v) - vmax * scale, 0)
        min_normal = 2.0 ** -6 if elem == "e4m3" else 1.0
        ulp_half = np.maximum(np.abs(v), scale * min_normal) * 2.0 ** (-mbits - 1)
        assert np.all(err <= np.maximum(ulp_half * (1 + 1e-12), clip + 1e-300))
