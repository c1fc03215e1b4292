"""Pins for the oracle's E4M3 / UE8M0 / bf16 codecs (CPU only).

The E4M3 element format is named in "Unified FP8: Beyond Mixed Precision...",
section "FP8 Format"; the OCP E4M3FN variant (bias 7, max 448, NaN = S.1111.111,
no infinities) with round-to-nearest-even and saturation is the reading taken.
Nothing here re-types the oracle's bit manipulation: the checks are the closed
form of the format, brute-force nearest-value search, hand-derived spot values
(tests/golden) and torch's independent float8 casts.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_spot_values.txt")


def closed_form_e4m3(code: int) -> float:
    """Value of an OCP E4M3FN code from the format's field definitions."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_decode_table_all_256_codes():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        ref = closed_form_e4m3(c)
        if math.isnan(ref):
            assert math.isnan(dec[c]), c
        else:
            assert dec[c] == ref, (c, dec[c], ref)
    assert int(np.isnan(dec).sum()) == 2 and np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert int((dec == 0).sum()) == 2
    fin = dec[~np.isnan(dec)]
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert dec[0x38] == 1.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    assert dec[0x7E] == 448.0
    assert math.copysign(1.0, dec[0x80]) == -1.0


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(t) & np.isnan(dec)
    assert np.array_equal(t[~both_nan], dec[~both_nan])
    assert np.array_equal(np.isnan(t), np.isnan(dec))


def test_encode_round_trip_all_finite_codes():
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = [c for c in range(256) if not math.isnan(dec[c])]
    enc = oracle.e4m3_encode(dec[finite].astype(np.float32))
    assert list(enc) == finite


def _positive_grid():
    dec = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # codes 0x00..0x7E ascending
    return dec


def test_encode_midpoints_tie_to_even_and_neighbours():
    grid = _positive_grid()
    for c in range(0x7E):
        lo, hi = grid[c], grid[c + 1]
        mid = np.float32((lo + hi) / 2.0)
        assert float(mid) == (lo + hi) / 2.0          # every midpoint is exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, (c, mid)
        assert oracle.e4m3_encode(-mid) == (even | 0x80)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert oracle.e4m3_encode(below) == c
        assert oracle.e4m3_encode(above) == c + 1


def test_encode_saturation_and_specials():
    vals = np.array([448.0, 448.5, 463.99997, 464.0, 480.0, 1e6, 3.4e38, np.inf], np.float32)
    assert all(oracle.e4m3_encode(vals) == 0x7E)
    assert all(oracle.e4m3_encode(-vals) == 0xFE)
    assert oracle.e4m3_encode(np.float32(np.nan)) & 0x7F == 0x7F
    assert oracle.e4m3_encode(np.float32(0.0)) == 0x00
    assert oracle.e4m3_encode(np.float32(-0.0)) == 0x80
    # fp32 subnormals are far below the smallest E4M3 subnormal
    assert oracle.e4m3_encode(np.float32(1e-40)) == 0x00
    assert oracle.e4m3_encode(np.float32(-1e-40)) == 0x80


def test_encode_golden_spot_values():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            val, code = line.split()[:2]
            v = float.fromhex(val) if "0x" in val and "p" in val else float(val)
            rows.append((np.float32(v), int(code, 16)))
    assert len(rows) >= 15
    for v, code in rows:
        assert oracle.e4m3_encode(v) == code, (v, hex(code))


def _nearest_even_bruteforce(v: float, grid: np.ndarray) -> int:
    """Code of the E4M3 value nearest to |v| (ties to even code), saturating."""
    a = abs(v)
    if a >= 448.0:
        c = 0x7E
    else:
        d = np.abs(grid - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_encode_bruteforce_random():
    rng = np.random.default_rng(1234)
    grid = _positive_grid()
    # log-uniform magnitudes over the whole E4M3 range and beyond, random signs
    mags = np.exp2(rng.uniform(-14, 10, size=4000)).astype(np.float32)
    vals = mags * rng.choice([-1, 1], size=mags.size).astype(np.float32)
    enc = oracle.e4m3_encode(vals)
    for v, c in zip(vals, enc):
        assert c == _nearest_even_bruteforce(float(v), grid), (v, c)


def test_encode_matches_torch_cast_after_clamp():
    # torch's float8_e4m3fn cast is round-to-nearest-even but returns NaN above
    # 464, so values are clamped to +-448 first.
    rng = np.random.default_rng(7)
    vals = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-12, 10, 200_000))).astype(np.float32)
    clamped = np.clip(vals, -448.0, 448.0)
    t = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    enc = oracle.e4m3_encode(vals)
    assert np.array_equal(t, enc)


def test_ue8m0_decode():
    dec = oracle.ue8m0_decode(np.arange(256, dtype=np.uint8))
    assert dec[127] == 1.0 and dec[128] == 2.0 and dec[126] == 0.5 and dec[0] == 2.0 ** -127
    assert math.isnan(dec[255])
    t = torch.arange(255, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(t, dec[:255])


def test_mx_exponent_bruteforce():
    """e = smallest integer with amax <= 448 * 2^e (clamped to [-127, 127])."""
    rng = np.random.default_rng(5)
    amaxes = [0.0, 448.0, 449.0, 224.0, 224.00002, 1.0, 2.0 ** -130, 3.0e38, 1e-45]
    for j in range(-20, 20):
        for f in (1.0, 1.75, 1.75 * (1 + 2 ** -7), 1.9921875, 1.0078125):
            amaxes.append(448.0 / 1.75 * f * 2.0 ** j)
    amaxes += list(np.exp2(rng.uniform(-140, 127, 2000)))
    for a in amaxes:
        a32 = float(np.float32(a))
        e = oracle.mx_exponent(a32)
        if a32 == 0.0:
            assert e == -127
            continue
        ref = next(k for k in range(-127, 128) if a32 <= 448.0 * 2.0 ** k) \
            if a32 <= 448.0 * 2.0 ** 127 else 127
        assert e == ref, (a32, e, ref)


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(11)
    vals = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-130, 120, 100_000))).astype(np.float32)
    t = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lib = oracle._load()
    mine = np.array([lib.or_f32_to_bf16(float(v)) for v in vals[:20000]], np.uint16)
    assert np.array_equal(mine, t[:20000])


def test_f64_to_bf16_is_nearest_even():
    """Single rounding fp64 -> bf16: brute-force check against the two bf16
    neighbours of every value (ties to even)."""
    rng = np.random.default_rng(13)
    vals = rng.standard_normal(5000) * np.exp2(rng.uniform(-135, 100, 5000))
    # exact ties between adjacent bf16 values
    base = rng.integers(0x0080, 0x7F00, size=500).astype(np.uint16)
    lo = oracle.bf16_to_f32(base).astype(np.float64)
    hi = oracle.bf16_to_f32(base + 1).astype(np.float64)
    vals = np.concatenate([vals, (lo + hi) / 2, -(lo + hi) / 2])
    codes = oracle.f64_to_bf16(vals)
    for v, c in zip(vals, codes):
        r = float(oracle.bf16_to_f32(np.uint16(c)))
        assert math.copysign(1.0, r) == math.copysign(1.0, v)
        mag = c & 0x7FFF
        up = float(oracle.bf16_to_f32(np.uint16(mag + 1)))
        dn = float(oracle.bf16_to_f32(np.uint16(mag - 1))) if mag else 0.0
        a, rr = abs(v), abs(r)
        assert abs(a - rr) <= abs(a - up) and abs(a - rr) <= abs(a - dn), (v, hex(c))
        if abs(a - rr) == abs(a - up) or (mag and abs(a - rr) == abs(a - dn)):
            assert mag % 2 == 0, (v, hex(c))
