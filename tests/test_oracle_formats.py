"""Pins for the oracle's number formats (FP8 E4M3FN codec, bf16 rounding).

The codec is pinned to the OCP 8-bit floating point specification's E4M3
table (a hand-written fixture), exhaustively to its own grid (every code
round-trips, every midpoint goes to the even code), and to an independent
library implementation (torch.float8_e4m3fn) on the whole in-range domain.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16_round_f64, fp8_e4m3fn_decode, fp8_e4m3fn_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_landmarks.txt")


def _landmarks():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


def test_landmarks_decode_and_encode():
    for code, val in _landmarks():
        dec = fp8_e4m3fn_decode(np.array([code], dtype=np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(dec)
            continue
        assert dec == val and math.copysign(1, dec) == math.copysign(1, val), (hex(code), dec, val)
        enc = fp8_e4m3fn_encode(np.array([val]))[0]
        assert enc == code, (hex(code), hex(enc))


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_every_finite_code_round_trips():
    codes = _finite_codes()
    assert len(codes) == 254
    vals = fp8_e4m3fn_decode(codes)
    assert np.array_equal(fp8_e4m3fn_encode(vals), codes)
    # the positive finite non-zero codes are strictly increasing in value
    pos = fp8_e4m3fn_decode(np.arange(1, 0x7F, dtype=np.uint8))
    assert len(pos) == 126 and np.all(np.diff(pos) > 0)


def test_midpoints_round_to_even_code():
    pos_codes = np.arange(0, 0x7F, dtype=np.uint8)   # 0 .. 448
    vals = fp8_e4m3fn_decode(pos_codes)
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2
    got = fp8_e4m3fn_encode(mid)
    even = np.where(pos_codes[:-1] % 2 == 0, pos_codes[:-1], pos_codes[1:])
    assert np.array_equal(got, even)
    # just off the midpoint goes to the nearer code
    eps = (hi - lo) * 1e-6
    assert np.array_equal(fp8_e4m3fn_encode(mid - eps), pos_codes[:-1])
    assert np.array_equal(fp8_e4m3fn_encode(mid + eps), pos_codes[1:])
    # negative side mirrors
    assert np.array_equal(fp8_e4m3fn_encode(-mid), even | 0x80)


def test_saturation_and_specials():
    enc = lambda x: int(fp8_e4m3fn_encode(np.array([x]))[0])  # noqa: E731
    assert enc(464.0) == 0x7E          # tie between 448 and (unrepresentable) 480 -> even
    assert enc(470.0) == 0x7E          # saturates
    assert enc(1e30) == 0x7E
    assert enc(math.inf) == 0x7E
    assert enc(-500.0) == 0xFE
    assert enc(2.0 ** -10) == 0x00     # half the smallest subnormal: tie -> 0 (even)
    assert enc(2.0 ** -10 * 1.0001) == 0x01
    assert enc(-(2.0 ** -11)) == 0x80  # negative value rounding to zero keeps its sign
    assert enc(math.nan) & 0x7F == 0x7F


def test_encoder_matches_torch_float8_e4m3fn_in_range():
    rng = np.random.default_rng(0)
    # every float32 between consecutive codes is covered by dense samples of
    # each binade plus exact grid points and midpoints
    pos = fp8_e4m3fn_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    samples = [pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
               np.nextafter(mids.astype(np.float32), np.float32(1e9))]
    for e in range(-12, 9):
        samples.append(rng.uniform(2.0 ** e, 2.0 ** (e + 1), 4000))
    y = np.concatenate(samples).astype(np.float32)
    y = y[np.abs(y) < 464]            # torch returns NaN instead of saturating above
    y = np.concatenate([y, -y])
    ours = fp8_e4m3fn_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (y[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_bf16_rounding_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40, -2.5e-41]])
    x = x.astype(np.float32)
    ours = bf16_round_f64(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_rounding_is_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-30: rounding through fp32 first would lose 2^-30 and then
    # tie to even (1.0); one rounding from the real value gives 1 + 2^-7.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_round_f64(np.array([x]))[0] == np.float32(1.0 + 2.0 ** -7)
    assert bf16_round_f64(np.array([1.0 + 2.0 ** -8]))[0] == np.float32(1.0)
    assert bf16_round_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == np.float32(1.0 + 2.0 ** -6)


@pytest.mark.parametrize("x", [0.1, -3.14159, 1e-39, 65504.0, 1.5e38])
def test_bf16_rounding_is_nearest(x):
    r = float(bf16_round_f64(np.array([x]))[0])
    # the two bf16 neighbours of x bracket it and r is the nearer
    b = np.array([r], dtype=np.float32).view(np.uint32)[0]
    up = np.array([b + 0x10000], dtype=np.uint32).view(np.float32)[0]
    dn = np.array([b - 0x10000], dtype=np.uint32).view(np.float32)[0]
    assert abs(r - x) <= abs(float(up) - x) and abs(r - x) <= abs(float(dn) - x)
