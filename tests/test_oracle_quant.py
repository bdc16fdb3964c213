"""Pins for the oracle's quantizers (INT8 per 32-row block, FP8 per channel).

* the per-element error bound |x - q*scale| <= scale/2 * (1 + 2^-14) (half a
  quantization step, with slack for the two fp32 roundings of the scale and
  of its reciprocal);
* brute force with exact rational arithmetic (``fractions.Fraction``) and an
  integer-only fp32 rounding written here, which pins the operation order and
  the rounding mode (including exact .5 ties);
* the FP8 V codes against torch's float8_e4m3fn cast of the same products;
* block boundaries, short tail blocks and the zero/degenerate cases.
"""
from fractions import Fraction

import numpy as np
import torch

import workloads
from fp_exact import rint_half_even, round_fraction_to_f32
from oracle import fp8_e4m3fn_decode, quant_qk, quant_v


_round_fraction_to_f32 = round_fraction_to_f32
_rint_half_even = rint_half_even


def _brute_block(block: np.ndarray):
    amax = max(Fraction(float(abs(x))) for x in block.ravel())
    if amax == 0:
        return 0.0, np.zeros(block.shape, dtype=np.int64)
    inv = _round_fraction_to_f32(Fraction(127) / amax)
    scale = _round_fraction_to_f32(amax / Fraction(127))
    q = np.empty(block.shape, dtype=np.int64)
    for idx, x in np.ndenumerate(block):
        y = _round_fraction_to_f32(Fraction(float(x)) * inv)
        q[idx] = min(127, max(-127, _rint_half_even(y)))
    return float(scale), q


def test_int8_bruteforce_random_blocks():
    q, _, _ = workloads.generate(2, S=64, H=1, seed=11)       # 2 blocks, K-like offsets absent on Q
    _, k, _ = workloads.generate(2, S=64, H=1, seed=12)       # K has channel offsets
    for x in (q, k):
        q8, sc = quant_qk(x)
        for t in range(2):
            blk = x[0, 32 * t:32 * t + 32, 0, :]
            s_ref, q_ref = _brute_block(blk)
            assert sc[0, 0, t] == np.float32(s_ref)
            assert np.array_equal(q8[0, 0, 32 * t:32 * t + 32].astype(np.int64), q_ref)


def test_int8_rounding_ties_go_to_even():
    # amax = 127 gives inverse 1 exactly, so q = rint(x): .5 ties are exact
    x = np.zeros((1, 32, 1, 128), dtype=np.float32)
    x[0, 0, 0, 0] = 127.0
    ties = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5, -126.5], dtype=np.float32)
    x[0, 1, 0, :len(ties)] = ties
    q8, sc = quant_qk(x)
    assert sc[0, 0, 0] == np.float32(1.0)
    assert list(q8[0, 0, 1, :len(ties)]) == [0, 2, 2, 4, 0, -2, -2, 126, -126]
    s_ref, q_ref = _brute_block(x[0, :, 0, :])
    assert np.array_equal(q8[0, 0].astype(np.int64), q_ref)


def test_int8_error_bound_and_range():
    for idx in (1, 2, 3):
        x = workloads.generate(idx, S=512, H=3)[1]            # K of each recipe
        q8, sc = quant_qk(x)
        B, S, H, D = x.shape
        xs = np.transpose(x, (0, 2, 1, 3)).astype(np.float64)  # [B,H,S,D]
        scale_rows = np.repeat(sc, 32, axis=2)[:, :, :S].astype(np.float64)[..., None]
        err = np.abs(xs - q8.astype(np.float64) * scale_rows)
        assert np.all(err <= scale_rows / 2 * (1 + 2.0 ** -14))
        assert q8.min() >= -127 and q8.max() <= 127
        # the element achieving each block's amax maps to +-127
        blocks = np.abs(q8.astype(np.int64)).reshape(B, H, S // 32, 32 * D).max(axis=-1)
        assert np.all(blocks == 127)


def test_int8_short_tail_block_uses_valid_rows_only():
    x = workloads.generate(1, S=80, H=2, seed=5)[0]
    x[0, 64:80] *= np.float32(0.25)                          # tail rows smaller than the rest
    q8, sc = quant_qk(x)
    assert sc.shape == (1, 2, 3)
    q8t, sct = quant_qk(np.ascontiguousarray(x[:, 64:80]))   # the 16 tail rows alone
    assert np.array_equal(sc[:, :, 2], sct[:, :, 0])
    assert np.array_equal(q8[:, :, 64:80], q8t)


def test_int8_zero_and_tiny_blocks():
    x = np.zeros((1, 64, 1, 128), dtype=np.float32)
    x[0, 32:, 0, :] = np.float32(1e-39)                      # 127/amax overflows fp32
    q8, sc = quant_qk(x)
    assert np.all(sc == 0) and np.all(q8 == 0)


def test_fp8_v_bound_codes_and_library_crosscheck():
    v = workloads.generate(3, S=512, H=3)[2]                 # V with per-channel gains
    v8, vs = quant_v(v)
    B, S, H, D = v.shape
    vt = np.transpose(v, (0, 2, 1, 3)).astype(np.float64)
    deq = fp8_e4m3fn_decode(v8) * vs[:, :, None, :].astype(np.float64)
    # half an FP8 step at each magnitude: 2^-4 relative (3 mantissa bits) for
    # normal values, 2^-10 * v_scale absolute in the subnormal range
    step = np.maximum(np.abs(vt) * 2.0 ** -4, 2.0 ** -10 * vs[:, :, None, :])
    assert np.all(np.abs(vt - deq) <= step * (1 + 2.0 ** -12))
    # each channel's amax element is coded +-448
    assert np.all(np.abs(fp8_e4m3fn_decode(v8)).max(axis=2) == 448.0)
    # independent codec: torch's float8_e4m3fn cast of fl32(v * fl32(448/amax))
    amax = np.abs(v).max(axis=1)                              # [B,H,D]
    inv = (np.float32(448) / amax).astype(np.float32)
    y = (np.transpose(v, (0, 2, 1, 3)) * inv[:, :, None, :]).astype(np.float32)
    assert np.all(np.abs(y) <= 448.0 * (1 + 2.0 ** -20))
    ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(v8, ref)
    assert np.array_equal(vs, (amax / np.float32(448)).astype(np.float32))


def test_fp8_v_zero_channel():
    v = workloads.generate(1, S=64, H=1)[2]
    v[..., 5] = 0.0
    v8, vs = quant_v(v)
    assert vs[0, 0, 5] == 0 and np.all(v8[0, 0, :, 5] == 0)
