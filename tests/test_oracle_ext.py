"""Pins for the oracle's extensions: K smoothing, the log-sum-exp output and
query/key sequences of different lengths (cross-attention).

* k_mean: equal to the exact rational mean rounded once to fp32 (brute
  force with ``fractions.Fraction``, including channels whose values span
  more binades than an int64 holds); exact for constant channels and for
  rows that cancel in pairs; planted mistakes (a sequential fp32 sum, a
  divisor of S + 1) fail it;
* K smoothing: a zero-mean K quantizes exactly as without smoothing; a
  shifted K gives the same smoothed codes as the unshifted one when the
  shift is exactly representable; smoothed quantized attention stays
  within the method's tolerance of exact fp64 attention on the original K,
  and beats unsmoothed quantization when one K channel carries a large
  constant offset;
* LSE: the exact-reference LSE equals scipy's logsumexp; the oracle's LSE
  equals the fp64 logsumexp of the dequantized scores within the bound of
  its fp32 exponent roundings; one key gives closed forms for O and LSE;
  planted mistakes (no ln 2, an offset) fail it;
* cross-attention: close to exact fp64 attention for Sq != Skv with ragged
  tails on both sides; Sq = Skv reproduces the self-attention call.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle.attention as oatt
import oracle.quant as oquant
import workloads
from fp_exact import round_fraction_to_f32
from oracle import (
    attention_head,
    exact_attention_fp64,
    fp8_e4m3fn_decode,
    k_mean,
    qk_scores,
    quant_k_smooth,
    quant_qk,
    quant_v,
    sage_attention,
)

SCALE = 1.0 / math.sqrt(128)
U32 = 2.0 ** -24


def _cos(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _cross_inputs(idx, Sq, Skv, H=2, seed=5):
    q, _, _ = workloads.generate(idx, S=Sq, H=H, B=1, seed=seed)
    _, k, v = workloads.generate(idx, S=Skv, H=H, B=1, seed=seed + 1000)
    return q, k, v


# ---------------------------------------------------------------- k_mean

def _brute_mean(k):
    B, S, H, D = k.shape
    out = np.empty((B, H, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for c in range(D):
                tot = sum(Fraction(float(x)) for x in k[b, :, h, c])
                out[b, h, c] = float(round_fraction_to_f32(tot / S))
    return out


def _mean_inputs(S):
    k = workloads.generate_custom((1, S, 3, 128), seed=S, kind="normal", scale=3.0)
    k[:, :, 1, 5] += np.float32(40.0)          # a channel with an offset
    k[:, :, 2, 9] = np.float32(2.0 ** -30)     # values 50 binades apart in one
    k[:, ::7, 2, 9] = np.float32(2.0 ** 22)    # channel: the Python-integer path
    return workloads.bf16_round(k)


@pytest.mark.parametrize("S", [1, 31, 32, 100, 777])
def test_k_mean_is_the_exact_mean_rounded_once(S):
    k = _mean_inputs(S)
    assert np.array_equal(k_mean(k).view(np.uint32), _brute_mean(k).view(np.uint32))


def test_planted_k_mean_mistakes_fail_the_pin(monkeypatch):
    k = _mean_inputs(777)
    ref = _brute_mean(k)

    def sequential_fp32(kk):                    # fp32 running sum over s
        acc = np.zeros((kk.shape[0], kk.shape[2], kk.shape[3]), np.float32)
        for s_ in range(kk.shape[1]):
            acc = (acc + kk[:, s_]).astype(np.float32)
        return (acc / np.float32(kk.shape[1])).astype(np.float32)

    real = oquant.k_mean

    def off_by_one(kk):                         # divides by S + 1
        return (real(kk).astype(np.float64) * kk.shape[1] / (kk.shape[1] + 1)).astype(np.float32)

    for mistake in (sequential_fp32, off_by_one):
        assert not np.array_equal(mistake(k), ref), mistake.__name__


def test_k_mean_constant_channels_exact():
    S = 100
    k = np.zeros((2, S, 2, 128), dtype=np.float32)
    k[...] = (np.arange(128, dtype=np.float32) * np.float32(0.25) - np.float32(8.0))[None, None, None, :]
    m = k_mean(k)
    assert np.array_equal(m, np.broadcast_to(k[:, 0, :, :], m.shape))


def test_zero_mean_k_quantizes_as_unsmoothed():
    # rows in cancelling pairs: the exact mean is 0
    half = workloads.generate_custom((1, 48, 2, 128), seed=9, kind="normal", scale=2.0)
    k = np.empty((1, 96, 2, 128), dtype=np.float32)
    k[:, 0::2] = half
    k[:, 1::2] = -half
    k8s, kss, mean = quant_k_smooth(k)
    assert np.all(mean == 0)
    k8, ks = quant_qk(k)
    assert np.array_equal(k8s, k8) and np.array_equal(kss, ks)


def test_smoothing_removes_exact_channel_shift():
    # k2 = k + c with c a small power-of-two multiple: k2 - mean(k2) equals
    # k - mean(k) exactly when every step is exact, so the codes agree.
    k = workloads.generate_custom((1, 64, 1, 128), seed=4, kind="uniform", scale=1.0)
    k = (np.round(k * 64) / 64).astype(np.float32)     # multiples of 2^-6, exact sums
    shift = (np.arange(128) % 5).astype(np.float32) * np.float32(4.0)
    a8, a_s, am = quant_k_smooth(k)
    b8, b_s, bm = quant_k_smooth((k + shift[None, None, None, :]).astype(np.float32))
    assert np.array_equal(bm - am, np.broadcast_to(shift, bm.shape))
    assert np.array_equal(a8, b8) and np.array_equal(a_s, b_s)


def test_smoothed_attention_close_to_exact_on_original_k():
    for idx in (1, 2, 5):
        cfg = workloads.config(idx)
        q, k, v = workloads.generate(idx, S=384, H=2, B=1, seed=17)
        o = sage_attention(q, k, v, cfg.softmax_scale, 128, smooth_k=True)
        e = exact_attention_fp64(q, k, v, cfg.softmax_scale)
        assert _cos(o, e) >= 0.99, idx


def test_smoothing_helps_with_a_constant_k_channel_offset():
    q, k, v = workloads.generate(1, S=256, H=1, B=1, seed=23)
    k = k.copy()
    k[:, :, :, 7] += np.float32(600.0)        # one K channel far from zero
    e = exact_attention_fp64(q, k, v, SCALE)
    plain = sage_attention(q, k, v, SCALE, 128)
    smooth = sage_attention(q, k, v, SCALE, 128, smooth_k=True)
    err_plain = np.linalg.norm(plain - e) / np.linalg.norm(e)
    err_smooth = np.linalg.norm(smooth - e) / np.linalg.norm(e)
    assert err_smooth < 0.5 * err_plain


# ------------------------------------------------------------------- LSE

def test_exact_reference_lse_is_logsumexp():
    q, k, v = _cross_inputs(2, 70, 130)
    _, lse = exact_attention_fp64(q, k, v, SCALE, return_lse=True)
    for h in range(q.shape[2]):
        s = (q[0, :, h].astype(np.float64) @ k[0, :, h].astype(np.float64).T) * SCALE
        assert np.allclose(lse[0, h], logsumexp(s, axis=1), rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("idx,Sq,Skv", [(1, 256, 256), (3, 300, 520), (5, 100, 1000)])
def test_oracle_lse_matches_dequantized_logsumexp(idx, Sq, Skv):
    cfg = workloads.config(idx)
    q, k, v = _cross_inputs(idx, Sq, Skv)
    q8, qs = quant_qk(q)
    k8, ks = quant_qk(k)
    v8, vs = quant_v(v)
    errs = []
    for h in range(q.shape[2]):
        _, lse = attention_head(q8[0, h], qs[0, h], k8[0, h], ks[0, h], v8[0, h], vs[0, h],
                                cfg.softmax_scale, 128, return_lse=True)
        A = qk_scores(q8[0, h], k8[0, h]).astype(np.float64)
        deq = (A * qs[0, h][np.arange(Sq) // 32][:, None].astype(np.float64)
               * ks[0, h][np.arange(Skv) // 32][None, :].astype(np.float64))
        ref = logsumexp(deq * cfg.softmax_scale, axis=1)
        # l sums the decoded FP8 codes of P' = 2^(t - m2): each is P' (1 +
        # eta) with |eta| <= 2^-4 in the normal range, or P' + zeta with
        # |zeta| <= 2^-10 below it, and l >= ~448 (the row's largest term),
        # so ln l is within ln(1 + 2^-4 + Skv 2^-10 / 448) of the exact sum's
        # logarithm; each exponent also carries fp32 roundings of about one
        # unit of f (the per-block factor in the log2 domain)
        f = (qs[0, h][np.arange(Sq) // 32][:, None].astype(np.float64)
             * ks[0, h][None, :].astype(np.float64) * cfg.softmax_scale * math.log2(math.e))
        fmax = f.max(axis=1)
        tmax = np.abs(deq).max(axis=1) * cfg.softmax_scale * math.log2(math.e)
        bound = (math.log1p(2.0 ** -4 + Skv * 2.0 ** -10 / 448)
                 + math.log(2.0) * (2.5 * fmax + 8 * U32 * (tmax + 30)) + 4 * U32 * np.abs(ref))
        err = lse.astype(np.float64) - ref
        assert np.all(np.abs(err) <= bound), h
        errs.append(err)
    # the FP8 roundings go either way: their mean effect over the rows is far
    # smaller than their per-row bound (measured 1e-4 to 7e-4 on these
    # inputs), which pins a systematic offset of the LSE
    assert abs(np.mean(np.concatenate(errs))) <= 2e-3


def test_planted_lse_mistakes_fail_the_pin(monkeypatch):
    real = oatt.lse_from_state
    for mistake in (lambda m2, l: np.float32(1.0 / math.log(2.0)) * real(m2, l) * np.float32(math.log(2.0) ** 2),
                    lambda m2, l: oatt.f32(np.asarray(m2, np.float64) + np.log2(np.asarray(l, np.float64))),
                    lambda m2, l: real(m2, l) + np.float32(0.01)):
        monkeypatch.setattr(oatt, "lse_from_state", mistake)
        with pytest.raises(AssertionError):
            test_oracle_lse_matches_dequantized_logsumexp(1, 256, 256)


def test_single_key_closed_forms():
    q = workloads.generate_custom((1, 40, 1, 128), seed=31, kind="normal")
    k = workloads.generate_custom((1, 1, 1, 128), seed=32, kind="normal")
    v = workloads.generate_custom((1, 1, 1, 128), seed=33, kind="normal", scale=5.0)
    out, lse = sage_attention(q, k, v, SCALE, 128, return_lse=True)
    v8, vs = quant_v(v)
    # one key: P' = 448 = p8, l = 448, so O = bf16(dec(v8) * v_scale)
    expect = fp8_e4m3fn_decode(v8[0, 0, 0]) * vs[0, 0].astype(np.float64)
    bf = np.array(expect, dtype=np.float32)
    assert np.allclose(out[0, :, 0, :], np.broadcast_to(bf, out[0, :, 0, :].shape), rtol=2 ** -8, atol=0)
    q8, qs = quant_qk(q)
    k8, ks = quant_qk(k)
    score = qk_scores(q8[0, 0], k8[0, 0])[:, 0].astype(np.float64) * qs[0, 0][np.arange(40) // 32] * ks[0, 0][0]
    f = qs[0, 0][np.arange(40) // 32].astype(np.float64) * ks[0, 0][0] * SCALE * math.log2(math.e)
    assert np.all(np.abs(lse[0, 0] - score * SCALE) <= math.log(2.0) * (2.5 * f + 1e-6) + 1e-6)


# -------------------------------------------------------- cross-attention

@pytest.mark.parametrize("idx,Sq,Skv", [(1, 300, 77), (2, 64, 700), (3, 250, 260), (5, 129, 1000)])
def test_cross_attention_close_to_exact(idx, Sq, Skv):
    cfg = workloads.config(idx)
    q, k, v = _cross_inputs(idx, Sq, Skv)
    o = sage_attention(q, k, v, cfg.softmax_scale, 128)
    e = exact_attention_fp64(q, k, v, cfg.softmax_scale)
    assert o.shape == q.shape
    assert _cos(o, e) >= 0.99


def test_equal_lengths_reproduce_self_attention_rows():
    q, k, v = workloads.generate(2, S=200, H=1, B=1, seed=8)
    full = sage_attention(q, k, v, SCALE, 128)
    rows = np.array([0, 31, 32, 150, 199])
    part = sage_attention(q, k, v, SCALE, 128, rows=rows)
    assert np.array_equal(full[:, rows], part[:, rows])


# ------------------------------------------------------------ head dim 64

def _d64(x):
    return np.ascontiguousarray(x[..., :64])


@pytest.mark.parametrize("idx,Sq,Skv", [(1, 256, 256), (2, 300, 77), (5, 129, 500)])
def test_head_dim_64_close_to_exact(idx, Sq, Skv):
    q, k, v = _cross_inputs(idx, Sq, Skv)
    q, k, v = _d64(q), _d64(k), _d64(v)
    scale = 1.0 / math.sqrt(64)
    o, lse = sage_attention(q, k, v, scale, 128, return_lse=True)
    e, lse_exact = exact_attention_fp64(q, k, v, scale, return_lse=True)
    assert o.shape == q.shape
    assert _cos(o, e) >= 0.99
    assert np.max(np.abs(lse - lse_exact)) < 0.05


def test_head_dim_64_quantization_matches_per_channel_slices():
    # channels are independent in V's quantization and K's mean: the first
    # 64 channels of a D=128 call equal a D=64 call on those channels
    _, k, v = workloads.generate(3, S=300, H=2, B=1, seed=77)
    v8, vs = quant_v(v)
    v8h, vsh = quant_v(_d64(v))
    assert np.array_equal(v8[..., :64], v8h) and np.array_equal(vs[..., :64], vsh)
    assert np.array_equal(k_mean(k)[..., :64], k_mean(_d64(k)))
