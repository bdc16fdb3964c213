"""Pins for the oracle's attention steps.

Each pin is chosen so that a plausible mistake in the oracle (a dropped
rescale, a wrong tile boundary, a transposed operand, a wrong scale index, a
sign error in the exponent) fails at least one of them:

* exact integer scores: int64 reference vs the float64 product;
* the tile loop with quantization switched off equals textbook fp64 softmax
  attention to 1e-12, at several tile widths and ragged tails;
* the whole oracle is within cosine 0.99 of exact fp64 attention;
* row sums: V = 1 gives O = 1 (exactly in the unquantized loop; exactly
  when quantized too, since the normalizer sums the same FP8 weights that
  multiply V), and the quantized weights of every row sum to one;
* invariances: joint K/V row permutations inside a 32-row block, Q row
  permutations inside a block, power-of-two scalings;
* closed forms: K = 0 (O = mean of dequantized V), V = 0, one dominant key;
* the masked tail equals the unpadded computation;
* the exponent step: every exponent the oracle forms is the exact real value
  A*f - m2 rounded once to fp32 (checked with rational arithmetic), m2 and
  the running maximum are the roundings of their exact definitions, P' is
  2^arg to half an ulp and p8 is the nearest FP8 code;
* an independent scalar implementation that takes the method's steps in
  their plain order (t = fl32(A f), fl32(t - m), 2^(...), then 448 * P) on
  tiny inputs, and a vectorized one of the same order on large-magnitude
  inputs, agree with the oracle within the output tolerance;
* planted mistakes in the exponent step (a biased accumulator read, a
  two-step rounding) fail these pins.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle.attention as oatt
import workloads
from fp_exact import round_fraction_to_f32
from oracle import (
    attention_head,
    exact_attention_fp64,
    exp2_scale,
    fp8_e4m3fn_decode,
    fp8_e4m3fn_encode,
    online_softmax_exact,
    online_softmax_pv,
    qk_scores,
    quant_qk,
    quant_v,
    sage_attention,
)

SCALE = 1.0 / math.sqrt(128)


def _cos(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def _head_inputs(q, k, v, b=0, h=0):
    q8, qs = quant_qk(q)
    k8, ks = quant_qk(k)
    v8, vs = quant_v(v)
    return q8[b, h], qs[b, h], k8[b, h], ks[b, h], v8[b, h], vs[b, h]


def test_scores_exact_integer():
    rng = np.random.default_rng(3)
    q8 = rng.integers(-127, 128, size=(70, 128)).astype(np.int8)
    k8 = rng.integers(-127, 128, size=(90, 128)).astype(np.int8)
    ref = np.einsum("ic,jc->ij", q8.astype(np.int64), k8.astype(np.int64))
    assert np.array_equal(qk_scores(q8, k8), ref)
    extreme = np.full((2, 128), 127, dtype=np.int8)
    extreme[1] = -127
    assert qk_scores(extreme, extreme)[0, 0] == 128 * 127 * 127 < 2 ** 24


@pytest.mark.parametrize("S,bn,n_valid", [(256, 64, None), (200, 64, None), (256, 32, None),
                                          (300, 128, None), (256, 128, 201)])
def test_unquantized_tile_loop_is_textbook_softmax(S, bn, n_valid):
    rng = np.random.default_rng(S + bn)
    q = rng.standard_normal((1, S, 1, 128)) * 2.0
    k = rng.standard_normal((1, S, 1, 128))
    v = rng.standard_normal((1, S, 1, 128))
    nv = S if n_valid is None else n_valid
    x = (q[0, :, 0] @ k[0, :, 0].T) * SCALE * math.log2(math.e)
    acc, l = online_softmax_exact(x, v[0, :, 0], bn, n_valid=n_valid)
    # textbook softmax over the first nv keys, written out here
    s = (q[0, :, 0] @ k[0, :nv, 0].T) * SCALE
    p = np.exp(s - s.max(axis=1, keepdims=True))
    ref = (p @ v[0, :nv, 0]) / p.sum(axis=1, keepdims=True)
    assert np.max(np.abs(acc / l[:, None] - ref)) < 1e-12
    # and the library's exact reference (Sq = S, Skv = nv) equals it too
    ex = exact_attention_fp64(q, k[:, :nv], v[:, :nv], SCALE)[0, :, 0]
    assert np.max(np.abs(ex - ref)) < 1e-12


def test_unquantized_row_sum_is_one():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 300)) * 20
    acc, l = online_softmax_exact(x, np.ones((300, 4)), 64)
    assert np.max(np.abs(acc / l[:, None] - 1.0)) < 1e-12


def test_quantized_row_sum_is_exactly_one():
    # V constant per channel: v8 = 448 everywhere and v_scale = fl32(0.75/448),
    # so O = sum dec(p8) * 448 * v_scale / sum dec(p8) = 448 * fl32(0.75/448)
    q, k, _ = workloads.generate(3, S=512, H=1)
    v = np.ones_like(q) * np.float32(0.75)
    args = _head_inputs(q, k, v)
    o, o64 = attention_head(*args, SCALE, 128, return_f64=True)
    vs = float(np.float32(0.75) / np.float32(448.0))
    assert np.all(np.abs(o64 - 448.0 * vs) <= 1e-14)
    assert np.all(o == np.float32(0.75))
    # the weights the tile loop applies to V sum to one in every row
    A = qk_scores(args[0], args[2])
    c = exp2_scale(SCALE)
    f = (args[1][np.arange(512) // 32][:, None] * args[3][None, :]).astype(np.float32)
    f = (f * c).astype(np.float32)[:, np.arange(512) // 32]
    acc, l = online_softmax_pv(A, f, np.ones((512, 1)), 128)
    assert np.all(np.abs(acc[:, 0] / l - 1.0) <= 1e-15)


def test_oracle_vs_exact_attention_config1():
    cfg = workloads.config(1)
    q, k, v = workloads.generate(1)
    for bn in (64, 128):
        o = sage_attention(q, k, v, cfg.softmax_scale, bn)
        e = exact_attention_fp64(q, k, v, cfg.softmax_scale)
        c = _cos(o, e)
        assert c >= 0.99
        assert c > 0.998      # FP8 P and V noise floor, about 0.9993 here


def test_oracle_vs_exact_attention_structured_recipes():
    for idx in (2, 3, 5):
        cfg = workloads.config(idx)
        q, k, v = workloads.generate(idx, S=512, H=2, B=1)
        o = sage_attention(q, k, v, cfg.softmax_scale, 128)
        e = exact_attention_fp64(q, k, v, cfg.softmax_scale)
        assert _cos(o, e) >= 0.99, idx


def test_joint_kv_permutation_inside_block_invariance():
    q, k, v = workloads.generate(2, S=256, H=1, seed=21)
    args = _head_inputs(q, k, v)
    o, o64 = attention_head(*args, SCALE, 64, return_f64=True)
    rng = np.random.default_rng(0)
    perm = np.arange(256)
    for blk in range(8):
        perm[32 * blk:32 * blk + 32] = 32 * blk + rng.permutation(32)
    kp, vp = k[:, perm], v[:, perm]
    args_p = _head_inputs(q, kp, vp)
    assert np.array_equal(args_p[3], args[3]) and np.array_equal(args_p[5], args[5])
    op, op64 = attention_head(*args_p, SCALE, 64, return_f64=True)
    assert np.max(np.abs(op64 - o64)) <= 1e-12 * np.max(np.abs(o64))
    assert np.mean(op == o) > 0.999
    # negative control: swapping rows across blocks changes the K block scales
    # and the output
    cross = np.arange(256)
    cross[[5, 40]] = cross[[40, 5]]
    cross[[70, 200]] = cross[[200, 70]]
    k[0, 5] *= 3.0
    args_c = _head_inputs(q, k[:, cross], v[:, cross])
    args_0 = _head_inputs(q, k, v)
    assert not np.array_equal(args_c[3], args_0[3])
    oc64 = attention_head(*args_c, SCALE, 64, return_f64=True)[1]
    o064 = attention_head(*args_0, SCALE, 64, return_f64=True)[1]
    assert np.max(np.abs(oc64 - o064)) > 1e-6


def test_query_permutation_inside_block_is_bit_exact():
    q, k, v = workloads.generate(1, S=128, H=1, seed=22)
    perm = np.arange(128)
    perm[32:64] = 32 + np.random.default_rng(1).permutation(32)
    o = attention_head(*_head_inputs(q, k, v), SCALE, 64)
    op = attention_head(*_head_inputs(q[:, perm], k, v), SCALE, 64)
    assert np.array_equal(op, o[perm])


def test_power_of_two_scalings_are_exact():
    q, k, v = workloads.generate(3, S=256, H=1, seed=23)
    o = attention_head(*_head_inputs(q, k, v), SCALE, 64)
    o_v = attention_head(*_head_inputs(q, k, v * np.float32(8.0)), SCALE, 64)
    assert np.array_equal(o_v, o * np.float32(8.0))
    o_q = attention_head(*_head_inputs(q * np.float32(4.0), k, v), SCALE / 4.0, 64)
    assert np.array_equal(o_q, o)


def test_closed_form_k_zero_gives_mean_of_dequantized_v():
    q, _, v = workloads.generate(1, S=256, H=1, seed=24)
    k = np.zeros_like(q)
    q8, qs, k8, ks, v8, vs = _head_inputs(q, k, v)
    _, o64 = attention_head(q8, qs, k8, ks, v8, vs, SCALE, 64, return_f64=True)
    mean = (fp8_e4m3fn_decode(v8) * vs[None, :].astype(np.float64)).mean(axis=0)
    # every P' is fl32(2^fl32(log2 448)) = 448 (1 +- 4e-7), encoded as 448
    assert np.max(np.abs(o64 - mean[None, :])) <= 1e-6 * np.max(np.abs(mean))


def test_closed_form_v_zero():
    q, k, _ = workloads.generate(1, S=128, H=1, seed=25)
    o = attention_head(*_head_inputs(q, k, np.zeros_like(q)), SCALE, 64)
    assert np.all(o == 0)


def test_closed_form_single_dominant_key():
    q, k, v = workloads.generate(1, S=256, H=1, seed=26)
    j = 77
    q[0, :, 0, :] = workloads.bf16_round(np.sign(k[0, j, 0, :]) * 4.0)
    k[0, j, 0, :] = workloads.bf16_round(np.sign(k[0, j, 0, :]) * 8.0)
    q8, qs, k8, ks, v8, vs = _head_inputs(q, k, v)
    _, o64 = attention_head(q8, qs, k8, ks, v8, vs, SCALE, 64, return_f64=True)
    vj = fp8_e4m3fn_decode(v8[j]) * vs.astype(np.float64)
    # every other key is 2^-400 below, so only key j carries weight; its P'
    # is 448 * 2^d with |d| bounded by the fp32 roundings of the running max
    # m (about 522 here, spacing 2^-14) and of m - log2 448
    m = float(qk_scores(q8[:1], k8[j:j + 1])[0, 0]) * qs[0] * ks[j // 32] * SCALE * math.log2(math.e)
    assert 512 <= m < 1024
    bound = 2.0 ** -14 * math.log(2) + 2.0 ** -22
    assert np.max(np.abs(o64 - vj[None, :])) <= bound * np.max(np.abs(vj))


def test_masked_tail_equals_unpadded():
    q, k, v = workloads.generate(5, S=80, H=1, B=1, seed=27)
    o = attention_head(*_head_inputs(q, k, v), SCALE, 64)
    pad = lambda x: np.concatenate([x, np.zeros((1, 48, 1, 128), np.float32)], axis=1)  # noqa: E731
    q8, qs, k8, ks, v8, vs = _head_inputs(pad(q), pad(k), pad(v))
    # zero rows change no block amax, so the quantized tensors agree on valid rows
    q8u, qsu, k8u, ksu, v8u, vsu = _head_inputs(q, k, v)
    assert np.array_equal(ks[:3], ksu) and np.array_equal(vs, vsu)
    op = attention_head(q8, qs, k8, ks, v8, vs, SCALE, 64, rows=np.arange(80), n_valid=80)
    assert np.array_equal(op, o)


# ---------------------------------------------------------------------------
# Independent scalar implementation (pure Python floats, tiny sizes only)

def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


_CODES = [(c, (c & 7) * 2.0 ** -9 if (c >> 3) == 0 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7))
          for c in range(0x7F)]


def _e4m3_scalar(y):
    """Nearest E4M3FN code by exhaustive search; ties to the even code."""
    a = min(abs(y), 448.0)
    best = None
    for c, val in _CODES:
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c, val)
    return math.copysign(best[2], y)


def _bf16_scalar(x):
    # nearest bf16 by checking the truncated value and the next one up
    b = struct.unpack("I", struct.pack("f", _f32(x)))[0] & 0xFFFF0000
    cands = []
    for bb in (b - 0x10000, b, b + 0x10000):
        if 0 <= bb < 2 ** 32:
            cands.append(struct.unpack("f", struct.pack("I", bb))[0])
    best = min(cands, key=lambda c: (abs(c - x), (struct.unpack("I", struct.pack("f", c))[0] >> 16) & 1))
    return best


def _scalar_method(q, k, v, scale, bn):
    """One head, every step with scalar Python arithmetic, in the plain step
    order of the method: t = fl32(A f), running max m, P~ = fl32(2^fl32(t - m)),
    p8 = E4M3FN(fl32(448 P~)), l = sum of p8 / 448, O = acc * v_scale / (448 l)
    (the oracle folds 448 into the exponent and forms A f - m2 with one
    rounding; the two orders differ only by fp32 roundings)."""
    S, D = len(q), len(q[0])
    def quant_rows(x):
        out, scales = [], []
        for t in range(0, S, 32):
            blk = x[t:t + 32]
            amax = max(abs(e) for row in blk for e in row)
            inv = _f32(127.0 / amax) if amax > 0 else 0.0
            scales.append(_f32(amax / 127.0) if amax > 0 else 0.0)
            for row in blk:
                out.append([max(-127, min(127, round(_f32(e * inv)))) for e in row])
        return out, scales
    q8, qs = quant_rows(q)
    k8, ks = quant_rows(k)
    vq, vs = [], []
    for c in range(D):
        amax = max(abs(v[j][c]) for j in range(S))
        inv = _f32(448.0 / amax)
        vs.append(_f32(amax / 448.0))
        vq.append([_e4m3_scalar(_f32(v[j][c] * inv)) for j in range(S)])
    c2 = _f32(_f32(scale) * _f32(math.log2(math.e)))
    out = []
    for i in range(S):
        A = [sum(q8[i][d] * k8[j][d] for d in range(D)) for j in range(S)]
        f = [_f32(_f32(qs[i // 32] * ks[j // 32]) * c2) for j in range(S)]
        t = [_f32(A[j] * f[j]) for j in range(S)]
        m = -math.inf
        l, acc = 0.0, [0.0] * D
        for j0 in range(0, S, bn):
            js = range(j0, min(S, j0 + bn))
            m_new = max(m, max(t[j] for j in js))
            if m != -math.inf:
                w = 2.0 ** (m - m_new)
                l *= w
                acc = [a * w for a in acc]
            for j in js:
                pt = _f32(2.0 ** _f32(t[j] - m_new))
                p8 = _e4m3_scalar(_f32(448.0 * pt))
                l += p8 / 448.0
                for c in range(D):
                    acc[c] += p8 * vq[c][j]
            m = m_new
        out.append([_bf16_scalar(acc[c] * vs[c] / (448.0 * l)) for c in range(D)])
    return out


def _gate_ratio(got, ref):
    """max|got - ref| in units of the output gate 1e-2 * max|ref|."""
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / (1e-2 * np.max(np.abs(ref))))


@pytest.mark.parametrize("S,bn", [(40, 32), (96, 64)])
def test_scalar_bruteforce_agrees(S, bn):
    q, k, v = workloads.generate(3, S=S, H=1, seed=30 + S)
    ref = np.array(_scalar_method(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(),
                                  SCALE, bn), dtype=np.float32)
    got = sage_attention(q, k, v, SCALE, bn)[0, :, 0]
    # the two orders round differently only at the fp32 level: most outputs
    # agree to the bit, and a rare FP8 flip of P stays inside the tolerance
    assert np.mean(got == ref) > 0.95
    assert _gate_ratio(got, ref) <= 1.0


# ---------------------------------------------------------------------------
# The exponent step, pinned with exact rational arithmetic

_L448 = Fraction(float(np.float32(math.log2(448.0))))


def _exponent_mismatches(q, k, v, scale, bn, rows):
    """Check every exponent, shift, P' and p8 of the oracle's tile loop for
    the given query rows against their exact definitions; returns the number
    of disagreements (0 when the oracle does what its reading states)."""
    q8, qs = quant_qk(q)
    k8, ks = quant_qk(k)
    v8, _ = quant_v(v)
    q8, qs, k8, ks, v8 = q8[0, 0], qs[0, 0], k8[0, 0], ks[0, 0], v8[0, 0]
    S = k8.shape[0]
    c = exp2_scale(scale)
    A = qk_scores(q8[rows], k8)
    f = ((qs[rows // 32][:, None] * ks[None, :]).astype(np.float32) * c).astype(np.float32)
    f = f[:, np.arange(S) // 32]
    trace = []
    online_softmax_pv(A, f, fp8_e4m3fn_decode(v8), bn, trace=trace)
    bad = 0
    for r in range(len(rows)):
        m = None
        for tile in trace:
            j0, j1 = tile["j0"], tile["j1"]
            ts = [round_fraction_to_f32(Fraction(int(A[r, j])) * Fraction(float(f[r, j]))) for j in range(j0, j1)]
            m = max(ts) if m is None else max(m, max(ts))
            m2 = round_fraction_to_f32(m - _L448)
            bad += Fraction(float(tile["m2"][r])) != m2
            for j in range(j0, j1):
                exact = Fraction(int(A[r, j])) * Fraction(float(f[r, j])) - m2
                arg = tile["arg"][r, j - j0]
                bad += Fraction(float(arg)) != round_fraction_to_f32(exact)
                p = float(tile["p"][r, j - j0])
                want = 2.0 ** float(arg)
                # half an ulp, relative for normal results, 2^-150 absolute
                # below the normal range (flush to zero included)
                bad += abs(p - want) > max(2.0 ** -24 * want, 2.0 ** -150)
                bad += _e4m3_scalar(p) != fp8_e4m3fn_decode(tile["p8"][r, j - j0])
    return bad


def _stress_inputs(kind, S, seed):
    q, k, v = workloads.generate(1 if kind != "c3" else 3, S=S, H=1, B=1, seed=seed)
    if kind == "x40":
        q, k = workloads.bf16_round(q * 40), workloads.bf16_round(k * 40)
    elif kind == "ch600":
        q, k = q.copy(), k.copy()
        q[..., 7] += 600
        k[..., 7] += 600
        q, k = workloads.bf16_round(q), workloads.bf16_round(k)
    return q, k, v


@pytest.mark.parametrize("kind", ["c3", "x40", "ch600", "plain"])
def test_exponent_step_is_the_exact_value_rounded_once(kind):
    q, k, v = _stress_inputs(kind, 200, seed=41)
    rows = np.array([0, 5, 31, 32, 77, 150, 199])
    assert _exponent_mismatches(q, k, v, SCALE, 128, rows) == 0


def test_planted_exponent_mistakes_fail_the_pins(monkeypatch):
    q, k, v = _stress_inputs("x40", 200, seed=41)
    rows = np.array([0, 5, 77, 199])

    def two_roundings(A, f, m2):          # fl32(fl32(A f) - m2)
        t = oatt.f32(A.astype(np.float64) * f.astype(np.float64))
        return oatt.f32(t.astype(np.float64) - np.asarray(m2, np.float64)[:, None])

    bias = 3 * 2 ** 22

    def biased(A, f, m2):                 # accumulator biased by 1.5 * 2^23
        X = (A + bias).astype(np.float64)
        C = ((np.float32(bias) * f).astype(np.float32) + np.asarray(m2, np.float32)[:, None]).astype(np.float32)
        return oatt.f32(X * f.astype(np.float64) - C.astype(np.float64))

    for mistake in (two_roundings, biased):
        monkeypatch.setattr(oatt, "exponent_arg", mistake)
        assert _exponent_mismatches(q, k, v, SCALE, 128, rows) > 0, mistake.__name__


def _plain_order_attention(q, k, v, scale, bn):
    """Vectorized evaluation of the method in its plain step order (see
    _scalar_method), for one head; written separately from the oracle."""
    q8, qs = quant_qk(q)
    k8, ks = quant_qk(k)
    v8, vs = quant_v(v)
    q8, qs, k8, ks, v8, vs = q8[0, 0], qs[0, 0], k8[0, 0], ks[0, 0], v8[0, 0], vs[0, 0]
    S = k8.shape[0]
    A = q8.astype(np.int64) @ k8.astype(np.int64).T
    c = np.float32(np.float32(scale) * np.float32(math.log2(math.e)))
    f = ((qs[:, None] * ks[None, :]).astype(np.float32) * c).astype(np.float32)[np.arange(S) // 32][:, np.arange(S) // 32]
    t = (A.astype(np.float64) * f.astype(np.float64)).astype(np.float32)
    vals = fp8_e4m3fn_decode(v8)
    R = A.shape[0]
    m = np.full(R, -np.inf, dtype=np.float32)
    l = np.zeros(R)
    acc = np.zeros((R, vals.shape[1]))
    for j0 in range(0, S, bn):
        tt = t[:, j0:j0 + bn]
        m_new = np.maximum(m, tt.max(axis=1))
        w = np.where(np.isinf(m), 0.0, np.exp2(m.astype(np.float64) - m_new.astype(np.float64)))
        pt = np.exp2((tt - m_new[:, None]).astype(np.float32).astype(np.float64)).astype(np.float32)
        p8 = fp8_e4m3fn_decode(fp8_e4m3fn_encode((np.float32(448.0) * pt).astype(np.float32)))
        l = l * w + p8.sum(axis=1) / 448.0
        acc = acc * w[:, None] + p8 @ vals[j0:j0 + bn]
        m = m_new
    out = acc * vs.astype(np.float64)[None, :] / (448.0 * l[:, None])
    return oatt.bf16_round_f64(out)


@pytest.mark.parametrize("kind", ["c3", "x40", "ch600"])
def test_plain_step_order_within_tolerance_on_large_magnitudes(kind, monkeypatch):
    q, k, v = _stress_inputs(kind, 768, seed=43)
    ref = sage_attention(q, k, v, SCALE, 128)[0, :, 0]
    plain = _plain_order_attention(q, k, v, SCALE, 128)
    assert _gate_ratio(plain, ref) <= 0.75
    assert _cos(plain, ref) >= 0.99999
