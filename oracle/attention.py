"""Quantized attention forward: scores, online softmax, FP8 P, PV, epilogue.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: diffusers issue #15014, "gfx1201 (RDNA4) SageAttention attention
backend: aiter package or Hub kernel?", problem statement: QK^T on INT8 codes
and PV on FP8 codes, each summed in fp32, over bf16 [B, S, H, 128] inputs
without a mask or causality,
operation ``gfx1201_sage_attention(q, k, v, softmax_scale)``; diffusers PR
#15060, "What does this PR do?": no LSE is returned.

The method is an approximation, so this module follows its steps rather than
exact attention (``exact_attention_fp64`` is the separate exact reference).
Readings taken where the pages are silent, in step order:

1. Scores A = q8 . k8^T are exact integers (|A| <= 128*127^2 < 2^24).
2. Dequantization in the log2 domain: c = fl32(fl32(softmax_scale) *
   fl32(log2 e)), f = fl32(fl32(q_scale * k_scale) * c) per (query block,
   key block), t = fl32(A * f).
3. Online softmax over consecutive key tiles of ``bn`` keys, in key order (a
   flash-style forward streams K/V tiles; the tile width is the kernel's and
   is passed in). Per query row and tile tau:
   m_tau = max(m_{tau-1}, max_{j in tau} t_j)  (m_0 = -inf).
4. P with the fixed 448 scale, folded into the exponent: m2_tau =
   fl32(m_tau - fl32(log2 448)); arg_j = fl32(A_j * f - m2_tau), the exact
   real value rounded once (one fused multiply-add: the fp32 evaluation with
   the fewest roundings; the two-step fl32(t_j - m2_tau) differs from it by
   at most half an ulp of t_j); P'_j = fl32(2^arg_j), so P'_j = 448 *
   2^(t_j - m_tau) up to rounding. p8_j = E4M3FN(P'_j) (saturating at 448).
   The row sum l accumulates the decoded codes dec(p8_j): the normalizer is
   the sum of the very weights that multiply V, so the quantized weights of a
   row sum to one (the fp32 P'_j would leave them off by the FP8 rounding
   noise). Diffusers issue #15014 (problem statement) fixes only that the
   softmax runs in fp32, not which of the two sums normalizes.
5. Across tiles, partial sums are combined with the factors 2^(m2_tau -
   m2_T) of the final tile T (here in float64; a kernel rescales its fp32
   accumulators as it goes, which agrees to fp32 rounding).
6. PV: acc[c] = sum_j dec(p8_j) * dec(v8[j, c]); products of two FP8 values
   are exact. Epilogue: O[c] = bf16(acc[c] * v_scale[c] / l), formed in
   float64 and rounded once.

Step 4's fused multiply-add is evaluated in float64: A * f is exact there (at
most 21 + 24 significant bits), and so is the subtraction of m2 unless |m2|
exceeds |A * f| by more than a factor 2^8; then the float64 result is rounded
a second time to fp32, which differs from a single rounding only when the
float64 value lands exactly on an fp32 midpoint. ``exponent_arg`` holds this
step alone.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_round_f64, f32, fp8_e4m3fn_decode, fp8_e4m3fn_encode
from .quant import QK_BLOCK, quant_k_smooth, quant_qk, quant_v

LOG2E = np.float32(math.log2(math.e))
LOG2_448 = np.float32(math.log2(448.0))


def exp2_scale(softmax_scale: float) -> np.float32:
    """c = fl32(fl32(softmax_scale) * fl32(log2 e)): scores to the log2 domain."""
    return (np.float32(softmax_scale) * LOG2E).astype(np.float32)


def qk_scores(q8: np.ndarray, k8: np.ndarray) -> np.ndarray:
    """Exact integer scores A = q8 . k8^T as int64.

    Computed by a float64 matrix product: every partial sum is an integer of
    magnitude below 2^53, so the product is exact in any summation order.
    """
    a = np.asarray(q8, dtype=np.float64) @ np.asarray(k8, dtype=np.float64).T
    return a.astype(np.int64)


def _combine(shifts, l_parts, acc_parts, D, with_shift=False):
    """Sum per-tile partials with factors 2^(shift_tau - shift_T) (float64).

    Returns (acc, l), or (acc, l, shift_T) with ``with_shift``."""
    final = shifts[-1]
    l = np.zeros(len(final))
    acc = np.zeros((len(final), D))
    for shift, l_t, acc_t in zip(shifts, l_parts, acc_parts):
        w = np.exp2(shift - final)
        l += w * l_t
        acc += w[:, None] * acc_t
    return (acc, l, final) if with_shift else (acc, l)


def exponent_arg(A, f, m2):
    """Step 4's exponent: fl32(A * f - m2) with one rounding.

    A: int64 [R, n] scores; f: float32 [R, n] factors; m2: fp32 values [R].
    """
    x = np.asarray(A, dtype=np.int64).astype(np.float64) * np.asarray(f, dtype=np.float32).astype(np.float64)
    return f32(x - np.asarray(m2, dtype=np.float32).astype(np.float64)[:, None])


def online_softmax_pv(A, f, vals, bn: int, n_valid: int | None = None, with_shift: bool = False,
                      trace: list | None = None):
    """Steps 2-5 for a set of query rows: the method's tile-scheduled online
    softmax with FP8 P, followed by PV.

    A:    int64 [R, S] exact integer scores.
    f:    float32 [R, S] dequantization factor of each (row, key) pair.
    vals: float64 [S, D] decoded FP8 V values (natural key order).
    bn:   key tile width; keys at index >= n_valid are masked.
    Returns (acc float64 [R, D], l float64 [R]); the output is
    acc * v_scale / l, with l = sum_j dec(p8_j) 2^(m2_tau(j) - m2_T). With
    ``with_shift`` also m2 of the last tile (float64 holding fp32 values):
    l = sum_j 2^(t_j - m2_T) up to the FP8 rounding of each term. With a
    ``trace`` list, one dict per tile (j0, j1, m2, arg, p, p8) is appended
    to it (used by the tests that pin the exponent step).
    """
    A = np.asarray(A, dtype=np.int64)
    f = np.asarray(f, dtype=np.float32)
    R, S = A.shape
    if n_valid is None:
        n_valid = S
    x = A.astype(np.float64) * f.astype(np.float64)     # A * f, exact
    m_prev = np.full(R, -np.inf)
    shifts, l_parts, acc_parts = [], [], []
    for j0 in range(0, min(S, n_valid), bn):
        j1 = min(S, n_valid, j0 + bn)
        t = f32(x[:, j0:j1])                             # fl32(A * f)
        m = np.maximum(m_prev, t.max(axis=1).astype(np.float64))
        m2 = (m.astype(np.float32) - LOG2_448).astype(np.float32)
        arg = exponent_arg(A[:, j0:j1], f[:, j0:j1], m2)  # fl32(A * f - m2)
        p = f32(np.exp2(arg.astype(np.float64)))         # P' in fp32
        p8 = fp8_e4m3fn_encode(p)
        p_used = fp8_e4m3fn_decode(p8)                   # dec(E4M3FN(P'))
        if trace is not None:
            trace.append(dict(j0=j0, j1=j1, m2=m2, arg=arg, p=p, p8=p8))
        shifts.append(m2.astype(np.float64))
        l_parts.append(p_used.sum(axis=1))
        acc_parts.append(p_used @ np.asarray(vals[j0:j1], dtype=np.float64))
        m_prev = m
    return _combine(shifts, l_parts, acc_parts, vals.shape[1], with_shift)


def online_softmax_exact(x, vals, bn: int, n_valid: int | None = None):
    """The same tile loop with quantization switched off: float64 scores x
    (already in the log2 domain), P = 2^(x - m) with no rounding or encoding.
    Used to pin the running-max bookkeeping against textbook softmax.
    Returns (acc, l) with output acc / l."""
    x = np.asarray(x, dtype=np.float64)
    R, S = x.shape
    if n_valid is None:
        n_valid = S
    m_prev = np.full(R, -np.inf)
    shifts, l_parts, acc_parts = [], [], []
    for j0 in range(0, min(S, n_valid), bn):
        j1 = min(S, n_valid, j0 + bn)
        xt = x[:, j0:j1]
        m = np.maximum(m_prev, xt.max(axis=1))
        p = np.exp2(xt - m[:, None])
        shifts.append(m)
        l_parts.append(p.sum(axis=1))
        acc_parts.append(p @ np.asarray(vals[j0:j1], dtype=np.float64))
        m_prev = m
    return _combine(shifts, l_parts, acc_parts, vals.shape[1])


def lse_from_state(m2_final, l):
    """Log-sum-exp of a row's scaled scores from the online-softmax state.

    l = sum_j 2^(t_j - m2_T) up to the FP8 rounding of each term (l sums the
    decoded codes), with t_j = softmax_scale * log2(e) * score_j, so
    ln sum_j exp(softmax_scale * score_j) = ln 2 * (m2_T + log2 l). Formed in
    float64 and rounded once to fp32 (the output type). Reading: the pages
    only say that ring attention needs the LSE (diffusers PR #15060, "What
    does this PR do?"); natural log, per query row, of the scaled dequantized
    scores.
    """
    m2_final = np.asarray(m2_final, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    return f32(math.log(2.0) * (m2_final + np.log2(l)))


def attention_head(q8, q_scale, k8, k_scale, v8, v_scale, softmax_scale, bn,
                   rows=None, n_valid=None, return_f64=False, return_lse=False):
    """Quantized attention output for one (batch, head).

    q8: int8 [Sq, D], q_scale: fp32 [ceil(Sq/32)]; k8: int8 [Skv, D],
    k_scale: fp32 [ceil(Skv/32)]; v8: uint8 E4M3FN codes [Skv, D] (natural
    key order); v_scale: fp32 [D]. Sq and Skv may differ (cross-attention).
    rows: query indices to compute (default: all).
    Returns bf16-valued float32 [len(rows), D]; with ``return_f64`` also the
    float64 value before the final rounding; with ``return_lse`` also the
    fp32 log-sum-exp of each row (``lse_from_state``).
    """
    S = k8.shape[0]
    if rows is None:
        rows = np.arange(q8.shape[0])
    rows = np.asarray(rows)
    c = exp2_scale(softmax_scale)
    A = qk_scores(q8[rows], k8)                                  # [R, Skv] exact
    f_blocks = f32(f32(q_scale[rows // QK_BLOCK][:, None].astype(np.float32)
                       * k_scale[None, :].astype(np.float32)) * c)  # [R, nbk]
    f_keys = f_blocks[:, np.arange(S) // QK_BLOCK]               # [R, Skv] fp32
    vals = fp8_e4m3fn_decode(v8)
    acc, l, m2_final = online_softmax_pv(A, f_keys, vals, bn, n_valid=n_valid, with_shift=True)
    o64 = acc * np.asarray(v_scale, dtype=np.float64)[None, :] / l[:, None]
    o = bf16_round_f64(o64)
    res = [o]
    if return_f64:
        res.append(o64)
    if return_lse:
        res.append(lse_from_state(m2_final, l))
    return tuple(res) if len(res) > 1 else o


def sage_attention(q, k, v, softmax_scale, bn, rows=None, heads=None, smooth_k=False, return_lse=False):
    """Whole method on bf16-valued float32 inputs: q [B, Sq, H, D], k and v
    [B, Skv, H, D] (Sq = Skv for the pages' operation; they may differ for
    cross-attention). ``smooth_k`` quantizes K with ``quant_k_smooth``.

    Returns O as float32 [B, Sq, H, D] holding bf16 values (and, with
    ``return_lse``, the fp32 log-sum-exp [B, H, Sq]). With ``rows`` (query
    indices) and/or ``heads`` (list of (b, h)), only those are computed and
    the rest is NaN.
    """
    B, Sq, H, D = q.shape
    q8, qs = quant_qk(q)
    if smooth_k:
        k8, ks, _ = quant_k_smooth(k)
    else:
        k8, ks = quant_qk(k)
    v8, vs = quant_v(v)
    out = np.full((B, Sq, H, D), np.nan, dtype=np.float32)
    lse = np.full((B, H, Sq), np.nan, dtype=np.float32)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    rws = np.arange(Sq) if rows is None else np.asarray(rows)
    for b, h in pairs:
        o, ls = attention_head(q8[b, h], qs[b, h], k8[b, h], ks[b, h], v8[b, h], vs[b, h],
                               softmax_scale, bn, rows=rws, return_lse=True)
        out[b, rws, h, :] = o
        lse[b, h, rws] = ls
    return (out, lse) if return_lse else out


def exact_attention_fp64(q, k, v, softmax_scale, return_lse=False):
    """Textbook softmax(q k^T * scale) v per (b, h), in float64.

    q [B, Sq, H, D], k and v [B, Skv, H, D]; returns [B, Sq, H, D] (and, with
    ``return_lse``, ln sum_j exp(scale * q.k_j) as float64 [B, H, Sq])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    out = np.empty((B, Sq, H, D))
    lse = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k[b, :, h, :].T) * softmax_scale
            mx = s.max(axis=1, keepdims=True)
            p = np.exp(s - mx)
            den = p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (p @ v[b, :, h, :]) / den
            lse[b, h] = (mx + np.log(den))[:, 0]
    return (out, lse) if return_lse else out
