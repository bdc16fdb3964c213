"""Quantization of Q/K (INT8 per 32-row block) and V (FP8 per channel).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: diffusers issue #15014, "gfx1201 (RDNA4) SageAttention attention
backend: aiter package or Hub kernel?", problem statement: the kernel itself
gives Q and K one INT8 scale per block of 32 rows and V one FP8 scale per
channel, feeding an INT8 QK^T and an FP8 PV. InvokeAI PR #9657, section "How it works": no K smoothing.

Readings taken where the pages are silent:

* a "32-row block" is 32 consecutive sequence positions of one (batch, head);
  the last block of a sequence may be shorter and its amax covers only its
  valid rows;
* INT8 is symmetric: scale = amax / 127 and q = clamp(rint(x * (127/amax)),
  -127, 127), with both fp32 operations correctly rounded (one rounding each)
  and rint rounding half to even; -128 is never produced;
* V maps its per-channel amax (over the whole sequence) to 448, the largest
  E4M3FN value: v_scale = amax/448, v8 = E4M3FN(fl32(v * (448/amax)));
* amax = 0 or a non-finite reciprocal gives scale 0 and all-zero codes.

K smoothing (``k_mean``, ``quant_k_smooth``) is the option InvokeAI PR #9657
measures on and off (sections "How it works" and "QA Instructions"); the
pages do not define it. Reading: K - mean_s(K) per (batch, head, channel),
quantized like K, where the mean is the exact mean of the (bf16) values
rounded once to fp32, so that it and the INT8 codes are unique.
"""
from __future__ import annotations

import numpy as np

from fractions import Fraction

from .formats import fp8_e4m3fn_encode, round_fraction_to_f32

QK_BLOCK = 32
INT8_MAX = np.float32(127.0)
FP8_MAX = np.float32(448.0)


def _scale_and_inverse(amax: np.ndarray, qmax: np.float32):
    """(scale, inverse) in fp32 from an fp32 amax: amax/qmax and qmax/amax."""
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = (qmax / amax).astype(np.float32)          # one fp32 division
        scale = (amax / qmax).astype(np.float32)        # one fp32 division
    ok = (amax > 0) & np.isfinite(inv)
    inv = np.where(ok, inv, np.float32(0)).astype(np.float32)
    scale = np.where(ok, scale, np.float32(0)).astype(np.float32)
    return scale, inv


def quant_qk(x: np.ndarray):
    """INT8 per-(b, h, 32-row block) quantization of Q or K.

    x: float32 [B, S, H, D] holding bfloat16 values.
    Returns (q8 int8 [B, H, S, D], scale float32 [B, H, ceil(S/32)]).
    """
    x = np.asarray(x, dtype=np.float32)
    B, S, H, D = x.shape
    nb = (S + QK_BLOCK - 1) // QK_BLOCK
    q8 = np.empty((B, H, S, D), dtype=np.int8)
    scales = np.empty((B, H, nb), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            xh = x[b, :, h, :]                            # [S, D]
            for t in range(nb):
                r0, r1 = t * QK_BLOCK, min(S, (t + 1) * QK_BLOCK)
                blk = xh[r0:r1]
                amax = np.max(np.abs(blk))                # exact
                scale, inv = _scale_and_inverse(amax, INT8_MAX)
                y = (blk * inv).astype(np.float32)        # fl32(x * inv)
                q = np.clip(np.rint(y), -127, 127)        # half to even
                q8[b, h, r0:r1] = q.astype(np.int8)
                scales[b, h, t] = scale
    return q8, scales


def quant_v(v: np.ndarray):
    """FP8 E4M3FN per-(b, h, channel) quantization of V, amax over all of S.

    v: float32 [B, S, H, D] holding bfloat16 values.
    Returns (v8 uint8 codes [B, H, S, D] in natural key order,
             v_scale float32 [B, H, D]).
    """
    v = np.asarray(v, dtype=np.float32)
    B, S, H, D = v.shape
    v8 = np.empty((B, H, S, D), dtype=np.uint8)
    vscale = np.empty((B, H, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            vh = v[b, :, h, :]                            # [S, D]
            amax = np.max(np.abs(vh), axis=0)             # per channel, exact
            scale, inv = _scale_and_inverse(amax, FP8_MAX)
            y = (vh * inv[None, :]).astype(np.float32)    # fl32(v * inv)
            v8[b, h] = fp8_e4m3fn_encode(y)
            vscale[b, h] = scale
    return v8, vscale


def _exact_sums(x: np.ndarray):
    """Exact sums along axis 1 of a float32 [C, S] array, as (num, e): the
    sum of row c is num[c] * 2^e[c] with Python integers num[c].

    Every float32 value is M * 2^E with an integer |M| < 2^24; the values of
    a row are brought to the row's smallest E and added as integers (int64
    when the shifted magnitudes cannot overflow it, Python integers
    otherwise), so no rounding happens anywhere.
    """
    x = np.asarray(x, dtype=np.float64)
    C, S = x.shape
    mant, ex = np.frexp(x)
    M = np.rint(mant * 2.0 ** 24).astype(np.int64)      # exact
    E = ex.astype(np.int64) - 24
    E = np.where(M == 0, np.iinfo(np.int64).max, E)
    E0 = E.min(axis=1)
    E0 = np.where(E0 == np.iinfo(np.int64).max, 0, E0)
    shift = np.where(M == 0, 0, E - E0[:, None])
    headroom = 62 - 24 - int(np.ceil(np.log2(max(S, 2))))
    nums = []
    for c in range(C):
        if shift[c].max() <= headroom:
            nums.append(int(np.sum(M[c] << shift[c])))
        else:
            nums.append(sum(int(m) << int(s) for m, s in zip(M[c], shift[c])))
    return nums, [int(e) for e in E0]


def k_mean(k: np.ndarray) -> np.ndarray:
    """Per-(b, h, channel) mean of K over the sequence: the exact mean of the
    values, rounded once to fp32 (nearest, ties to even).

    k: float32 [B, S, H, D] holding bfloat16 values. Returns float32 [B, H, D].
    """
    k = np.asarray(k, dtype=np.float32)
    B, S, H, D = k.shape
    rows = np.ascontiguousarray(k.transpose(0, 2, 3, 1)).reshape(B * H * D, S)
    nums, exps = _exact_sums(rows)
    out = np.empty(B * H * D, dtype=np.float32)
    for c, (n, e) in enumerate(zip(nums, exps)):
        out[c] = round_fraction_to_f32(Fraction(n) * Fraction(2) ** e / S)
    return out.reshape(B, H, D)


def quant_k_smooth(k: np.ndarray):
    """K smoothing then INT8 quantization: quant_qk(fl32(k - k_mean(k))).

    Returns (k8 int8 [B, H, S, D], scale float32 [B, H, ceil(S/32)],
             mean float32 [B, H, D]).
    """
    k = np.asarray(k, dtype=np.float32)
    mean = k_mean(k)
    smoothed = (k - mean[:, None, :, :]).astype(np.float32)   # fl32(k - mean)
    k8, scales = quant_qk(smoothed)
    return k8, scales, mean
