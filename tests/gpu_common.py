"""Helpers shared by the GPU parity tests (test code only).

The output gates: max|O_gpu - O_oracle| <= 1e-2 * max|O_oracle| and cosine
>= 0.9999 against the oracle; against exact fp64 attention, cosine >= 0.99
wherever the method itself (the oracle) reaches it, and otherwise no worse
than the oracle minus 1e-4 (inputs whose quantization loses the scores, such
as a +600 Q/K channel). Every call prints its maxima, so that a log shows how
far each case is from its bound.

The LSE gate: -(ln(1 / (1 - 7 * 2^-13)) + r) <= lse_gpu - lse_oracle <= r,
with r = 4e-5 + 1e-6 |lse_oracle|. The oracle sums the decoded FP8 codes of P
exactly; the kernel sums them with an FP8 MFMA and an all-ones operand, which
within each group of 8 codes cuts every code toward zero to a multiple of
2^(E-13), E the exponent of the group's largest code (the rule is pinned in
test_gpu_fp8_mfma.py). Each group keeps more than 1 - 7 * 2^-13 of its sum, so
the kernel's l is low by at most that fraction and its LSE by at most
8.55e-4. The symmetric part r
covers the fp32 additions and rescalings along a row's chain (each 2^-24
relative: <= 2e-5 in ln l), the hardware log2 (about 1 ulp) and the final
fp32 roundings of m2 + log2 l and of the product with ln 2.
"""
import sys

import numpy as np
import torch

import oracle

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(DEV)


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def gate(got, ref, exact=None, label=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), label
    err = np.max(np.abs(got - ref))
    bound = 1e-2 * np.max(np.abs(ref))
    c = cosine(got, ref)
    msg = f"  {label}: max|err| {err:.4g} = {err / bound:.3f} x bound {bound:.4g}, cosine {c:.7f}"
    if exact is not None:
        c_gpu, c_ora = cosine(got, exact), cosine(ref, exact)
        msg += f", cos vs fp64 {c_gpu:.5f} (oracle {c_ora:.5f})"
    say(msg)
    assert err <= bound, label
    assert c >= 0.9999, label
    if exact is not None:
        if c_ora >= 0.99:
            assert c_gpu >= 0.99, label
        else:
            assert c_gpu >= c_ora - 1e-4, label


LSE_CUT = -np.log1p(-7 * 2.0 ** -13)     # the row-sum MFMA's largest loss, in ln l


def lse_gate(got, ref, label=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), label
    d = got - ref
    r = 4e-5 + 1e-6 * np.abs(ref)
    say(f"  {label}: lse - oracle in [{d.min():.3g}, {d.max():.3g}] "
        f"(bounds [-{LSE_CUT:.3g} - r, r], r <= {r.max():.3g}), mean {d.mean():.3g}")
    assert np.all(d <= r), label
    assert np.all(d >= -(LSE_CUT + r)), label


def kappa(p):
    """Key of slot p in a 64-key group of the V^T layout (include/sage.h)."""
    g, u, r = p // 32, (p // 16) % 2, p % 16
    return 32 * u + 8 * (r // 4) + 4 * g + (r % 4)


def unpermute_vt(vt, S):
    """[B,H,D,S_pad] permuted -> [B,H,S,D] natural key order."""
    B, H, D, Sp = vt.shape
    perm = np.empty(Sp, dtype=np.int64)
    for w in range(Sp // 64):
        for p in range(64):
            perm[w * 64 + kappa(p)] = w * 64 + p
    nat = vt[:, :, :, perm]
    return np.transpose(nat, (0, 1, 3, 2))[:, :, :S]


def exact_rows(q, k, v, b, h, rows, scale):
    """Exact fp64 softmax attention for the given query rows of (b, h)."""
    qh = q[b, rows, h, :].astype(np.float64)
    s = qh @ k[b, :, h, :].astype(np.float64).T * scale
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v[b, :, h, :].astype(np.float64)) / p.sum(axis=1, keepdims=True)


def oracle_rows(q, k, v, b, h, rows, scale, bn, return_lse=False):
    """The oracle's output (and LSE) for the given query rows of (b, h)."""
    sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1, :])  # noqa: E731
    q8, qs = oracle.quant_qk(sl(q))
    k8, ks = oracle.quant_qk(sl(k))
    v8, vs = oracle.quant_v(sl(v))
    return oracle.attention_head(q8[0, 0], qs[0, 0], k8[0, 0], ks[0, 0], v8[0, 0], vs[0, 0], scale, bn,
                                 rows=rows, return_lse=return_lse)
