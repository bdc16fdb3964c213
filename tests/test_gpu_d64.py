"""GPU parity for head dim 64 (the VAE's head dim, a fallback cause the
pages name), through the C ABI, against the CPU oracle: quantized codes,
scales and K means bit-exact; outputs and LSE within the gates of
test_gpu_parity / test_gpu_ext. Inputs are the recipes' first 64 channels.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
sage = pytest.importorskip("quantized_attention_quant_amd")
from gpu_common import DEV, check_p_codes_and_models, gate, kappa, lse_gate, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu
D = 64
SCALE = 1.0 / math.sqrt(D)


_say = say


def d64(x):
    return np.ascontiguousarray(x[..., :D])


@pytest.mark.parametrize("S", [1, 33, 300, 1000])
def test_quant_bit_exact_d64(S):
    _say(f"quant D=64 S={S}")
    q, k, v = workloads.generate(3, S=S, H=3, B=1, seed=40 + S)
    q, k, v = d64(q), d64(k), d64(v)
    Sp = sage.sage_seq_pad(S)
    q8, qs = sage.sage_quant_qk(to_dev(q))
    k8, ks, km = sage.sage_quant_k_smooth(to_dev(k))
    vt, vs = sage.sage_quant_v(to_dev(v))
    torch.cuda.synchronize()
    r8, rs = oracle.quant_qk(q)
    assert np.array_equal(q8.cpu().numpy()[:, :, :S], r8)
    assert np.all(q8.cpu().numpy()[:, :, S:] == 0)
    nb = (S + 31) // 32
    assert np.array_equal(qs.cpu().numpy()[:, :, :nb], rs)
    s8, ss, sm = oracle.quant_k_smooth(k)
    assert np.array_equal(km.cpu().numpy(), sm)
    assert np.array_equal(k8.cpu().numpy()[:, :, :S], s8)
    assert np.array_equal(ks.cpu().numpy()[:, :, :nb], ss)
    v8, vsr = oracle.quant_v(v)
    gt = vt.cpu().numpy()                                   # [B, H, 64, S_pad] permuted
    perm = np.empty(Sp, dtype=np.int64)
    for w in range(Sp // 64):
        for p in range(64):
            perm[w * 64 + kappa(p)] = w * 64 + p
    nat = np.transpose(gt[:, :, :, perm], (0, 1, 3, 2))
    assert np.array_equal(nat[:, :, :S], v8)
    assert np.all(nat[:, :, S:] == 0)
    assert np.array_equal(vs.cpu().numpy(), vsr)


@pytest.mark.parametrize("idx,Sq,Skv,H", [(1, 256, 256, 2), (3, 129, 129, 2), (2, 300, 77, 3), (5, 64, 1000, 2),
                                          (3, 600, 600, 1), (3, 200, 512, 1), (2, 100, 700, 1)])
def test_attention_d64_full_compare(idx, Sq, Skv, H):
    _say(f"attention D=64 config {idx} Sq={Sq} Skv={Skv} H={H}")
    q, _, _ = workloads.generate(idx, S=Sq, H=H, B=1, seed=60 + Sq)
    _, k, v = workloads.generate(idx, S=Skv, H=H, B=1, seed=1060 + Skv)
    q, k, v = d64(q), d64(k), d64(v)
    out, lse = sage.sage_attention_ex(to_dev(q), to_dev(k), to_dev(v), SCALE, return_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.sage_attention(q, k, v, SCALE, sage.sage_kv_tile(), return_lse=True)
    ex = oracle.exact_attention_fp64(q, k, v, SCALE)
    gate(out.float().cpu().numpy(), ref, ex, f"Sq={Sq} Skv={Skv}")
    lse_gate(lse.cpu().numpy(), rlse, f"Sq={Sq} Skv={Skv}")


def test_attention_d64_split_equals_one_shot():
    _say("D=64 split entry points vs one-shot")
    q, k, v = workloads.generate(2, S=700, H=2, B=1, seed=8)
    q, k, v = d64(q), d64(k), d64(v)
    q8, qs = sage.sage_quant_qk(to_dev(q))
    k8, ks = sage.sage_quant_qk(to_dev(k))
    v8, vs = sage.sage_quant_v(to_dev(v))
    a = sage.sage_attn_fwd(q8, qs, k8, ks, v8, vs, 1, 700, 2, D, SCALE)
    b = sage.sage_attention(to_dev(q), to_dev(k), to_dev(v), SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attention_d64_large_sampled():
    """B=1, S=16384, H=8, D=64 (a VAE-like 128x128 latent) in one call;
    first, last and random rows of three heads against the oracle."""
    _say("attention D=64 at S=16384 H=8; generating inputs")
    S, H = 16384, 8
    q, k, v = workloads.generate(3, S=S, H=H, B=1, seed=99)
    q, k, v = d64(q), d64(k), d64(v)
    out = sage.sage_attention(to_dev(q), to_dev(k), to_dev(v), SCALE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for h in (0, H - 1, int(rng.integers(H))):
        rows = np.unique(np.concatenate([np.arange(32), np.arange(S - 32, S), rng.choice(S, 512, replace=False)]))
        sl = lambda x: np.ascontiguousarray(x[:, :, h:h + 1, :])  # noqa: E731
        q8, qs = oracle.quant_qk(sl(q))
        k8, ks = oracle.quant_qk(sl(k))
        v8, vs = oracle.quant_v(sl(v))
        ref = oracle.attention_head(q8[0, 0], qs[0, 0], k8[0, 0], ks[0, 0], v8[0, 0], vs[0, 0], SCALE,
                                    sage.sage_kv_tile(), rows=rows)
        g = out[0, torch.as_tensor(rows, device=DEV), h, :].float().cpu().numpy()
        qh = q[0, rows, h, :].astype(np.float64)
        s = qh @ k[0, :, h, :].astype(np.float64).T * SCALE
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        ex = (p @ v[0, :, h, :].astype(np.float64)) / p.sum(axis=1, keepdims=True)
        gate(g, ref, ex, f"head {h} rows={len(rows)}")


def test_debug_scores_d64():
    _say("debug scores D=64")
    q, k, _ = workloads.generate(2, S=700, H=2, B=1, seed=55)
    q, k = d64(q), d64(k)
    q8, _ = sage.sage_quant_qk(to_dev(q))
    k8, _ = sage.sage_quant_qk(to_dev(k))
    oq, _ = oracle.quant_qk(q)
    ok, _ = oracle.quant_qk(k)
    for (r0, nr, c0, nc) in [(0, 700, 0, 700), (250, 33, 600, 100)]:
        got = sage.sage_debug_qk_scores(q8, k8, 1, 700, 2, 0, 1, r0, nr, c0, nc, D=D)
        torch.cuda.synchronize()
        ref = oracle.qk_scores(oq[0, 1], ok[0, 1])[r0:r0 + nr, c0:c0 + nc]
        assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("idx,S", [(3, 16384), (5, 4000)])
def test_p_codes_and_models_d64(idx, S):
    """Head dim 64 at a large S: the FP8 codes of P, the LSE and the output of
    one head against the oracle's tile loop and the FP8 MFMA model, on sampled
    rows (gpu_common.check_p_codes_and_models)."""
    say(f"D=64 P codes and models, recipe {idx}, S={S}: generating inputs")
    q, k, v = workloads.generate(idx, S=S, H=1, B=1, seed=990 + S)
    q, k, v = (np.ascontiguousarray(x[..., :64]) for x in (q, k, v))
    check_p_codes_and_models(q, k, v, 1.0 / math.sqrt(64), np.random.default_rng(idx), f"D=64 recipe {idx}")
