"""GPU parity of the extensions, through the C ABI, against the CPU oracle:
K smoothing (codes, scales and the K mean bit-exact), the log-sum-exp output
and query/key sequences of different lengths (cross-attention).

Output and LSE gates as stated in gpu_common.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
sage = pytest.importorskip("quantized_attention_quant_amd")
from gpu_common import DEV, exact_rows, gate, lse_gate, oracle_rows, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu

_say = say


def cross_inputs(idx, Sq, Skv, H, seed):
    q, _, _ = workloads.generate(idx, S=Sq, H=H, B=1, seed=seed)
    _, k, v = workloads.generate(idx, S=Skv, H=H, B=1, seed=seed + 1000)
    return q, k, v


# --------------------------------------------------------------------------
# K smoothing: bit-exact codes, scales and mean

@pytest.mark.parametrize("idx,S,H", [(2, 1, 2), (2, 31, 2), (3, 33, 3), (5, 300, 2), (2, 1000, 2), (3, 4096, 2)])
def test_quant_k_smooth_bit_exact(idx, S, H):
    _say(f"quant_k_smooth config {idx} S={S} H={H}")
    k = workloads.generate(idx, S=S, H=H, B=1, seed=700 + S)[1]
    B, _, _, D = k.shape
    Sp = sage.sage_seq_pad(S)
    k8 = torch.full((B, H, Sp, D), 77, dtype=torch.int8, device=DEV)               # poison
    ks = torch.full((B, H, Sp // 32), float("nan"), dtype=torch.float32, device=DEV)
    km = torch.full((B, H, D), float("nan"), dtype=torch.float32, device=DEV)
    sage.sage_quant_k_smooth(to_dev(k), k8, ks, km)
    torch.cuda.synchronize()
    r8, rs, rm = oracle.quant_k_smooth(k)
    g8, gs, gm = k8.cpu().numpy(), ks.cpu().numpy(), km.cpu().numpy()
    assert np.array_equal(gm, rm)
    assert np.array_equal(g8[:, :, :S], r8)
    assert np.all(g8[:, :, S:] == 0)
    nb = (S + 31) // 32
    assert np.array_equal(gs[:, :, :nb].view(np.uint32), rs.view(np.uint32))
    assert np.all(gs[:, :, nb:] == 0)


def test_quant_k_smooth_full_size_sampled_heads():
    """Wan 720p shape (B=2, S=75600, H=40; S % 32 = 16): the mean of sampled
    heads and the codes of their first, last and a random block, bit-exact."""
    cfg = workloads.config(5)
    _say("quant_k_smooth at B=2 S=75600 H=40; generating inputs")
    k = workloads.generate(5, chunk_elems=1 << 26)[1]
    k8, ks, km = sage.sage_quant_k_smooth(to_dev(k))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    nb = (cfg.S + 31) // 32
    for b, h in [(0, 0), (1, 39), (int(rng.integers(2)), int(rng.integers(40)))]:
        kh = np.ascontiguousarray(k[b:b + 1, :, h:h + 1, :])
        r8, rs, rm = oracle.quant_k_smooth(kh)
        assert np.array_equal(km[b, h].cpu().numpy(), rm[0, 0]), (b, h)
        for t in (0, nb - 1, int(rng.integers(nb))):
            r0, r1 = 32 * t, min(cfg.S, 32 * t + 32)
            assert np.array_equal(k8[b, h, r0:r1].cpu().numpy(), r8[0, 0, r0:r1]), (b, h, t)
            assert ks[b, h, t].item() == rs[0, 0, t], (b, h, t)
        _say(f"  (b,h)=({b},{h}) mean and sampled blocks bit-exact")


# --------------------------------------------------------------------------
# cross-attention and LSE through the split entry points

@pytest.mark.parametrize("idx,Sq,Skv,H", [(1, 256, 256, 2), (2, 300, 77, 3), (3, 64, 700, 2),
                                          (5, 1000, 260, 2), (2, 257, 1, 2), (3, 40, 4096, 2)])
def test_attn_fwd_ex_cross_and_lse(idx, Sq, Skv, H):
    cfg = workloads.config(idx)
    _say(f"attn_fwd_ex config {idx} Sq={Sq} Skv={Skv} H={H}")
    q, k, v = cross_inputs(idx, Sq, Skv, H, seed=900 + Sq)
    q8, qs = sage.sage_quant_qk(to_dev(q))
    k8, ks = sage.sage_quant_qk(to_dev(k))
    v8, vs = sage.sage_quant_v(to_dev(v))
    out = torch.full((1, Sq, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((1, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    sage.sage_attn_fwd_ex(q8, qs, k8, ks, v8, vs, 1, Sq, Skv, H, 128, cfg.softmax_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ref, rlse = oracle.sage_attention(q, k, v, cfg.softmax_scale, sage.sage_kv_tile(), return_lse=True)
    ex = oracle.exact_attention_fp64(q, k, v, cfg.softmax_scale)
    gate(out.float().cpu().numpy(), ref, ex, f"Sq={Sq} Skv={Skv}")
    lse_gate(lse.cpu().numpy(), rlse, f"Sq={Sq} Skv={Skv}")


def _merge(parts):
    """Attention over the union of key shards from per-shard outputs and
    log-sum-exps (fp64): O = sum_i e^(lse_i) O_i / sum_i e^(lse_i)."""
    lses = np.stack([np.transpose(l.astype(np.float64), (0, 2, 1))[..., None] for _, l in parts])   # [n,B,S,H,1]
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    outs = np.stack([o.astype(np.float64) for o, _ in parts])
    return (w * outs).sum(axis=0) / w.sum(axis=0)


@pytest.mark.parametrize("idx,Sq,splits,H", [(1, 300, (384, 316), 2), (3, 200, (256, 128, 333), 2)])
def test_lse_merges_key_shards(idx, Sq, splits, H):
    """The use the LSE output exists for (ring attention): attention over K/V
    split into shards, each run on its own with its LSE, merged on the host.
    The merge of the GPU shards equals the merge of the oracle's shards
    within the output gate, and approximates exact attention over all keys."""
    cfg = workloads.config(idx)
    Skv = sum(splits)
    _say(f"LSE merge config {idx} Sq={Sq} shards={splits} H={H}")
    q, k, v = cross_inputs(idx, Sq, Skv, H, seed=1300 + Sq)
    qd = to_dev(q)
    gpu_parts, ref_parts = [], []
    j0 = 0
    for n in splits:
        ks, vs = np.ascontiguousarray(k[:, j0:j0 + n]), np.ascontiguousarray(v[:, j0:j0 + n])
        o, l = sage.sage_attention_ex(qd, to_dev(ks), to_dev(vs), cfg.softmax_scale, return_lse=True)
        torch.cuda.synchronize()
        gpu_parts.append((o.float().cpu().numpy(), l.cpu().numpy()))
        ref_parts.append(oracle.sage_attention(q, ks, vs, cfg.softmax_scale, sage.sage_kv_tile(), return_lse=True))
        j0 += n
    got, ref = _merge(gpu_parts), _merge(ref_parts)
    ex = oracle.exact_attention_fp64(q, k, v, cfg.softmax_scale)
    gate(got, ref, ex, f"merged shards {splits}")


def test_attn_fwd_ex_equal_lengths_is_attn_fwd():
    _say("attn_fwd_ex(S, S, lse=NULL) vs attn_fwd")
    q, k, v = workloads.generate(3, S=700, H=3, B=1, seed=41)
    q8, qs = sage.sage_quant_qk(to_dev(q))
    k8, ks = sage.sage_quant_qk(to_dev(k))
    v8, vs = sage.sage_quant_v(to_dev(v))
    a = sage.sage_attn_fwd(q8, qs, k8, ks, v8, vs, 1, 700, 3, 128, 0.09)
    b = sage.sage_attn_fwd_ex(q8, qs, k8, ks, v8, vs, 1, 700, 700, 3, 128, 0.09)
    c, lse = sage.sage_attn_fwd_ex(q8, qs, k8, ks, v8, vs, 1, 700, 700, 3, 128, 0.09, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    assert bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("idx,S,H,B,parts", [(2, 1000, 4, 1, 2), (5, 333, 6, 2, 3)])
def test_head_shards_are_bit_identical(idx, S, H, B, parts):
    """A head-sharded run, one GPU's share under Ulysses context parallelism
    (diffusers PR #15060, "What does this PR do?"), gives bit for bit the
    heads of the full run: every (b, h) is quantized and attended on its own
    (the Q/K blocks lie inside one head, V's scale is per (b, h, channel),
    the softmax per row), so no result depends on the other heads."""
    cfg = workloads.config(idx)
    _say(f"head shards config {idx} B={B} S={S} H={H} parts={parts}")
    q, k, v = workloads.generate(idx, S=S, H=H, B=B, seed=880 + S)
    full, lse = sage.sage_attention_ex(to_dev(q), to_dev(k), to_dev(v), cfg.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    hs = H // parts
    for p in range(parts):
        sl = slice(p * hs, (p + 1) * hs)
        qs_, ks_, vs_ = (np.ascontiguousarray(x[:, :, sl, :]) for x in (q, k, v))
        o, l = sage.sage_attention_ex(to_dev(qs_), to_dev(ks_), to_dev(vs_), cfg.softmax_scale, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, full[:, :, sl, :]), f"shard {p}: output differs"
        assert torch.equal(l, lse[:, sl, :]), f"shard {p}: LSE differs"


# --------------------------------------------------------------------------
# one-shot entry point

@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("idx,Sq,Skv,H", [(2, 333, 1000, 2), (5, 512, 77, 3)])
def test_attention_ex_one_shot(idx, Sq, Skv, H, flags):
    cfg = workloads.config(idx)
    _say(f"attention_ex config {idx} Sq={Sq} Skv={Skv} flags={flags}")
    q, k, v = cross_inputs(idx, Sq, Skv, H, seed=300 + Skv)
    out, lse = sage.sage_attention_ex(to_dev(q), to_dev(k), to_dev(v), cfg.softmax_scale, flags=flags,
                                      return_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.sage_attention(q, k, v, cfg.softmax_scale, sage.sage_kv_tile(),
                                      smooth_k=bool(flags & 1), return_lse=True)
    ex = oracle.exact_attention_fp64(q, k, v, cfg.softmax_scale)
    gate(out.float().cpu().numpy(), ref, ex, f"flags={flags}")
    lse_gate(lse.cpu().numpy(), rlse, f"flags={flags}")


# --------------------------------------------------------------------------
# Q quantized inside the attention kernel

@pytest.mark.parametrize("D,Sq,Skv,H", [(128, 1, 1, 2), (128, 33, 300, 2), (128, 1000, 1000, 3), (64, 300, 77, 2),
                                        (64, 256, 256, 1)])
def test_attn_fwd_qbf16_equals_split_path(D, Sq, Skv, H):
    _say(f"attn_fwd_qbf16 D={D} Sq={Sq} Skv={Skv} vs quant_qk + attn_fwd_ex")
    q, _, _ = workloads.generate(3, S=Sq, H=H, B=1, seed=70 + Sq)
    _, k, v = workloads.generate(3, S=Skv, H=H, B=1, seed=170 + Skv)
    q, k, v = (np.ascontiguousarray(x[..., :D]) for x in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    qd = to_dev(q)
    q8, qs = sage.sage_quant_qk(qd)
    k8, ks = sage.sage_quant_qk(to_dev(k))
    v8, vs = sage.sage_quant_v(to_dev(v))
    a, la = sage.sage_attn_fwd_ex(q8, qs, k8, ks, v8, vs, 1, Sq, Skv, H, D, scale, return_lse=True)
    b, lb = sage.sage_attn_fwd_qbf16(qd, k8, ks, v8, vs, Skv=Skv, softmax_scale=scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(la, lb)


@pytest.mark.parametrize("idx,Sq,Skv,H", [(3, 2048, 16384, 2), (5, 16384, 1000, 2)])
def test_cross_attention_large_sampled_rows(idx, Sq, Skv, H):
    """Cross-attention at large lengths (many key tiles against few query
    tiles and the reverse), through the one-shot entry point with the LSE,
    on sampled query rows against the oracle, under the stated gates."""
    cfg = workloads.config(idx)
    _say(f"large cross-attention config {idx} Sq={Sq} Skv={Skv} H={H}")
    q, k, v = cross_inputs(idx, Sq, Skv, H, seed=1300 + Sq)
    out, lse = sage.sage_attention_ex(to_dev(q), to_dev(k), to_dev(v), cfg.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(Sq + Skv)
    bn = sage.sage_kv_tile()
    for h in range(H):
        rows = np.unique(np.concatenate([np.arange(32), np.arange(Sq - 32, Sq), rng.choice(Sq, 192, replace=False)]))
        ti = torch.as_tensor(rows, device=DEV)
        got = out[0, ti, h, :].float().cpu().numpy()
        ref, rl = oracle_rows(q, k, v, 0, h, rows, cfg.softmax_scale, bn, return_lse=True)
        ex = exact_rows(q, k, v, 0, h, rows, cfg.softmax_scale)
        gate(got, ref, ex, f"cross {Sq}x{Skv} h={h} rows={len(rows)}")
        lse_gate(lse[0, h, ti].cpu().numpy(), rl, f"cross {Sq}x{Skv} h={h}")


@pytest.mark.parametrize("idx,S,H", [(2, 4096, 2), (5, 16384, 1)])
def test_smoothed_attention_large_sampled_rows(idx, S, H):
    """K smoothing in the one-shot entry point at large S, on sampled query
    rows against the oracle with smoothing, output and LSE under the stated
    gates; the recipes carry K channel offsets, the case smoothing is for."""
    cfg = workloads.config(idx)
    _say(f"smoothed attention config {idx} S={S} H={H}")
    q, k, v = workloads.generate(idx, S=S, H=H, B=1, seed=1700 + S)
    out, lse = sage.sage_attention_ex(to_dev(q), to_dev(k), to_dev(v), cfg.softmax_scale, flags=sage.SAGE_SMOOTH_K,
                                      return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(S)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(S - 32, S), rng.choice(S, 192, replace=False)]))
    ref, rl = oracle.sage_attention(q, k, v, cfg.softmax_scale, sage.sage_kv_tile(), rows=rows, smooth_k=True,
                                    return_lse=True)
    ti = torch.as_tensor(rows, device=DEV)
    for h in range(H):
        got = out[0, ti, h, :].float().cpu().numpy()
        ex = exact_rows(q, k, v, 0, h, rows, cfg.softmax_scale)
        gate(got, ref[0, rows, h, :], ex, f"smoothed S={S} h={h} rows={len(rows)}")
        lse_gate(lse[0, h, ti].cpu().numpy(), rl[0, h, rows], f"smoothed S={S} h={h}")
