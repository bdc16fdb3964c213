"""GPU parity at the full sizes of the image- and video-DiT workloads, in the
launch configuration the benchmark times (sage_quant_kv for K and V, the
attention kernel quantizing Q itself), against the CPU oracle on samples it
can compute one by one:

* INT8 Q/K codes and scales and FP8 V codes and scales of whole sampled
  heads, bit-exact;
* int32 scores of sampled 128 x 128 windows (first, last with the ragged
  tail, random) through the attention kernel's staging and MFMA path,
  bit-exact;
* the output on sampled query rows (first, last and random 32-row blocks plus
  random rows of three heads), with the stated output gates, and the
  log-sum-exp of the same rows.

The tests take their inputs from a module-scoped fixture with one parameter
per workload, so pytest runs all tests of one workload before generating the
next, and keeps the inputs of one workload at a time.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
sage = pytest.importorskip("quantized_attention_quant_amd")
from gpu_common import (DEV, check_p_codes_and_models, exact_rows, gate, lse_gate, oracle_rows, say,  # noqa: E402
                        to_dev, unpermute_vt)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=[2, 3, 4, 5])
def workload(request):
    """(index, host inputs as bf16-valued float32, their device copies)."""
    idx = request.param
    say(f"  generating the inputs of workload {idx} ({workloads.config(idx).name})")
    q, k, v = workloads.generate(idx, chunk_elems=1 << 26)
    yield idx, (q, k, v), (to_dev(q), to_dev(k), to_dev(v))


def _heads(cfg, seed):
    rng = np.random.default_rng(seed)
    return [(0, 0), (cfg.B - 1, cfg.H - 1), (int(rng.integers(cfg.B)), int(rng.integers(cfg.H)))]


def _head(x, b, h):
    return np.ascontiguousarray(x[b:b + 1, :, h:h + 1, :])


def test_quantizers_bit_exact_on_sampled_heads(workload):
    idx, (q, k, v), (qd, kd, vd) = workload
    cfg = workloads.config(idx)
    say(f"quantizers at full size, workload {idx}")
    q8, qs = sage.sage_quant_qk(qd)
    k8, ks, v8, vs = sage.sage_quant_kv(kd, vd)
    torch.cuda.synchronize()
    nb = (cfg.S + 31) // 32
    for b, h in _heads(cfg, 10 + idx):
        for name, x, g8, gs in (("Q", q, q8, qs), ("K", k, k8, ks)):
            r8, rs = oracle.quant_qk(_head(x, b, h))
            assert np.array_equal(g8[b, h, :cfg.S].cpu().numpy(), r8[0, 0]), (name, b, h)
            assert np.all(g8[b, h, cfg.S:].cpu().numpy() == 0), (name, b, h)
            assert np.array_equal(gs[b, h, :nb].cpu().numpy().view(np.uint32), rs[0, 0].view(np.uint32)), (name, b, h)
        rv8, rvs = oracle.quant_v(_head(v, b, h))
        gv = unpermute_vt(v8[b:b + 1, h:h + 1].cpu().numpy(), cfg.S)
        assert np.array_equal(gv, rv8), (b, h)
        assert np.array_equal(vs[b, h].cpu().numpy().view(np.uint32), rvs[0, 0].view(np.uint32)), (b, h)
        say(f"  (b,h)=({b},{h}): Q/K codes and scales, V codes and scales bit-exact over S={cfg.S}")


def test_scores_bit_exact_on_sampled_windows(workload):
    idx, (q, k, _), (qd, kd, _) = workload
    cfg = workloads.config(idx)
    say(f"int32 score windows at full size, workload {idx}")
    q8, _ = sage.sage_quant_qk(qd)
    k8, _ = sage.sage_quant_qk(kd)
    rng = np.random.default_rng(20 + idx)
    S, n = cfg.S, 128
    for b, h in _heads(cfg, 10 + idx):
        oq, _ = oracle.quant_qk(_head(q, b, h))
        ok, _ = oracle.quant_qk(_head(k, b, h))
        last = (S - 1) // n * n                     # the last key tile (ragged when S % 128 != 0)
        wins = [(0, 0), (S - n, last), (int(rng.integers(S - n)), int(rng.integers(S - n)))]
        for r0, c0 in wins:
            nc = min(n, S - c0)
            got = sage.sage_debug_qk_scores(q8, k8, cfg.B, S, cfg.H, b, h, r0, n, c0, nc)
            torch.cuda.synchronize()
            ref = oracle.qk_scores(oq[0, 0][r0:r0 + n], ok[0, 0][c0:c0 + nc])
            assert np.array_equal(got.cpu().numpy(), ref), (b, h, r0, c0)
        say(f"  (b,h)=({b},{h}): windows {wins} bit-exact")


def _sample_rows(S, rng, nrand=2, nrows=1024):
    """First, last (tail) and random 32-row blocks, plus random single rows.

    Whole blocks exercise the per-block scales and the ragged tail; the
    random rows make the cosine against exact attention a stable estimate
    for the head (about a quarter of the blocks of the outlier recipe hold an
    x8 row, and those blocks are far less accurate than the rest).
    """
    nb = (S + 31) // 32
    blocks = sorted(set([0, nb - 1] + list(rng.choice(nb, nrand, replace=False))))
    rows = np.concatenate([np.arange(32 * t, min(S, 32 * t + 32)) for t in blocks]
                          + [rng.choice(S, nrows, replace=False)])
    return np.unique(rows)


def test_attention_sampled_rows_and_lse(workload):
    idx, (q, k, v), (qd, kd, vd) = workload
    cfg = workloads.config(idx)
    say(f"attention at full size, workload {idx}: one-shot sage_attention, then sage_attention_ex with the LSE")
    out = sage.sage_attention(qd, kd, vd, cfg.softmax_scale)
    out_ex, lse = sage.sage_attention_ex(qd, kd, vd, cfg.softmax_scale, return_lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    assert torch.equal(out.view(torch.int16), out_ex.view(torch.int16))
    rng = np.random.default_rng(idx)
    bn = sage.sage_kv_tile()
    for b, h in _heads(cfg, 30 + idx):
        rows = _sample_rows(cfg.S, rng)
        ti = torch.as_tensor(rows, device=DEV)
        g = out[b, ti, h, :].float().cpu().numpy()
        ref, rl = oracle_rows(q, k, v, b, h, rows, cfg.softmax_scale, bn, return_lse=True)
        ex = exact_rows(q, k, v, b, h, rows, cfg.softmax_scale)
        gate(g, ref, ex, f"workload {idx} (b,h)=({b},{h}) rows={len(rows)}")
        lse_gate(lse[b, h, ti].cpu().numpy(), rl, f"workload {idx} (b,h)=({b},{h})")


def test_p_codes_on_sampled_rows(workload):
    """The FP8 codes of P, the LSE and the output at full size, on one head
    and sampled rows, against the oracle's tile loop and the FP8 MFMA model
    (gpu_common.check_p_codes_and_models)."""
    idx, (q, k, v), _ = workload
    cfg = workloads.config(idx)
    b, h = 0, cfg.H - 1
    check_p_codes_and_models(_head(q, b, h), _head(k, b, h), _head(v, b, h), cfg.softmax_scale,
                             np.random.default_rng(70 + idx), f"workload {idx}, (b,h)=({b},{h})")
