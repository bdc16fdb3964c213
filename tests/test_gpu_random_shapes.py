"""GPU parity on seeded random combinations of the supported shapes, against
the CPU oracle: batch, heads, query and key lengths (equal or not, ragged
against the 32-row blocks and the 128-key tiles), head dim 64 or 128, every
input recipe, with and without K smoothing. Each case goes through the
one-shot entry point with the log-sum-exp and is held to the output and LSE
gates of gpu_common; the fixed cases elsewhere pin each feature alone, these
mix them.
"""
import math

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
sage = pytest.importorskip("quantized_attention_quant_amd")
from gpu_common import gate, lse_gate, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        Sq = int(rng.integers(1, 1201))
        Skv = Sq if rng.random() < 0.5 else int(rng.integers(1, 1201))
        D = int(rng.choice([64, 128]))
        idx = int(rng.integers(1, 6))
        smooth = bool(rng.random() < 0.3)
        out.append((i, idx, B, H, Sq, Skv, D, smooth))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"c{c[0]}-w{c[1]}-B{c[2]}H{c[3]}-{c[4]}x{c[5]}-D{c[6]}"
                                             + ("-smooth" if c[7] else "") for c in CASES])
def test_random_shape_parity(case):
    i, idx, B, H, Sq, Skv, D, smooth = case
    say(f"random case {i}: workload recipe {idx}, B={B} H={H} Sq={Sq} Skv={Skv} D={D} smooth={smooth}")
    q, _, _ = workloads.generate(idx, S=Sq, H=H, B=B, seed=5000 + i)
    _, k, v = workloads.generate(idx, S=Skv, H=H, B=B, seed=6000 + i)
    q, k, v = (np.ascontiguousarray(x[..., :D]) for x in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    flags = sage.SAGE_SMOOTH_K if smooth else 0
    out, lse = sage.sage_attention_ex(to_dev(q), to_dev(k), to_dev(v), scale, flags=flags, return_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.sage_attention(q, k, v, scale, sage.sage_kv_tile(), smooth_k=smooth, return_lse=True)
    ex = oracle.exact_attention_fp64(q, k, v, scale)
    label = f"case {i}"
    gate(out.float().cpu().numpy(), ref, ex, label)
    lse_gate(lse.cpu().numpy(), rlse, label)
