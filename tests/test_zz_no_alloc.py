"""GPU test of sage_quant_v_noalloc, the allocation-free variant of
sage_quant_v for callers that cannot allocate device memory: through the C
ABI, its codes and scales equal sage_quant_v's bit for bit, on two calls in a
row that share the library's static scratch (the second smaller than the
first), for head dims 128 and 64.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
sage = pytest.importorskip("quantized_attention_quant_amd")
from gpu_common import DEV, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _pair(v):
    """(noalloc codes, noalloc scales, reference codes, reference scales)."""
    B, S, H, D = v.shape
    Sp = sage.sage_seq_pad(S)
    vd = to_dev(v)
    a8 = torch.full((B, H, D, Sp), 0x7F, dtype=torch.uint8, device=DEV)          # poison
    a_s = torch.full((B, H, D), float("nan"), dtype=torch.float32, device=DEV)
    sage.sage_quant_v_noalloc(vd, a8, a_s)
    b8, b_s = sage.sage_quant_v(vd)
    torch.cuda.synchronize()
    return a8, a_s, b8, b_s


@pytest.mark.parametrize("D", [128, 64])
def test_noalloc_equals_quant_v_on_consecutive_calls(D):
    shapes = [(2, 5000, 7), (1, 333, 3)]          # the second call is smaller
    for i, (B, S, H) in enumerate(shapes):
        say(f"sage_quant_v_noalloc D={D} call {i}: B={B} S={S} H={H}")
        v = workloads.generate(3, S=S, H=H, B=B, seed=60 + i)[2][..., :D]
        v = np.ascontiguousarray(v)
        a8, a_s, b8, b_s = _pair(v)
        assert torch.equal(a8, b8)
        assert torch.equal(a_s.view(torch.int32), b_s.view(torch.int32))


def test_noalloc_full_size_then_small():
    for i, (idx, S, H) in enumerate([(3, 16384, 24), (1, 256, 2)]):
        say(f"sage_quant_v_noalloc config {idx} S={S} H={H}")
        v = workloads.generate(idx, S=S, H=H, B=1, seed=80 + i)[2]
        a8, a_s, b8, b_s = _pair(v)
        assert torch.equal(a8, b8)
        assert torch.equal(a_s.view(torch.int32), b_s.view(torch.int32))


def test_noalloc_rejects_shapes_beyond_its_buffer():
    # 512 x 32 chunks x 128 channels x 4 bytes = 8 MiB fits; 513 heads do not
    v = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device=DEV)
    B, S, H, D = 1, 1 << 14, 513, 128
    assert sage.sage_quant_v_scratch_bytes(B, S, H, D) > (8 << 20)
    rc = sage.lib().sage_quant_v_noalloc(sage._ptr(v), B, S, H, D, sage._ptr(v), sage._ptr(v), None)
    assert rc == 5 and b"static buffer" in sage.lib().sage_last_error()
