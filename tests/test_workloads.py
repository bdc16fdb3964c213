"""The seeded input recipes: determinism, chunked drawing, structure."""
import numpy as np

import workloads


def test_deterministic_and_bf16_valued():
    a = workloads.generate(1)
    b = workloads.generate(1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
        assert x.dtype == np.float32 and x.shape == (1, 256, 2, 128)
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0)      # bf16 values


def test_chunked_drawing_reproduces_one_shot_stream():
    one = workloads.generate(5, S=300, H=3, B=2)
    chunked = workloads.generate(5, S=300, H=3, B=2, chunk_elems=1000)
    for x, y in zip(one, chunked):
        assert np.array_equal(x, y)


def test_recipe_structure():
    q, k, v = workloads.generate(2, S=1024, H=4)
    # K: 8 channels per head carry an offset (mean far from 0)
    means = k.mean(axis=(0, 1))                       # [H, D]
    assert all(int((np.abs(means[h]) > 0.3).sum()) <= 8 for h in range(4))
    q, k, v = workloads.generate(3, S=1024, H=4)
    n = round(0.01 * 1024 * 4)
    big = (np.abs(q).reshape(-1, 128).max(axis=1) > 12).sum()
    assert 0.5 * n <= big <= n
    g = v.std(axis=(0, 1))
    assert g.min() > 0.35 and g.max() < 2.3
    q, k, v = workloads.generate(5, S=512, H=2, B=1)
    assert np.abs(k.mean(axis=(0, 1))).mean() > 0.5   # offsets on all channels
