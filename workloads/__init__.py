"""Seeded synthetic attention inputs (Q, K, V) for the quantized attention forward.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the method's arithmetic (no quantization, no scores, no softmax), so
both the CPU oracle's tests and the GPU path's tests and benchmark can take
their inputs from it.

The pages measure on trained diffusion models (MiniMax-H3, FLUX, SDXL, Krea-2,
Qwen-Image, Wan); none of those weights are available, so these recipes stand
in for them. They use the attention shapes the pages name (bf16 [B, S, H, 128],
self-attention, equal Q/K/V shapes: diffusers issue #15014, "gfx1201 (RDNA4)
SageAttention attention backend: aiter package or Hub kernel?", problem
statement) and the outlier structures the pages describe (one Q/K channel of
about 600 on every image token, and V values of about 3500 across the
channels: InvokeAI PR #9657,
"feat(attention): add opt-in SageAttention backend for diffusion models",
sections "How it works" and "Remaining risks").

Recipe (identical for every consumer):

* generator: ``numpy.random.Generator(numpy.random.PCG64(seed))`` with
  ``seed`` = the config number (1-5) unless a caller passes another seed;
* draw order: Q, K, V as float32 standard normals of shape [B, S, H, D] in
  C order (``standard_normal(dtype=float32)``), then the structure draws of
  the config, in the order listed below;
* transforms are applied in float32, then every tensor is rounded once to
  bfloat16 (round to nearest even, via ``torch.Tensor.to(torch.bfloat16)``).

N(mu, var) below takes a variance: "N(0,4)" has standard deviation 2.

=====  =====================  =======================  ======================
config Q                      K                        V
=====  =====================  =======================  ======================
1      N(0,1)                 N(0,1)                   N(0,1)
2      N(0,1)                 N(0,1) + off[h,c]        N(0,1)
3      1.5*N(0,1), outliers   1.5*N(0,1), outliers     N(0,1)*g[h,c]
4      N(0,1)                 as config 2              N(0,1)
5      N(0,1)                 N(0,1) + off[h,c]        N(0,1)
=====  =====================  =======================  ======================

* configs 2 and 4: for each head h in order, ``rng.choice(128, 8,
  replace=False)`` picks 8 channels, then ``rng.standard_normal(8) * 2``
  gives their offsets (0 elsewhere); the offset is added to every (b, s).
* config 3: ``n = round(0.01 * B * S * H)`` (b, s, h) rows are drawn without
  replacement with ``rng.choice(B*S*H, n, replace=False)``, first for Q, then
  for K; the whole 128-vector of each drawn row is multiplied by 8 (after the
  1.5 scale). Then ``g = rng.uniform(0.5, 2.0, size=(H, 128))`` scales V.
* config 5: ``off = rng.standard_normal((H, 128)) * sqrt(2)`` on all channels.

softmax_scale is 1/sqrt(128) for every config.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = ["Config", "CONFIGS", "config", "generate", "generate_custom", "bf16_round"]


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    S: int
    H: int
    D: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def numel(self) -> int:
        return self.B * self.S * self.H * self.D

    @property
    def ops(self) -> float:
        """Effective operation count 4*B*H*S^2*D (QK^T and PV, 2 ops per MAC)."""
        return 4.0 * self.B * self.H * float(self.S) ** 2 * self.D


CONFIGS = {
    1: Config(1, "tiny B1 S256 H2 D128", 1, 256, 2, 128),
    2: Config(2, "image-DiT 1024^2 B1 S4096 H24 D128", 1, 4096, 24, 128),
    3: Config(3, "image-DiT 2048^2 B1 S16384 H24 D128", 1, 16384, 24, 128),
    4: Config(4, "video-DiT B1 S30720 H24 D128", 1, 30720, 24, 128),
    5: Config(5, "720p video-DiT B2 S75600 H40 D128", 2, 75600, 40, 128),
}


def config(index: int) -> Config:
    return CONFIGS[index]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _normals(rng: np.random.Generator, shape, chunk_elems: int | None) -> np.ndarray:
    """float32 standard normals of ``shape``, optionally drawn in chunks.

    Drawing in consecutive chunks consumes the generator's stream in the same
    order as one draw (the bit generator keeps its buffered half-word across
    calls), so the result is identical; a test checks this.
    """
    n = int(np.prod(shape))
    if chunk_elems is None or chunk_elems >= n:
        return rng.standard_normal(n, dtype=np.float32).reshape(shape)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def _k_offsets_sparse(rng: np.random.Generator, H: int, D: int) -> np.ndarray:
    off = np.zeros((H, D), dtype=np.float32)
    for h in range(H):
        ch = rng.choice(D, 8, replace=False)
        vals = rng.standard_normal(8, dtype=np.float32) * np.float32(2.0)
        off[h, ch] = vals
    return off


def generate(index: int, seed: int | None = None, chunk_elems: int | None = None,
             S: int | None = None, H: int | None = None, B: int | None = None):
    """Return (q, k, v) as float32 arrays [B, S, H, D] holding bfloat16 values.

    ``S``, ``H`` and ``B`` override the config's sizes (same recipe, smaller
    shape), for tests that need the config's value structure at a size the
    oracle finishes quickly.
    """
    cfg = CONFIGS[index]
    B = cfg.B if B is None else B
    S = cfg.S if S is None else S
    H = cfg.H if H is None else H
    D = cfg.D
    rng = np.random.Generator(np.random.PCG64(index if seed is None else seed))
    shape = (B, S, H, D)
    q = _normals(rng, shape, chunk_elems)
    k = _normals(rng, shape, chunk_elems)
    v = _normals(rng, shape, chunk_elems)
    if index in (2, 4):
        k += _k_offsets_sparse(rng, H, D)[None, None]
    elif index == 3:
        q *= np.float32(1.5)
        k *= np.float32(1.5)
        n = int(round(0.01 * B * S * H))
        for t in (q, k):
            rows = rng.choice(B * S * H, n, replace=False)
            flat = t.reshape(B * S * H, D)
            flat[rows] *= np.float32(8.0)
        g = rng.uniform(0.5, 2.0, size=(H, D)).astype(np.float32)
        v *= g[None, None]
    elif index == 5:
        off = rng.standard_normal((H, D), dtype=np.float32) * np.float32(math.sqrt(2.0))
        k += off[None, None]
    return bf16_round(q), bf16_round(k), bf16_round(v)


def generate_custom(shape, seed: int, kind: str = "normal", scale: float = 1.0) -> np.ndarray:
    """A single bf16-valued float32 tensor for edge-case tests.

    kind: "normal" (N(0,1)*scale), "zeros", "ones" (constant ``scale``),
    "uniform" (U(-scale, scale)).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "normal":
        x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape) * np.float32(scale)
    elif kind == "zeros":
        x = np.zeros(shape, dtype=np.float32)
    elif kind == "ones":
        x = np.full(shape, scale, dtype=np.float32)
    elif kind == "uniform":
        x = rng.uniform(-scale, scale, size=shape).astype(np.float32)
    else:
        raise ValueError(kind)
    return bf16_round(x)
