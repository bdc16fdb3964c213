"""CPU oracle for the SageAttention-style quantized attention forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call or link anything in this package; only the
tests, the smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code, constants or tables with the GPU path.

It is a plain, slow, numpy implementation of what the method computes, in the
order the method states it, written for a reader to check by eye:

* ``formats``   - OCP FP8 E4M3FN encoding/decoding and bfloat16 rounding;
* ``quant``     - symmetric INT8 per 32-row block for Q/K, FP8 per channel for V,
  and the optional K smoothing (K minus its mean over the sequence);
* ``attention`` - exact integer QK^T, dequantization, tile-scheduled online
  softmax in fp32, P to FP8 with the fixed 448 scale, PV, the epilogue and
  the per-row log-sum-exp; query and key lengths may differ; plus exact fp64
  softmax attention as an independent reference.

Sources (cited by page title and section throughout):

* diffusers issue #15014, "gfx1201 (RDNA4) SageAttention attention backend:
  aiter package or Hub kernel?", problem statement: QK^T multiplies INT8
  codes and PV FP8 codes, both summing in fp32; the kernel itself gives Q and
  K one scale per 32 sequence rows and V one scale per channel; the inputs
  are bf16 [B, S, H, 128], one shape for Q, K and V, unmasked and
  non-causal. The operation is ``gfx1201_sage_attention(q, k, v, softmax_scale)``.
* diffusers PR #15060, "Add aiter_sage_hub attention backend for AMD RDNA4
  (gfx1201)", section "What does this PR do?": inference only, no LSE.
* InvokeAI PR #9657, "feat(attention): add opt-in SageAttention backend for
  diffusion models", section "How it works": K smoothing is left off.

Where the pages are silent (rounding modes, scale formulas, the FP8 variant,
how P is quantized, the exp base), the readings taken are listed in each
function's docstring. Every function here is pinned by the ``-m "not gpu"``
tests against something other than itself (closed forms, brute force,
library codecs, invariants, exact fp64 attention).
"""
from .formats import (  # noqa: F401
    E4M3_MAX,
    bf16_round_f64,
    f32,
    fp8_e4m3fn_decode,
    fp8_e4m3fn_encode,
)
from .quant import k_mean, quant_k_smooth, quant_qk, quant_v  # noqa: F401
from .attention import (  # noqa: F401
    LOG2_448,
    LOG2E,
    attention_head,
    exact_attention_fp64,
    exp2_scale,
    lse_from_state,
    online_softmax_exact,
    online_softmax_pv,
    qk_scores,
    sage_attention,
)
