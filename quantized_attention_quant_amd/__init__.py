"""Python binding of the MI355X quantized attention library (libsage.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/sage.h``. PyTorch provides
device memory (``torch.empty``) and the current HIP stream. The names match
the C entry points; outputs may be passed in or are allocated here.

There is no CPU fallback: if the library is missing, importing works but
every call raises ``RuntimeError`` (build it with ``__graft_entry__.build()``
or ``python -m quantized_attention_quant_amd.build``).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "SageError", "lib", "library_path", "sage_abi_version", "sage_kv_tile", "sage_seq_pad",
    "sage_workspace_bytes", "sage_quant_v_scratch_bytes", "sage_quant_qk", "sage_quant_v",
    "sage_attn_fwd", "sage_attention", "sage_debug_qk_scores", "v_key_order",
    "SAGE_SMOOTH_K", "sage_k_smooth_scratch_bytes", "sage_quant_k_smooth", "sage_attn_fwd_ex",
    "sage_workspace_bytes_ex", "sage_attention_ex", "sage_attn_fwd_qbf16", "sage_quant_v_noalloc",
    "sage_quant_kv", "sage_debug_p_codes", "sage_debug_fp8_dot",
]

SAGE_SMOOTH_K = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libsage.so")

_lib = None

_STATUS = {0: "SAGE_OK", 1: "SAGE_ERR_NULL", 2: "SAGE_ERR_SHAPE", 3: "SAGE_ERR_UNSUPPORTED",
           4: "SAGE_ERR_ALIGN", 5: "SAGE_ERR_WORKSPACE", 6: "SAGE_ERR_HIP", 7: "SAGE_ERR_RANGE"}


class SageError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libsage.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(library_path)
    i64, p, f32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    sigs = {
        "sage_abi_version": (ctypes.c_int, []),
        "sage_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "sage_last_error": (ctypes.c_char_p, []),
        "sage_kv_tile": (ctypes.c_int, []),
        "sage_seq_pad": (i64, [i64]),
        "sage_quant_v_scratch_bytes": (sz, [i64, i64, i64, i64]),
        "sage_workspace_bytes": (sz, [i64, i64, i64, i64]),
        "sage_quant_qk": (ctypes.c_int, [p, i64, i64, i64, i64, p, p, p]),
        "sage_quant_v": (ctypes.c_int, [p, i64, i64, i64, i64, p, p, p, sz, p]),
        "sage_quant_v_noalloc": (ctypes.c_int, [p, i64, i64, i64, i64, p, p, p]),
        "sage_quant_kv": (ctypes.c_int, [p, p, i64, i64, i64, i64, p, p, p, p, p, sz, p]),
        "sage_attn_fwd": (ctypes.c_int, [p, p, p, p, p, p, i64, i64, i64, i64, f32, p, p]),
        "sage_attention": (ctypes.c_int, [p, p, p, i64, i64, i64, i64, f32, p, p, sz, p]),
        "sage_debug_qk_scores": (ctypes.c_int, [p, p, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                                i64, p, p]),
        "sage_debug_p_codes": (ctypes.c_int, [p, p, p, p, p, p, i64, i64, i64, i64, f32, p, p, p]),
        "sage_debug_fp8_dot": (ctypes.c_int, [p, p, i64, p, p, p]),
        "sage_k_smooth_scratch_bytes": (sz, [i64, i64, i64, i64]),
        "sage_quant_k_smooth": (ctypes.c_int, [p, i64, i64, i64, i64, p, p, p, p, sz, p]),
        "sage_attn_fwd_ex": (ctypes.c_int, [p, p, p, p, p, p, i64, i64, i64, i64, i64, f32, p, p, p]),
        "sage_workspace_bytes_ex": (sz, [i64, i64, i64, i64, i64]),
        "sage_attn_fwd_qbf16": (ctypes.c_int, [p, p, p, p, p, i64, i64, i64, i64, i64, f32, p, p, p]),
        "sage_attention_ex": (ctypes.c_int, [p, p, p, i64, i64, i64, i64, i64, f32, ctypes.c_uint, p, p, p,
                                             sz, p]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise SageError(status, lib().sage_last_error().decode())


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _shape_bshd(x):
    if x.dim() != 4:
        raise ValueError(f"expected a [B, S, H, D] tensor, got shape {tuple(x.shape)}")
    return tuple(int(s) for s in x.shape)


def _require(x, dtype, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def sage_abi_version() -> int:
    return lib().sage_abi_version()


def sage_kv_tile() -> int:
    return lib().sage_kv_tile()


def sage_seq_pad(S: int) -> int:
    return lib().sage_seq_pad(S)


def sage_workspace_bytes(B, S, H, D=128) -> int:
    return lib().sage_workspace_bytes(B, S, H, D)


def sage_quant_v_scratch_bytes(B, S, H, D=128) -> int:
    return lib().sage_quant_v_scratch_bytes(B, S, H, D)


def v_key_order() -> list:
    """Key held by each of the 64 slots of a permuted V^T group (from sage.h)."""
    order = []
    for p in range(64):
        g, u, r = p >> 5, (p >> 4) & 1, p & 15
        order.append(32 * u + 8 * (r // 4) + 4 * g + (r % 4))
    return order


def sage_quant_qk(x, x_i8=None, x_scale=None, stream=None):
    """INT8 per-32-row-block quantization. Returns (x_i8 [B,H,S_pad,D], x_scale [B,H,S_pad/32])."""
    torch = _torch()
    _require(x, torch.bfloat16, "x")
    B, S, H, D = _shape_bshd(x)
    Sp = sage_seq_pad(S)
    if x_i8 is None:
        x_i8 = torch.empty((B, H, Sp, D), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty((B, H, Sp // 32), dtype=torch.float32, device=x.device)
    _require(x_i8, torch.int8, "x_i8")
    _require(x_scale, torch.float32, "x_scale")
    if x_i8.numel() < B * H * Sp * D or x_scale.numel() < B * H * (Sp // 32):
        raise ValueError("output buffers too small")
    _check(lib().sage_quant_qk(_ptr(x), B, S, H, D, _ptr(x_i8), _ptr(x_scale), _stream_ptr(stream)))
    return x_i8, x_scale


def sage_quant_v(v, v_fp8_t=None, v_scale=None, scratch=None, stream=None):
    """FP8 per-channel quantization. Returns (v_fp8_t uint8 [B,H,D,S_pad], v_scale [B,H,D])."""
    torch = _torch()
    _require(v, torch.bfloat16, "v")
    B, S, H, D = _shape_bshd(v)
    Sp = sage_seq_pad(S)
    if v_fp8_t is None:
        v_fp8_t = torch.empty((B, H, D, Sp), dtype=torch.uint8, device=v.device)
    if v_scale is None:
        v_scale = torch.empty((B, H, D), dtype=torch.float32, device=v.device)
    nbytes = sage_quant_v_scratch_bytes(B, S, H, D)
    if scratch is None:
        scratch = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=v.device)
    _require(v_fp8_t, torch.uint8, "v_fp8_t")
    _require(v_scale, torch.float32, "v_scale")
    if v_fp8_t.numel() < B * H * D * Sp or v_scale.numel() < B * H * D:
        raise ValueError("output buffers too small")
    _check(lib().sage_quant_v(_ptr(v), B, S, H, D, _ptr(v_fp8_t), _ptr(v_scale), _ptr(scratch),
                              scratch.numel() * scratch.element_size(), _stream_ptr(stream)))
    return v_fp8_t, v_scale


def sage_quant_kv(k, v, k_i8=None, k_scale=None, v_fp8_t=None, v_scale=None, scratch=None, stream=None):
    """K to INT8 and V to FP8 in one call (fused first pass).
    Returns (k_i8, k_scale, v_fp8_t, v_scale)."""
    torch = _torch()
    _require(k, torch.bfloat16, "k")
    _require(v, torch.bfloat16, "v")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    B, S, H, D = _shape_bshd(k)
    Sp = sage_seq_pad(S)
    dev = k.device
    if k_i8 is None:
        k_i8 = torch.empty((B, H, Sp, D), dtype=torch.int8, device=dev)
    if k_scale is None:
        k_scale = torch.empty((B, H, Sp // 32), dtype=torch.float32, device=dev)
    if v_fp8_t is None:
        v_fp8_t = torch.empty((B, H, D, Sp), dtype=torch.uint8, device=dev)
    if v_scale is None:
        v_scale = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    if scratch is None:
        scratch = torch.empty(max(sage_quant_v_scratch_bytes(B, S, H, D), 256), dtype=torch.uint8, device=dev)
    for t, n, dt, name in ((k_i8, B * H * Sp * D, torch.int8, "k_i8"), (k_scale, B * H * (Sp // 32), torch.float32,
                           "k_scale"), (v_fp8_t, B * H * D * Sp, torch.uint8, "v_fp8_t"),
                           (v_scale, B * H * D, torch.float32, "v_scale")):
        _require(t, dt, name)
        if t.numel() < n:
            raise ValueError(f"{name} too small")
    _check(lib().sage_quant_kv(_ptr(k), _ptr(v), B, S, H, D, _ptr(k_i8), _ptr(k_scale), _ptr(v_fp8_t),
                               _ptr(v_scale), _ptr(scratch), scratch.numel() * scratch.element_size(),
                               _stream_ptr(stream)))
    return k_i8, k_scale, v_fp8_t, v_scale


def sage_quant_v_noalloc(v, v_fp8_t, v_scale, stream=None):
    """sage_quant_v with its scratch in the library's static device buffer:
    allocates nothing (outputs must be passed in). Returns (v_fp8_t, v_scale)."""
    torch = _torch()
    _require(v, torch.bfloat16, "v")
    B, S, H, D = _shape_bshd(v)
    Sp = sage_seq_pad(S)
    _require(v_fp8_t, torch.uint8, "v_fp8_t")
    _require(v_scale, torch.float32, "v_scale")
    if v_fp8_t.numel() < B * H * D * Sp or v_scale.numel() < B * H * D:
        raise ValueError("output buffers too small")
    _check(lib().sage_quant_v_noalloc(_ptr(v), B, S, H, D, _ptr(v_fp8_t), _ptr(v_scale), _stream_ptr(stream)))
    return v_fp8_t, v_scale


def sage_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_fp8_t, v_scale, B, S, H, D=128,
                  softmax_scale=None, out=None, stream=None):
    """Fused attention on quantized inputs. Returns bf16 [B, S, H, D]."""
    torch = _torch()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q_i8.device)
    _require(out, torch.bfloat16, "out")
    Sp = sage_seq_pad(S)
    for t, n, dt in ((q_i8, B * H * Sp * D, torch.int8), (k_i8, B * H * Sp * D, torch.int8),
                     (v_fp8_t, B * H * D * Sp, torch.uint8), (q_scale, B * H * (Sp // 32), torch.float32),
                     (k_scale, B * H * (Sp // 32), torch.float32), (v_scale, B * H * D, torch.float32),
                     (out, B * S * H * D, torch.bfloat16)):
        _require(t, dt, "tensor")
        if t.numel() < n:
            raise ValueError("buffer too small for the given sizes")
    _check(lib().sage_attn_fwd(_ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(v_fp8_t),
                               _ptr(v_scale), B, S, H, D, float(softmax_scale), _ptr(out),
                               _stream_ptr(stream)))
    return out


def sage_attention(q, k, v, softmax_scale=None, out=None, workspace=None, stream=None):
    """gfx1201_sage_attention(q, k, v, softmax_scale) on MI355X: bf16 [B, S, H, D] -> same (D = 128, or 64)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    B, S, H, D = _shape_bshd(q)
    if D not in (64, 128):
        raise ValueError("head dim must be 64 or 128")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _require(out, torch.bfloat16, "out")
    nbytes = sage_workspace_bytes(B, S, H, D)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(lib().sage_attention(_ptr(q), _ptr(k), _ptr(v), B, S, H, D, float(softmax_scale), _ptr(out),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream_ptr(stream)))
    return out


def sage_debug_qk_scores(q_i8, k_i8, B, S, H, b, h, r0, nr, c0, nc, D=128, scores=None, stream=None):
    """Exact int32 scores of one (b, h) window through the fused kernel's MFMA path."""
    torch = _torch()
    if scores is None:
        scores = torch.empty((nr, nc), dtype=torch.int32, device=q_i8.device)
    _require(scores, torch.int32, "scores")
    if scores.numel() < nr * nc:
        raise ValueError("scores buffer too small")
    _check(lib().sage_debug_qk_scores(_ptr(q_i8), _ptr(k_i8), B, S, H, D, b, h, r0, nr, c0, nc,
                                      _ptr(scores), _stream_ptr(stream)))
    return scores


def sage_debug_p_codes(q_i8, q_scale, k_i8, k_scale, v_fp8_t, v_scale, B, S, H, D=128, softmax_scale=None,
                       codes=None, out=None, stream=None):
    """Attention (as sage_attn_fwd) that also returns the FP8 codes of P per
    (b, h, query, key): uint8 [B, H, S, S_pad]. Returns (out, codes)."""
    torch = _torch()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    dev = q_i8.device
    Sp = sage_seq_pad(S)
    if codes is None:
        codes = torch.zeros((B, H, S, Sp), dtype=torch.uint8, device=dev)
    _require(codes, torch.uint8, "codes")
    if codes.numel() < B * H * S * Sp:
        raise ValueError("codes buffer too small")
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
    _check(lib().sage_debug_p_codes(_ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(v_fp8_t),
                                    _ptr(v_scale), B, S, H, D, float(softmax_scale), _ptr(codes), _ptr(out),
                                    _stream_ptr(stream)))
    return out, codes


def sage_debug_fp8_dot(a, b, init=None, out=None, stream=None):
    """init + a[c] . b[c] for each row pair of a and b (uint8 E4M3FN codes,
    [n, 64]) through the PV step's FP8 MFMA. Returns fp32 [n]."""
    torch = _torch()
    _require(a, torch.uint8, "a")
    _require(b, torch.uint8, "b")
    if a.dim() != 2 or a.shape[1] != 64 or b.shape != a.shape:
        raise ValueError("a and b must both be [n, 64]")
    n = a.shape[0]
    if init is None:
        init = torch.zeros(n, dtype=torch.float32, device=a.device)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=a.device)
    _require(init, torch.float32, "init")
    _require(out, torch.float32, "out")
    if init.numel() < n or out.numel() < n:
        raise ValueError("init or out too small")
    _check(lib().sage_debug_fp8_dot(_ptr(a), _ptr(b), n, _ptr(init), _ptr(out), _stream_ptr(stream)))
    return out


def sage_k_smooth_scratch_bytes(B, S, H, D=128) -> int:
    return lib().sage_k_smooth_scratch_bytes(B, S, H, D)


def sage_workspace_bytes_ex(B, Sq, Skv, H, D=128) -> int:
    return lib().sage_workspace_bytes_ex(B, Sq, Skv, H, D)


def sage_quant_k_smooth(k, k_i8=None, k_scale=None, k_mean=None, scratch=None, stream=None):
    """K smoothing + INT8 quantization. Returns (k_i8 [B,H,S_pad,D], k_scale [B,H,S_pad/32], k_mean [B,H,D])."""
    torch = _torch()
    _require(k, torch.bfloat16, "k")
    B, S, H, D = _shape_bshd(k)
    Sp = sage_seq_pad(S)
    if k_i8 is None:
        k_i8 = torch.empty((B, H, Sp, D), dtype=torch.int8, device=k.device)
    if k_scale is None:
        k_scale = torch.empty((B, H, Sp // 32), dtype=torch.float32, device=k.device)
    if k_mean is None:
        k_mean = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    nbytes = sage_k_smooth_scratch_bytes(B, S, H, D)
    if scratch is None:
        scratch = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=k.device)
    _require(k_i8, torch.int8, "k_i8")
    _require(k_scale, torch.float32, "k_scale")
    _require(k_mean, torch.float32, "k_mean")
    if k_i8.numel() < B * H * Sp * D or k_scale.numel() < B * H * (Sp // 32) or k_mean.numel() < B * H * D:
        raise ValueError("output buffers too small")
    _check(lib().sage_quant_k_smooth(_ptr(k), B, S, H, D, _ptr(k_i8), _ptr(k_scale), _ptr(k_mean), _ptr(scratch),
                                     scratch.numel() * scratch.element_size(), _stream_ptr(stream)))
    return k_i8, k_scale, k_mean


def sage_attn_fwd_ex(q_i8, q_scale, k_i8, k_scale, v_fp8_t, v_scale, B, Sq, Skv, H, D=128,
                     softmax_scale=None, out=None, lse=None, return_lse=False, stream=None):
    """Fused attention on quantized inputs with Sq queries and Skv keys.

    Returns bf16 out [B, Sq, H, D], or (out, lse fp32 [B, H, Sq]) when ``lse``
    is given or ``return_lse`` is set."""
    torch = _torch()
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q_i8.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q_i8.device)
    Sqp, Skp = sage_seq_pad(Sq), sage_seq_pad(Skv)
    checks = [(q_i8, B * H * Sqp * D, torch.int8), (k_i8, B * H * Skp * D, torch.int8),
              (v_fp8_t, B * H * D * Skp, torch.uint8), (q_scale, B * H * (Sqp // 32), torch.float32),
              (k_scale, B * H * (Skp // 32), torch.float32), (v_scale, B * H * D, torch.float32),
              (out, B * Sq * H * D, torch.bfloat16)]
    if lse is not None:
        checks.append((lse, B * H * Sq, torch.float32))
    for t, n, dt in checks:
        _require(t, dt, "tensor")
        if t.numel() < n:
            raise ValueError("buffer too small for the given sizes")
    _check(lib().sage_attn_fwd_ex(_ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(v_fp8_t),
                                  _ptr(v_scale), B, Sq, Skv, H, D, float(softmax_scale), _ptr(out), _ptr(lse),
                                  _stream_ptr(stream)))
    return (out, lse) if lse is not None else out


def sage_attention_ex(q, k, v, softmax_scale=None, flags=0, out=None, lse=None, return_lse=False,
                      workspace=None, stream=None):
    """Quantized attention for q [B, Sq, H, D] and k, v [B, Skv, H, D] (bf16, D = 64 or 128).

    ``flags`` may hold SAGE_SMOOTH_K. Returns out [B, Sq, H, 128], or
    (out, lse [B, H, Sq]) when ``lse`` is given or ``return_lse`` is set."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    B, Sq, H, D = _shape_bshd(q)
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError("k and v must be [B, Skv, H, D] with q's B, H and D")
    Skv = int(k.shape[1])
    if D not in (64, 128):
        raise ValueError("head dim must be 64 or 128")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _require(out, torch.bfloat16, "out")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _require(lse, torch.float32, "lse")
        if lse.numel() < B * H * Sq:
            raise ValueError("lse buffer too small")
    nbytes = sage_workspace_bytes_ex(B, Sq, Skv, H, D)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(lib().sage_attention_ex(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, H, D, float(softmax_scale),
                                   int(flags), _ptr(out), _ptr(lse), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return (out, lse) if lse is not None else out


def sage_attn_fwd_qbf16(q, k_i8, k_scale, v_fp8_t, v_scale, Skv=None, softmax_scale=None, out=None, lse=None,
                        return_lse=False, stream=None):
    """Attention with bf16 Q [B, Sq, H, D] quantized inside the kernel and
    quantized K/V (Skv keys; default Sq). Returns out, or (out, lse)."""
    torch = _torch()
    _require(q, torch.bfloat16, "q")
    B, Sq, H, D = _shape_bshd(q)
    Skv = Sq if Skv is None else int(Skv)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    Skp = sage_seq_pad(Skv)
    checks = [(k_i8, B * H * Skp * D, torch.int8), (v_fp8_t, B * H * D * Skp, torch.uint8),
              (k_scale, B * H * (Skp // 32), torch.float32), (v_scale, B * H * D, torch.float32),
              (out, B * Sq * H * D, torch.bfloat16)]
    if lse is not None:
        checks.append((lse, B * H * Sq, torch.float32))
    for t, n, dt in checks:
        _require(t, dt, "tensor")
        if t.numel() < n:
            raise ValueError("buffer too small for the given sizes")
    _check(lib().sage_attn_fwd_qbf16(_ptr(q), _ptr(k_i8), _ptr(k_scale), _ptr(v_fp8_t), _ptr(v_scale), B, Sq, Skv,
                                     H, D, float(softmax_scale), _ptr(out), _ptr(lse), _stream_ptr(stream)))
    return (out, lse) if lse is not None else out
