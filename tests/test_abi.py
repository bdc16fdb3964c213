"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/sage.h declares, and rejects bad arguments before any launch.

Only validation paths and pure queries are called here; fake device pointers
are never dereferenced because every call below returns before launching.
"""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_attention_quant_amd as sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_HIP, ERR_RANGE = range(8)
FAKE = 0x100000          # aligned, never dereferenced
MISALIGNED = 0x100008


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("sage_quant_qk", "sage_quant_v", "sage_attn_fwd", "sage_attention", "sage_debug_qk_scores",
              "sage_workspace_bytes", "sage_kv_tile", "sage_seq_pad", "sage_quant_k_smooth",
              "sage_k_smooth_scratch_bytes", "sage_attn_fwd_ex", "sage_workspace_bytes_ex",
              "sage_attention_ex", "sage_debug_p_codes", "sage_debug_fp8_dot"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = sage.lib()
    for n in _declared():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sage.library_path], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT (sage_\w+)", out.stdout))
        assert set(_declared()) <= exported


def test_queries():
    assert sage.sage_abi_version() == 1
    bn = sage.sage_kv_tile()
    assert bn % 32 == 0 and bn >= 32
    for S, Sp in ((1, 256), (256, 256), (257, 512), (75600, 75776), (16384, 16384)):
        assert sage.sage_seq_pad(S) == Sp
    # workspace: the one-byte K and V codes plus small scales/scratch (Q is
    # quantized inside the attention kernel), i.e. about 2/3 byte per element
    # of the three inputs
    for B, S, H in ((1, 256, 2), (1, 16384, 24), (2, 75600, 40)):
        Sp = sage.sage_seq_pad(S)
        ws = sage.sage_workspace_bytes(B, S, H, 128)
        base = 2 * B * H * Sp * 128
        assert base <= ws <= base * 1.02 + 65536
        assert ws <= 0.68 * 3 * B * S * H * 128 + 65536
        wx = sage.lib().sage_workspace_bytes_ex(B, S, S, H, 128)
        assert base <= wx <= base * 1.03 + 65536
    assert sage.sage_workspace_bytes(1, 256, 2, 96) == 0
    # head dim 64: half the bytes of the one-byte tensors
    assert sage.sage_workspace_bytes(1, 256, 2, 64) < sage.sage_workspace_bytes(1, 256, 2, 128)
    assert sage.sage_workspace_bytes(1, 256, 2, 64) >= 2 * 2 * 256 * 64
    assert sage.sage_workspace_bytes(0, 256, 2, 128) == 0
    assert sage.lib().sage_status_str(ERR_WS) == b"SAGE_ERR_WORKSPACE"


def _call(name, *args):
    fn = getattr(sage.lib(), name)
    return fn(*args)


def test_validation_codes():
    p = ctypes.c_void_p
    f, m = p(FAKE), p(MISALIGNED)
    z = p(0)
    # the fused K/V quantizer
    assert _call("sage_quant_kv", f, f, 1, 256, 2, 96, f, f, f, f, f, 1 << 20, z) == ERR_UNSUP
    assert _call("sage_quant_kv", f, z, 1, 256, 2, 128, f, f, f, f, f, 1 << 20, z) == ERR_NULL
    assert _call("sage_quant_kv", f, f, 1, 256, 2, 128, f, f, f, m, f, 1 << 20, z) == ERR_ALIGN
    assert _call("sage_quant_kv", f, f, 1, 256, 2, 128, f, f, f, f, f, 16, z) == ERR_WS
    # B*H beyond 65535 is accepted by the size checks (1-D grids)
    assert _call("sage_quant_kv", f, f, 1, 256, 70000, 128, f, f, f, f, f, 16, z) == ERR_WS
    # the allocation-free V quantizer: shapes beyond its static buffer
    assert _call("sage_quant_v_noalloc", f, 1, 16384, 513, 128, f, f, z) == ERR_WS
    assert b"static buffer" in sage.lib().sage_last_error()
    assert _call("sage_quant_v_noalloc", z, 1, 256, 2, 128, f, f, z) == ERR_NULL
    # head dim, sizes
    assert _call("sage_quant_qk", f, 1, 256, 2, 96, f, f, z) == ERR_UNSUP
    assert _call("sage_quant_qk", f, 1, 256, 2, 256, f, f, z) == ERR_UNSUP
    assert _call("sage_quant_qk", f, 0, 256, 2, 128, f, f, z) == ERR_SHAPE
    # the score dump covers head dim 128 only
    assert _call("sage_debug_qk_scores", f, f, 1, 256, 2, 96, 0, 0, 0, 1, 0, 1, f, z) == ERR_UNSUP
    assert _call("sage_quant_qk", f, 1, -5, 2, 128, f, f, z) == ERR_SHAPE
    assert _call("sage_quant_qk", f, 1, 1 << 40, 2, 128, f, f, z) == ERR_SHAPE
    assert _call("sage_quant_qk", f, 1, (1 << 24) + 1, 2, 128, f, f, z) == ERR_SHAPE
    # pointers
    assert _call("sage_quant_qk", z, 1, 256, 2, 128, f, f, z) == ERR_NULL
    assert _call("sage_quant_qk", m, 1, 256, 2, 128, f, f, z) == ERR_ALIGN
    assert b"not 16-byte aligned" in sage.lib().sage_last_error()
    # scratch / workspace sizes
    need = sage.sage_quant_v_scratch_bytes(1, 256, 2)
    assert _call("sage_quant_v", f, 1, 256, 2, 128, f, f, f, need - 1, z) == ERR_WS
    ws = sage.sage_workspace_bytes(1, 256, 2)
    assert _call("sage_attention", f, f, f, 1, 256, 2, 128, ctypes.c_float(0.1), f, f, ws - 1, z) == ERR_WS
    assert _call("sage_attention", f, f, f, 1, 256, 2, 128, ctypes.c_float(0.1), f, p(FAKE + 16), ws, z) == ERR_ALIGN
    assert _call("sage_attention", f, f, f, 1, 256, 2, 128, ctypes.c_float(float("nan")), f, f, ws, z) == ERR_SHAPE
    assert _call("sage_attention", f, f, f, 1, 256, 2, 128, ctypes.c_float(-0.1), f, f, ws, z) == ERR_SHAPE
    assert _call("sage_attn_fwd", f, f, f, f, f, f, 1, 256, 2, 128, ctypes.c_float(-1.0), f, z) == ERR_SHAPE
    assert _call("sage_attn_fwd", f, f, f, f, f, z, 1, 256, 2, 128, ctypes.c_float(0.1), f, z) == ERR_NULL
    # debug window
    assert _call("sage_debug_qk_scores", f, f, 1, 256, 2, 128, 0, 0, 0, 256, 0, 257, f, z) == ERR_RANGE
    assert _call("sage_debug_qk_scores", f, f, 1, 256, 2, 128, 0, 2, 0, 1, 0, 1, f, z) == ERR_RANGE
    assert _call("sage_debug_qk_scores", f, f, 1, 256, 2, 128, 0, 0, 0, 0, 0, 1, f, z) == ERR_RANGE
    # P-code dump: same checks as sage_attn_fwd, plus the codes buffer and the sequence limit
    c01 = ctypes.c_float(0.1)
    assert _call("sage_debug_p_codes", f, f, f, f, f, f, 1, 256, 2, 128, c01, z, f, z) == ERR_NULL
    assert _call("sage_debug_p_codes", f, f, f, f, f, f, 1, 256, 2, 96, c01, f, f, z) == ERR_UNSUP
    assert _call("sage_debug_p_codes", f, f, f, f, f, f, 1, 131073, 2, 128, c01, f, f, z) == ERR_RANGE
    assert _call("sage_debug_p_codes", f, f, f, f, f, f, 1, 256, 2, 128, ctypes.c_float(-1.0), f, f, z) == ERR_SHAPE
    assert _call("sage_debug_p_codes", m, f, f, f, f, f, 1, 256, 2, 128, c01, f, f, z) == ERR_ALIGN
    # FP8 MFMA probe: pointers, alignment, pair count
    assert _call("sage_debug_fp8_dot", z, f, 1, f, f, z) == ERR_NULL
    assert _call("sage_debug_fp8_dot", f, z, 1, f, f, z) == ERR_NULL
    assert _call("sage_debug_fp8_dot", f, f, 1, z, f, z) == ERR_NULL
    assert _call("sage_debug_fp8_dot", f, f, 1, f, z, z) == ERR_NULL
    assert _call("sage_debug_fp8_dot", m, f, 1, f, f, z) == ERR_ALIGN
    assert _call("sage_debug_fp8_dot", f, m, 1, f, f, z) == ERR_ALIGN
    assert _call("sage_debug_fp8_dot", f, f, 1, f, p(FAKE + 2), z) == ERR_ALIGN
    assert _call("sage_debug_fp8_dot", f, f, 0, f, f, z) == ERR_RANGE
    assert _call("sage_debug_fp8_dot", f, f, (1 << 24) + 1, f, f, z) == ERR_RANGE

def test_extended_entry_points_validation():
    p = ctypes.c_void_p
    f, m, z = p(FAKE), p(MISALIGNED), p(0)
    fl = ctypes.c_float(0.1)
    # workspace for cross-attention covers both lengths and the smoothing scratch
    for B, Sq, Skv, H in ((1, 300, 77, 2), (1, 64, 4096, 24), (2, 75600, 75600, 40)):
        ws = sage.sage_workspace_bytes_ex(B, Sq, Skv, H, 128)
        Sqp, Skp = sage.sage_seq_pad(Sq), sage.sage_seq_pad(Skv)
        base = B * H * 128 * 2 * Skp               # K and V codes (Q is quantized in the kernel)
        assert base <= ws <= base * 1.03 + 65536   # + scales and the larger scratch
        if Sq == Skv:
            assert ws >= sage.sage_workspace_bytes(B, Sq, H, 128)
    assert sage.sage_workspace_bytes_ex(1, 300, 0, 2, 128) == 0
    assert sage.sage_workspace_bytes_ex(1, 300, 77, 2, 96) == 0
    assert 0 < sage.sage_workspace_bytes_ex(1, 300, 77, 2, 64) < sage.sage_workspace_bytes_ex(1, 300, 77, 2, 128)
    nb = sage.sage_k_smooth_scratch_bytes(1, 300, 2, 128)
    assert nb >= 2 * 2 * 128 * 8                    # fp64 sums of two 256-row chunks per head
    # sage_quant_k_smooth
    assert _call("sage_quant_k_smooth", f, 1, 300, 2, 128, f, f, f, f, nb - 1, z) == ERR_WS
    assert _call("sage_quant_k_smooth", f, 1, 300, 2, 128, f, f, z, f, nb, z) == ERR_NULL
    assert _call("sage_quant_k_smooth", f, 1, 300, 2, 128, m, f, f, f, nb, z) == ERR_ALIGN
    assert _call("sage_quant_k_smooth", f, 1, 300, 2, 96, f, f, f, f, nb, z) == ERR_UNSUP
    assert sage.sage_k_smooth_scratch_bytes(1, 300, 2, 64) * 2 == sage.sage_k_smooth_scratch_bytes(1, 300, 2, 128)
    # sage_attn_fwd_ex: both lengths are checked, lse alignment is checked
    args = [f, f, f, f, f, f]
    assert _call("sage_attn_fwd_ex", *args, 1, 300, 0, 2, 128, fl, f, z, z) == ERR_SHAPE
    assert _call("sage_attn_fwd_ex", *args, 1, 0, 77, 2, 128, fl, f, z, z) == ERR_SHAPE
    assert _call("sage_attn_fwd_ex", *args, 1, 300, 77, 2, 128, fl, f, p(FAKE + 2), z) == ERR_ALIGN
    assert _call("sage_attn_fwd_ex", *args, 1, 300, 77, 2, 128, ctypes.c_float(float("inf")), f, z, z) == ERR_SHAPE
    assert _call("sage_attn_fwd_ex", f, f, f, f, f, f, 1, 300, 77, 2, 128, fl, z, z, z) == ERR_NULL
    # sage_attention_ex: flags, workspace
    ws = sage.sage_workspace_bytes_ex(1, 300, 77, 2, 128)
    assert _call("sage_attention_ex", f, f, f, 1, 300, 77, 2, 128, fl, 2, f, z, f, ws, z) == ERR_UNSUP
    assert _call("sage_attention_ex", f, f, f, 1, 300, 77, 2, 128, fl, 1, f, z, f, ws - 1, z) == ERR_WS
    assert _call("sage_attention_ex", f, f, f, 1, 300, 77, 2, 128, fl, 1, f, z, z, ws, z) == ERR_NULL
    assert _call("sage_attention_ex", f, f, f, 1, 300, 77, 2, 128, fl, 0, f, z, p(FAKE + 64), ws, z) == ERR_ALIGN


def test_attn_fwd_qbf16_validation():
    p = ctypes.c_void_p
    f, m, z = p(FAKE), p(MISALIGNED), p(0)
    fl = ctypes.c_float(0.1)
    args = [f, f, f, f]
    assert _call("sage_attn_fwd_qbf16", z, *args, 1, 300, 77, 2, 128, fl, f, z, z) == ERR_NULL
    assert _call("sage_attn_fwd_qbf16", m, *args, 1, 300, 77, 2, 128, fl, f, z, z) == ERR_ALIGN
    assert _call("sage_attn_fwd_qbf16", f, *args, 1, 300, 77, 2, 96, fl, f, z, z) == ERR_UNSUP
    assert _call("sage_attn_fwd_qbf16", f, *args, 1, 300, 0, 2, 128, fl, f, z, z) == ERR_SHAPE
    assert _call("sage_attn_fwd_qbf16", f, *args, 1, 300, 77, 2, 128, ctypes.c_float(-1.0), f, z, z) == ERR_SHAPE
    assert _call("sage_attn_fwd_qbf16", f, *args, 1, 300, 77, 2, 128, fl, f, p(FAKE + 1), z) == ERR_ALIGN


def test_forced_launch_failure_hook(monkeypatch):
    monkeypatch.setenv("SAGE_TEST_FAIL_LAUNCH", "1")
    p = ctypes.c_void_p
    f, z = p(FAKE), p(0)
    assert _call("sage_quant_qk", f, 1, 256, 2, 128, f, f, z) == ERR_HIP
    ws = sage.sage_workspace_bytes(1, 256, 2)
    assert _call("sage_attention", f, f, f, 1, 256, 2, 128, ctypes.c_float(0.1), f, f, ws, z) == ERR_HIP
    assert b"forced" in sage.lib().sage_last_error()
    wsx = sage.sage_workspace_bytes_ex(1, 300, 77, 2, 128)
    assert _call("sage_attention_ex", f, f, f, 1, 300, 77, 2, 128, ctypes.c_float(0.1), 1, f, f, f, wsx, z) == ERR_HIP
    nb = sage.sage_k_smooth_scratch_bytes(1, 300, 2, 128)
    assert _call("sage_quant_k_smooth", f, 1, 300, 2, 128, f, f, f, f, nb, z) == ERR_HIP
    assert _call("sage_attn_fwd_ex", f, f, f, f, f, f, 1, 300, 77, 2, 128, ctypes.c_float(0.1), f, f, z) == ERR_HIP
    assert _call("sage_attn_fwd_qbf16", f, f, f, f, f, 1, 300, 77, 2, 128, ctypes.c_float(0.1), f, f, z) == ERR_HIP
    # validation still runs first
    assert _call("sage_quant_qk", f, 1, 256, 2, 96, f, f, z) == ERR_UNSUP
    assert _call("sage_quant_qk", f, 1, 256, 2, 64, f, f, z) == ERR_HIP


def test_binding_raises_on_missing_library(monkeypatch):
    monkeypatch.setattr(sage, "_lib", None)
    monkeypatch.setattr(sage, "library_path", "/nonexistent/libsage.so")
    with pytest.raises(RuntimeError, match="not built"):
        sage.lib()


def test_binding_rejects_non_bf16_inputs():
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 32, 1, 128), dtype=torch.float32)
    with pytest.raises((ValueError, TypeError)):
        sage.sage_quant_qk(x)
    with pytest.raises(ValueError):
        sage.sage_attention(x, x, x)
