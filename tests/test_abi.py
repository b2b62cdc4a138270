"""C-ABI library checks that need no GPU: it loads, exports every function
declared in include/nvfp4.h, and rejects bad arguments on the host before
touching the device (no kernel is launched for any call here)."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")

EINVAL, EALIGN, EWORKSPACE, ENOTSUP, EHIP, ETIMEOUT = -1, -2, -3, -4, -5, -6
FAKE = 0x7F0000000000          # aligned, never dereferenced: validation fails first
P = ctypes.c_void_p


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    L = nv.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), f"libnvfp4.so does not export {n}"


def test_status_strings_and_version():
    L = nv.lib()
    assert L.nvfp4_abi_version() == 1
    for s in (0, EINVAL, EALIGN, EWORKSPACE, ENOTSUP, EHIP, ETIMEOUT, 42):
        assert L.nvfp4_status_string(s)
    assert L.nvfp4_status_string(0) == b"NVFP4_OK"


def _q(x=FAKE, b=1, r=4, c=32, q=FAKE, sf=FAKE, g=FAKE, ws=FAKE, wsb=1 << 20, flags=0):
    return nv.lib().nvfp4_quantize(P(x), b, r, c, P(q), P(sf), P(g), P(ws), wsb, flags, None)


def test_quantize_validation():
    assert _q(c=15) == EINVAL
    assert _q(r=-1) == EINVAL
    assert _q(b=-2) == EINVAL
    assert _q(x=0) == EINVAL
    assert _q(g=0) == EINVAL
    assert _q(x=FAKE + 2) == EALIGN
    assert _q(q=FAKE + 8) == EALIGN
    assert _q(ws=0) == EWORKSPACE
    assert _q(wsb=16) == EWORKSPACE
    assert _q(flags=7) == ENOTSUP
    assert _q(b=0) == 0                       # empty batch: no-op success
    L = nv.lib()
    assert L.nvfp4_quantize_workspace_bytes(0, 1, 16) == 0
    assert L.nvfp4_quantize_workspace_bytes(64, 2048, 7168) >= 64 * 4


def test_quantize_with_scale_and_dequant_validation():
    L = nv.lib()
    assert L.nvfp4_quantize_with_scale(P(FAKE), 1, 2, 17, P(FAKE), P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_quantize_with_scale(P(FAKE), 1, 2, 16, P(0), P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_quantize_with_scale(P(FAKE + 4), 1, 2, 16, P(FAKE), P(FAKE), P(FAKE), None) == EALIGN
    assert L.nvfp4_quantize_with_scale(P(FAKE), 1, 0, 16, P(FAKE), P(FAKE), P(FAKE), None) == 0
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 1, 2, 40, P(FAKE), None) == EINVAL
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 1, 2, 32, P(0), None) == EINVAL
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE + 2), 1, 2, 32, P(FAKE), None) == EALIGN


def _desc(L_=32, H=8, D=128, cap=131072, **kw):
    d = nv.KVCacheDesc(L_, H, D, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_kv_bytes_matches_worked_example():
    with open(os.path.join(ROOT, "tests", "golden", "kv_size_example.json")) as f:
        gk = json.load(f)
    L = nv.lib()
    d = _desc(gk["layers"], gk["kv_heads"], gk["head_dim"], gk["context_tokens"])
    nbytes = L.nvfp4_kv_bytes(ctypes.byref(d))
    assert nbytes == gk["rows"]["nvfp4"]["per_context_GiB"] * 2 ** 30 == 4_831_838_208
    d1 = _desc(gk["layers"], gk["kv_heads"], gk["head_dim"], 1)
    assert L.nvfp4_kv_bytes(ctypes.byref(d1)) == gk["rows"]["nvfp4"]["per_token_KiB"] * 1024
    assert L.nvfp4_kv_bytes(ctypes.byref(_desc(D=100))) == 0
    assert L.nvfp4_kv_bytes(None) == 0


def test_kv_validation():
    L = nv.lib()
    d = _desc(cap=1000)
    by = ctypes.byref
    assert L.nvfp4_kv_append(by(d), 990, 11, P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_append(by(d), -1, 1, P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_append(by(d), 0, 1, P(0), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_append(by(d), 0, 1, P(FAKE + 8), P(FAKE), None) == EALIGN
    assert L.nvfp4_kv_append(by(d), 1000, 0, P(FAKE), P(FAKE), None) == 0
    assert L.nvfp4_kv_append(by(_desc(D=24)), 0, 1, P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_append(by(_desc(k=0)), 0, 1, P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_append(by(_desc(k_sf=FAKE + 1)), 0, 1, P(FAKE), P(FAKE), None) == EALIGN
    assert L.nvfp4_kv_read(by(d), 30, 3, 0, 10, P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_read(by(d), 0, 1, 995, 10, P(FAKE), P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_read(by(d), 0, 1, 0, 10, P(0), P(0), None) == 0
    assert L.nvfp4_kv_decode_qk(by(d), P(FAKE), 12, 10, P(FAKE), None) == EINVAL    # 12 % 8 != 0
    assert L.nvfp4_kv_decode_qk(by(d), P(FAKE), 32, 1001, P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_decode_qk(by(d), P(0), 32, 10, P(FAKE), None) == EINVAL
    assert L.nvfp4_kv_decode_qk(by(d), P(FAKE), 32, 0, P(FAKE), None) == 0


def test_gemm_validation():
    L = nv.lib()
    args = [P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE)]
    assert L.nvfp4_gemm(*args, 64, 64, 40, P(FAKE), None) == EINVAL
    assert L.nvfp4_gemm(*args, -1, 64, 32, P(FAKE), None) == EINVAL
    assert L.nvfp4_gemm(*args, 64, 64, 32, P(0), None) == EINVAL
    assert L.nvfp4_gemm(*args, 64, 64, 32, P(FAKE + 4), None) == EALIGN
    assert L.nvfp4_gemm(*args, 0, 64, 32, P(FAKE), None) == 0
    # K beyond 2^22 (32-bit offsets of a 256-row operand slab) is rejected up front
    assert L.nvfp4_gemm(*args, 64, 64, (1 << 22) + 16, P(FAKE), None) == EINVAL


def test_kv_append_token_count_limit():
    """n * head_dim/8 half blocks must fit a 32-bit token index per lane."""
    L = nv.lib()
    d = _desc(cap=1 << 40, D=128)
    assert L.nvfp4_kv_append(ctypes.byref(d), 0, (1 << 31) // 16 + 1, P(FAKE), P(FAKE), None) == EINVAL


def test_valid_call_without_gpu_fails_cleanly():
    """With no usable GPU a fully valid call must return an error, not crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the fake pointers would reach a kernel")
    assert _q() in (EHIP, ENOTSUP)


def test_quantize_status_validation():
    """The status query rejects a missing or undersized workspace before it
    touches the device."""
    L = nv.lib()
    assert L.nvfp4_quantize_status(None, 1 << 20, None) == EWORKSPACE
    assert L.nvfp4_quantize_status(P(FAKE), 4, None) == EWORKSPACE
    assert L.nvfp4_status_string(ETIMEOUT).startswith(b"NVFP4_ETIMEOUT")
