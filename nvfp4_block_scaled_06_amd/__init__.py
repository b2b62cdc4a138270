"""Python binding for libnvfp4, the gfx950 NVFP4 two-level microscaling library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libnvfp4.so (built in-tree by nvfp4_block_scaled_06_amd/build.py).  PyTorch
provides device memory and the current HIP stream.  There is no CPU path:
if the library is missing or the device is not gfx950, calls raise.

Function names mirror the C-ABI in include/nvfp4.h.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

TWO_KERNEL = 0
FUSED = 1
_FLAGS = {"two_kernel": TWO_KERNEL, "fused": FUSED, TWO_KERNEL: TWO_KERNEL, FUSED: FUSED}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


class NVFP4Error(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib().nvfp4_status_string(status).decode()
        if status == -5:
            msg += f" (hipError {_lib().nvfp4_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


class KVCacheDesc(ctypes.Structure):
    """Mirror of the C struct nvfp4_kv_cache."""
    _fields_ = [
        ("layers", _I32), ("kv_heads", _I32), ("head_dim", _I32),
        ("capacity", _I64),
        ("k", _P), ("v", _P), ("k_sf", _P), ("v_sf", _P),
        ("k_g", _P), ("v_g", _P),
    ]


_SIGS = {
    "nvfp4_abi_version": (_I32, []),
    "nvfp4_status_string": (ctypes.c_char_p, [_I32]),
    "nvfp4_last_hip_error": (_I32, []),
    "nvfp4_quantize_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "nvfp4_quantize": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, ctypes.c_uint32, _P]),
    "nvfp4_quantize_noalloc": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, ctypes.c_uint32, _P]),
    "nvfp4_quantize_status": (_I32, [_P, _SZ, _P]),
    "nvfp4_set_wait_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
    "nvfp4_quantize_with_scale": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "nvfp4_dequantize": (_I32, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "nvfp4_kv_bytes": (_SZ, [ctypes.POINTER(KVCacheDesc)]),
    "nvfp4_kv_append": (_I32, [ctypes.POINTER(KVCacheDesc), _I64, _I64, _P, _P, _P]),
    "nvfp4_kv_read": (_I32, [ctypes.POINTER(KVCacheDesc), _I32, _I32, _I64, _I64, _P, _P, _P]),
    "nvfp4_kv_decode_qk": (_I32, [ctypes.POINTER(KVCacheDesc), _P, _I32, _I64, _P, _P]),
    "nvfp4_gemm": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "nvfp4_grouped_gemm": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _P]),
    "nvfp4_kv_attention_workspace_bytes": (ctypes.c_size_t, [_P, _I32, _I64]),
    "nvfp4_kv_decode_attention": (_I32, [_P, _P, _I32, _I64, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]),
    "nvfp4_quantize_ex_workspace_bytes": (_SZ, [_I64]),
    "nvfp4_quantize_ex": (_I32, [_P, _I64, _I64, _I64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                 ctypes.c_uint64, _P, _P, _P, _P, _SZ, _P]),
    "nvfp4_mxfp4_quantize": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "nvfp4_mxfp4_dequantize": (_I32, [_P, _P, _I64, _I64, _P, _P]),
    "nvfp4_mxfp4_gemm": (_I32, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
}

_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python nvfp4_block_scaled_06_amd/build.py (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _L = L
    return _L


def lib():
    """The loaded ctypes library (raises if libnvfp4.so is not built)."""
    return _lib()


def _check(fn, status):
    if status != 0:
        raise NVFP4Error(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _numel(t, n, name):
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")


# ---------------------------------------------------------------- codec
def workspace_bytes(batch, rows, cols):
    return int(_lib().nvfp4_quantize_workspace_bytes(batch, rows, cols))


def make_workspace(batch, rows, cols, device="cuda"):
    return torch.zeros(workspace_bytes(batch, rows, cols), dtype=torch.uint8, device=device)


def _split(shape):
    if len(shape) == 2:
        return 1, shape[0], shape[1]
    if len(shape) == 3:
        return shape
    raise ValueError("expected [rows, cols] or [batch, rows, cols]")


def quantize(x, flags="two_kernel", workspace=None, out=None):
    """x: bf16 [rows, cols] or [batch, rows, cols] -> (q uint8 [..., cols/2],
    sf uint8 [..., cols/16], g float32 [batch])."""
    _need(x, torch.bfloat16, "x")
    b, r, c = _split(x.shape)
    lead = tuple(x.shape[:-1])
    if out is None:
        q = torch.empty(lead + (c // 2,), dtype=torch.uint8, device=x.device)
        sf = torch.empty(lead + (c // 16,), dtype=torch.uint8, device=x.device)
        g = torch.empty((b,), dtype=torch.float32, device=x.device)
    else:
        q, sf, g = out
        _need(q, torch.uint8, "q")
        _need(sf, torch.uint8, "sf")
        _need(g, torch.float32, "g")
        _shape(q, lead + (c // 2,), "q")
        _shape(sf, lead + (c // 16,), "sf")
        _numel(g, b, "g")
    if workspace is None:
        workspace = make_workspace(b, r, c, x.device)
    _need(workspace, torch.uint8, "workspace")
    _check("nvfp4_quantize", _lib().nvfp4_quantize(
        _ptr(x), b, r, c, _ptr(q), _ptr(sf), _ptr(g), _ptr(workspace), workspace.numel(),
        _FLAGS[flags], _stream(x.device)))
    return q, sf, g


def quantize_noalloc(x, flags="two_kernel", out=None):
    """nvfp4_quantize with the library's fixed device scratch instead of a
    workspace (no allocation inside the call; batch <= 101).  Calls on one
    GPU must not overlap in time."""
    _need(x, torch.bfloat16, "x")
    b, r, c = _split(x.shape)
    lead = tuple(x.shape[:-1])
    if out is None:
        q = torch.empty(lead + (c // 2,), dtype=torch.uint8, device=x.device)
        sf = torch.empty(lead + (c // 16,), dtype=torch.uint8, device=x.device)
        g = torch.empty((b,), dtype=torch.float32, device=x.device)
    else:
        q, sf, g = out
        _need(q, torch.uint8, "q")
        _need(sf, torch.uint8, "sf")
        _need(g, torch.float32, "g")
        _shape(q, lead + (c // 2,), "q")
        _shape(sf, lead + (c // 16,), "sf")
        _numel(g, b, "g")
    _check("nvfp4_quantize_noalloc", _lib().nvfp4_quantize_noalloc(
        _ptr(x), b, r, c, _ptr(q), _ptr(sf), _ptr(g), _FLAGS[flags], _stream(x.device)))
    return q, sf, g


ETIMEOUT = -6


def quantize_status(workspace):
    """Synchronizes the current stream and reports whether a FUSED quantize
    on `workspace` had a bounded cross-workgroup wait give up since the last
    report (those tensors' g are NaN).  Clears the report; returns True when
    the calls were clean, raises NVFP4Error (status ETIMEOUT) otherwise."""
    _need(workspace, torch.uint8, "workspace")
    _check("nvfp4_quantize_status", _lib().nvfp4_quantize_status(
        _ptr(workspace), workspace.numel(), _stream(workspace.device)))
    return True


def set_wait_limit(polls):
    """Polls after which the co-resident kernels' bounded waits give up, on the
    current device (default 2^24); returns the previous value.  0 makes every
    wait give up at once: a test hook for the timeout path."""
    return int(_lib().nvfp4_set_wait_limit(int(polls)))


def quantize_with_scale(x, g, out=None):
    _need(x, torch.bfloat16, "x")
    _need(g, torch.float32, "g")
    b, r, c = _split(x.shape)
    if g.numel() != b:
        raise ValueError("g must hold one scale per batch item")
    lead = tuple(x.shape[:-1])
    if out is None:
        q = torch.empty(lead + (c // 2,), dtype=torch.uint8, device=x.device)
        sf = torch.empty(lead + (c // 16,), dtype=torch.uint8, device=x.device)
    else:
        q, sf = out
        _need(q, torch.uint8, "q")
        _need(sf, torch.uint8, "sf")
        _shape(q, lead + (c // 2,), "q")
        _shape(sf, lead + (c // 16,), "sf")
    _check("nvfp4_quantize_with_scale", _lib().nvfp4_quantize_with_scale(
        _ptr(x), b, r, c, _ptr(g), _ptr(q), _ptr(sf), _stream(x.device)))
    return q, sf


def dequantize(q, sf, g, out=None):
    _need(q, torch.uint8, "q")
    _need(sf, torch.uint8, "sf")
    _need(g, torch.float32, "g")
    c = q.shape[-1] * 2
    b, r, _ = _split(tuple(q.shape[:-1]) + (c,))
    _shape(sf, tuple(q.shape[:-1]) + (c // 16,), "sf")
    _numel(g, b, "g")
    if out is not None:
        _need(out, torch.bfloat16, "out")
        _shape(out, tuple(q.shape[:-1]) + (c,), "out")
    y = out if out is not None else torch.empty(tuple(q.shape[:-1]) + (c,), dtype=torch.bfloat16, device=q.device)
    _check("nvfp4_dequantize", _lib().nvfp4_dequantize(
        _ptr(q), _ptr(sf), _ptr(g), b, r, c, _ptr(y), _stream(q.device)))
    return y


# ---------------------------------------------------------------- KV cache
class KVCache:
    """Caller-owned NVFP4 KV cache: K/V codes [L][H][capacity][D/2], block
    scales [L][H][capacity][D/16] and fixed per-(layer, head) tensor scales."""

    def __init__(self, layers, kv_heads, head_dim, capacity, k_g, v_g, device="cuda"):
        self.layers, self.kv_heads, self.head_dim, self.capacity = layers, kv_heads, head_dim, capacity
        shp = (layers, kv_heads, capacity)
        self.k = torch.empty(shp + (head_dim // 2,), dtype=torch.uint8, device=device)
        self.v = torch.empty_like(self.k)
        self.k_sf = torch.empty(shp + (head_dim // 16,), dtype=torch.uint8, device=device)
        self.v_sf = torch.empty_like(self.k_sf)
        self.k_g = k_g.to(device=device, dtype=torch.float32).contiguous().reshape(layers, kv_heads)
        self.v_g = v_g.to(device=device, dtype=torch.float32).contiguous().reshape(layers, kv_heads)
        self.desc = KVCacheDesc(layers, kv_heads, head_dim, capacity,
                                self.k.data_ptr(), self.v.data_ptr(), self.k_sf.data_ptr(),
                                self.v_sf.data_ptr(), self.k_g.data_ptr(), self.v_g.data_ptr())

    def nbytes(self):
        return int(_lib().nvfp4_kv_bytes(ctypes.byref(self.desc)))

    def append(self, start, k_new, v_new, stream=None):
        """Encodes tokens [start, start + n) into the cache on `stream` (a
        torch.cuda.Stream; default: the current stream).  Appends of disjoint
        token ranges may run on different streams at once."""
        _need(k_new, torch.bfloat16, "k_new")
        _need(v_new, torch.bfloat16, "v_new")
        if k_new.dim() != 4:
            raise ValueError("k_new must be [layers][n][kv_heads][head_dim]")
        n = k_new.shape[1]
        _shape(k_new, (self.layers, n, self.kv_heads, self.head_dim), "k_new")
        _shape(v_new, (self.layers, n, self.kv_heads, self.head_dim), "v_new")
        st = _stream(k_new.device) if stream is None else ctypes.c_void_p(stream.cuda_stream)
        _check("nvfp4_kv_append", _lib().nvfp4_kv_append(
            ctypes.byref(self.desc), start, n, _ptr(k_new), _ptr(v_new), st))

    def read(self, layer0, nlayers, t0, n, k_out=None, v_out=None, want_k=True, want_v=True):
        shp = (nlayers, self.kv_heads, n, self.head_dim)
        dev = self.k.device
        for t, nm in ((k_out, "k_out"), (v_out, "v_out")):
            if t is not None:
                _need(t, torch.bfloat16, nm)
                _shape(t, shp, nm)
        if want_k and k_out is None:
            k_out = torch.empty(shp, dtype=torch.bfloat16, device=dev)
        if want_v and v_out is None:
            v_out = torch.empty(shp, dtype=torch.bfloat16, device=dev)
        _check("nvfp4_kv_read", _lib().nvfp4_kv_read(
            ctypes.byref(self.desc), layer0, nlayers, t0, n, _ptr(k_out), _ptr(v_out), _stream(dev)))
        return k_out, v_out

    def attention_workspace_bytes(self, q_heads, n):
        return int(_lib().nvfp4_kv_attention_workspace_bytes(ctypes.byref(self.desc), q_heads, n))

    def decode_attention(self, q, n, scale, out=None, workspace=None):
        """One decode step of attention over the first n cached tokens:
        softmax(scale * q K^T) V per query head, fp32 [layers][q_heads][head_dim]."""
        _need(q, torch.bfloat16, "q")
        L, Hq, D = self._query_shape(q)
        if out is not None:
            _need(out, torch.float32, "out")
            _shape(out, (L, Hq, D), "out")
        o = out if out is not None else torch.empty((L, Hq, D), dtype=torch.float32, device=q.device)
        nb = self.attention_workspace_bytes(Hq, n)
        ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
        _need(ws, torch.uint8, "workspace")
        _check("nvfp4_kv_decode_attention", _lib().nvfp4_kv_decode_attention(
            ctypes.byref(self.desc), _ptr(q), Hq, n, float(scale), _ptr(o), _ptr(ws), ws.numel(),
            _stream(q.device)))
        return o

    def _query_shape(self, q):
        if q.dim() != 3 or q.shape[0] != self.layers or q.shape[2] != self.head_dim:
            raise ValueError(f"q must be [layers={self.layers}][q_heads][head_dim={self.head_dim}], "
                             f"got {tuple(q.shape)}")
        return tuple(q.shape)

    def decode_qk(self, q, n, out=None):
        _need(q, torch.bfloat16, "q")
        L, Hq, D = self._query_shape(q)
        if out is not None:
            _need(out, torch.float32, "out")
            _shape(out, (L, Hq, n), "out")
        logits = out if out is not None else torch.empty((L, Hq, n), dtype=torch.float32, device=q.device)
        _check("nvfp4_kv_decode_qk", _lib().nvfp4_kv_decode_qk(
            ctypes.byref(self.desc), _ptr(q), Hq, n, _ptr(logits), _stream(q.device)))
        return logits


# ---------------------------------------------------------------- GEMM
def gemm(a_q, a_sf, a_g, b_q, b_sf, b_g, out=None):
    """C[M][N] = gA*gB * sum_k deq(A)[m][k] deq(B)[n][k]; fp32 output."""
    for t, n in ((a_q, "a_q"), (a_sf, "a_sf"), (b_q, "b_q"), (b_sf, "b_sf")):
        _need(t, torch.uint8, n)
    _need(a_g, torch.float32, "a_g")
    _need(b_g, torch.float32, "b_g")
    if a_q.dim() != 2 or b_q.dim() != 2:
        raise ValueError("a_q and b_q must be [rows][K/2]")
    M, K2 = a_q.shape
    N = b_q.shape[0]
    _shape(b_q, (N, K2), "b_q")
    _shape(a_sf, (M, K2 // 8), "a_sf")
    _shape(b_sf, (N, K2 // 8), "b_sf")
    _numel(a_g, 1, "a_g")
    _numel(b_g, 1, "b_g")
    if out is not None:
        _need(out, torch.float32, "out")
        _shape(out, (M, N), "out")
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a_q.device)
    _check("nvfp4_gemm", _lib().nvfp4_gemm(
        _ptr(a_q), _ptr(a_sf), _ptr(a_g), _ptr(b_q), _ptr(b_sf), _ptr(b_g), M, N, 2 * K2, _ptr(c),
        _stream(a_q.device)))
    return c


def grouped_gemm(a_q, a_sf, a_g, b_q, b_sf, b_g, offsets, out=None):
    """MoE grouped GEMM: rows [offsets[e], offsets[e+1]) of A use expert e's
    weight b[e]; C[M][N] = gA*gB[e] * sum_k deq(A)[m][k] deq(B_e)[n][k]."""
    for t, n in ((a_q, "a_q"), (a_sf, "a_sf"), (b_q, "b_q"), (b_sf, "b_sf")):
        _need(t, torch.uint8, n)
    _need(a_g, torch.float32, "a_g")
    _need(b_g, torch.float32, "b_g")
    _need(offsets, torch.int32, "offsets")
    if a_q.dim() != 2 or b_q.dim() != 3:
        raise ValueError("a_q must be [M][K/2] and b_q [experts][N][K/2]")
    M, K2 = a_q.shape
    E, N = b_q.shape[0], b_q.shape[1]
    if offsets.numel() != E + 1 or b_g.numel() != E:
        raise ValueError("offsets must hold experts+1 entries and b_g one scale per expert")
    _shape(b_q, (E, N, K2), "b_q")
    _shape(a_sf, (M, K2 // 8), "a_sf")
    _shape(b_sf, (E, N, K2 // 8), "b_sf")
    _numel(a_g, 1, "a_g")
    if out is not None:
        _need(out, torch.float32, "out")
        _shape(out, (M, N), "out")
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a_q.device)
    _check("nvfp4_grouped_gemm", _lib().nvfp4_grouped_gemm(
        _ptr(a_q), _ptr(a_sf), _ptr(a_g), _ptr(b_q), _ptr(b_sf), _ptr(b_g), _ptr(offsets), E, M, N, 2 * K2,
        _ptr(c), _stream(a_q.device)))
    return c


# ---------------------------------------------------------------- training variants
VAR_COLWISE, VAR_2D, VAR_RHT, VAR_SR = 1, 2, 4, 8


def quantize_ex(x, variant, rht_signs=0, seed=0, offset=0, workspace=None, out=None):
    """Training-recipe quantize of bf16 x [..., rows, cols]: variant is an OR
    of VAR_COLWISE (quantize x^T), VAR_2D (16x16 tile scales), VAR_RHT
    (16-point random Hadamard transform with the sign mask rht_signs) and
    VAR_SR (stochastic element rounding from Philox4x32-10 with seed,
    offset).  Returns (q, sf, g); under VAR_COLWISE they describe x^T."""
    _need(x, torch.bfloat16, "x")
    if x.dim() < 2:
        raise ValueError("x must be [..., rows, cols]")
    rows, cols = x.shape[-2], x.shape[-1]
    lead = tuple(x.shape[:-2])
    batch = 1
    for d in lead:
        batch *= d
    R, C = (cols, rows) if variant & VAR_COLWISE else (rows, cols)
    if out is not None:
        q, sf, g = out
        _need(q, torch.uint8, "q")
        _need(sf, torch.uint8, "sf")
        _need(g, torch.float32, "g")
        _shape(q, lead + (R, C // 2), "q")
        _shape(sf, lead + (R, C // 16), "sf")
        _numel(g, batch, "g")
    else:
        q = torch.empty(lead + (R, C // 2), dtype=torch.uint8, device=x.device)
        sf = torch.empty(lead + (R, C // 16), dtype=torch.uint8, device=x.device)
        g = torch.empty(lead if lead else (1,), dtype=torch.float32, device=x.device)
    wsb = int(_lib().nvfp4_quantize_ex_workspace_bytes(batch))
    if workspace is None:
        workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=x.device)
    _check("nvfp4_quantize_ex", _lib().nvfp4_quantize_ex(
        _ptr(x), batch, rows, cols, variant, rht_signs, seed, offset, _ptr(q), _ptr(sf), _ptr(g),
        _ptr(workspace), workspace.numel(), _stream(x.device)))
    return q, sf, g


# ---------------------------------------------------------------- MXFP4
def mxfp4_quantize(x, out=None):
    """bf16 x [..., cols] (cols % 32 == 0) -> (q [..., cols/2] u8, sf [..., cols/32] u8):
    32-value blocks, one E8M0 (power-of-two) scale each, no tensor scale."""
    _need(x, torch.bfloat16, "x")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    lead = tuple(x.shape[:-1])
    if out is not None:
        q, sf = out
        _need(q, torch.uint8, "q")
        _need(sf, torch.uint8, "sf")
        _shape(q, lead + (cols // 2,), "q")
        _shape(sf, lead + (cols // 32,), "sf")
    else:
        q = torch.empty(lead + (cols // 2,), dtype=torch.uint8, device=x.device)
        sf = torch.empty(lead + (cols // 32,), dtype=torch.uint8, device=x.device)
    _check("nvfp4_mxfp4_quantize", _lib().nvfp4_mxfp4_quantize(
        _ptr(x), rows, cols, _ptr(q), _ptr(sf), _stream(x.device)))
    return q, sf


def mxfp4_dequantize(q, sf, out=None):
    """MXFP4 codes and scale bytes -> bf16 [..., cols]."""
    _need(q, torch.uint8, "q")
    _need(sf, torch.uint8, "sf")
    cols = q.shape[-1] * 2
    rows = q.numel() // q.shape[-1] if q.shape[-1] else 0
    if sf.numel() != rows * (cols // 32):
        raise ValueError("sf must hold one scale byte per 32 values")
    if out is not None:
        _need(out, torch.bfloat16, "out")
        _shape(out, tuple(q.shape[:-1]) + (cols,), "out")
    y = out if out is not None else torch.empty(tuple(q.shape[:-1]) + (cols,), dtype=torch.bfloat16, device=q.device)
    _check("nvfp4_mxfp4_dequantize", _lib().nvfp4_mxfp4_dequantize(
        _ptr(q), _ptr(sf), rows, cols, _ptr(y), _stream(q.device)))
    return y


def mxfp4_gemm(a_q, a_sf, b_q, b_sf, out=None):
    """C[M][N] = sum_k deq(A)[m][k] deq(B)[n][k] on the block-scaled MFMA; fp32 output."""
    for t, n in ((a_q, "a_q"), (a_sf, "a_sf"), (b_q, "b_q"), (b_sf, "b_sf")):
        _need(t, torch.uint8, n)
    M, K2 = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K2 or a_sf.shape != (M, K2 // 16) or b_sf.shape != (N, K2 // 16):
        raise ValueError("operands must be q [rows][K/2] and sf [rows][K/32] with a common K")
    if out is not None:
        _need(out, torch.float32, "out")
        _shape(out, (M, N), "out")
    c = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=a_q.device)
    _check("nvfp4_mxfp4_gemm", _lib().nvfp4_mxfp4_gemm(
        _ptr(a_q), _ptr(a_sf), _ptr(b_q), _ptr(b_sf), M, N, 2 * K2, _ptr(c), _stream(a_q.device)))
    return c
