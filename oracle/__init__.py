"""CPU oracle for NVFP4 two-level microscaling -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never calls it and shares no code with
it.  The codec (quantize / dequantize / KV rows) runs in plain C
(nvfp4_oracle.c, one binary32 rounding per step, brute-force grid rounding);
the contractions (block-scaled GEMM, decode QK) are fp64 definitions built on
the oracle's exact fp64 dequantization plus a library matmul.

Sources of the method: the E2M1 grid, 16-value blocks with an E4M3 scale and
one FP32 tensor scale (axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B
model on 10 trillion tokens", section "E2M1 format and two-level scaling";
theddari.com, "What is FP4 quantization? KV cache in 4 bits", format table);
the KV cache layout per token (theddari.com, same page, "KV cache size
example"); NVFP4 for weights and activations of MoE expert linears
(iwan.kr, "NVIDIA shrank GLM-5.2 to 4 bits", section 1).  The MXFP4 variant
(32-value blocks, one power-of-two scale each, no tensor scale; iwan.kr, same
page, section 3; theddari.com, format table) follows the published
Microscaling exponent rule, which the pages leave open.  The training-recipe
variants (16x16 2D weight scales, a random Hadamard transform of Wgrad
inputs, stochastic rounding of gradients, the column-wise Dgrad/Wgrad
operand layout; axbrief.com, same page, section "Four stabilizers for
training: from RHT to stochastic rounding") run in nvfp4_oracle.c as well,
with their random draws from Philox4x32-10.

Parity pins live in tests/test_oracle_*.py; functions without an independent
pin would say "parity unpinned" here -- every function below has one.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [i32]
        L.orc_e2m1_encode.restype = i32
        L.orc_e2m1_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [i32]
        L.orc_e4m3_encode.restype = i32
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_global_scale.restype = ctypes.c_float
        L.orc_global_scale.argtypes = [ctypes.c_float]
        L.orc_block_scale.restype = i32
        L.orc_block_scale.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_decode_element.restype = ctypes.c_float
        L.orc_decode_element.argtypes = [i32, i32, ctypes.c_float]
        L.orc_max_threads.restype = i32
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [i32]
        L.orc_mx_block_scale.restype = i32
        L.orc_mx_block_scale.argtypes = [ctypes.c_float]
        L.orc_mx_decode_element.restype = ctypes.c_float
        L.orc_mx_decode_element.argtypes = [i32, i32]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_e2m1_encode_sr.restype = i32
        L.orc_e2m1_encode_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
        L.orc_rht16.restype = None
        L.orc_rht16.argtypes = [P, ctypes.c_uint32]
        for name, args in {
            "orc_quantize": [P, i64, i64, i64, P, P, P, i32],
            "orc_quantize_with_scale": [P, i64, i64, i64, P, P, P, i32],
            "orc_dequantize": [P, P, P, i64, i64, i64, P, i32],
            "orc_dequantize_f64_unscaled": [P, P, i64, i64, P, i32],
            "orc_mx_quantize": [P, i64, i64, P, P, i32],
            "orc_mx_dequantize": [P, P, i64, i64, P, i32],
            "orc_mx_dequantize_f64": [P, P, i64, i64, P, i32],
            "orc_quantize_ex": [P, i64, i64, i64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                ctypes.c_uint64, P, P, P],
        }.items():
            getattr(L, name).restype = i32
            getattr(L, name).argtypes = args
        for name, args in {
            "orc_e2m1_encode_array": [P, i64, P, i32],
            "orc_e4m3_encode_array": [P, i64, P, i32],
            "orc_f32_to_bf16_array": [P, i64, P, i32],
        }.items():
            getattr(L, name).restype = None
            getattr(L, name).argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- scalars
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e2m1_encode(y: float) -> int:
    return lib().orc_e2m1_encode(float(y))


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(int(byte))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def global_scale(amax: float) -> float:
    return lib().orc_global_scale(float(amax))


def block_scale(bamax: float, g: float) -> int:
    return lib().orc_block_scale(float(bamax), float(g))


def decode_element(code: int, sbyte: int, g: float) -> float:
    return lib().orc_decode_element(int(code), int(sbyte), float(g))


def e2m1_encode_array(y: np.ndarray, nthreads: int = 0) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.int8)
    lib().orc_e2m1_encode_array(_p(y), y.size, _p(out), nthreads)
    return out


def e4m3_encode_array(v: np.ndarray, nthreads: int = 0) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.int16)
    lib().orc_e4m3_encode_array(_p(v), v.size, _p(out), nthreads)
    return out


def f32_to_bf16_array(f: np.ndarray, nthreads: int = 0) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_p(f), f.size, _p(out), nthreads)
    return out


# ---------------------------------------------------------------- codec
def _shape3(x: np.ndarray):
    if x.ndim == 2:
        return 1, x.shape[0], x.shape[1]
    assert x.ndim == 3
    return x.shape


def quantize(x_bits: np.ndarray, nthreads: int = 0):
    """x_bits: uint16 bf16 bit patterns, [rows][cols] or [batch][rows][cols].

    Returns (q uint8 [..., cols/2], sf uint8 [..., cols/16], g float32 [batch]).
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    b, r, c = _shape3(x_bits)
    lead = x_bits.shape[:-1]
    q = np.empty(lead + (c // 2,), dtype=np.uint8)
    sf = np.empty(lead + (c // 16,), dtype=np.uint8)
    g = np.empty((b,), dtype=np.float32)
    rc = lib().orc_quantize(_p(x_bits), b, r, c, _p(q), _p(sf), _p(g), nthreads)
    if rc != 0:
        raise ValueError("oracle quantize: bad shape or non-finite input")
    return q, sf, g


def quantize_with_scale(x_bits: np.ndarray, g: np.ndarray, nthreads: int = 0):
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    b, r, c = _shape3(x_bits)
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float32).reshape(b))
    lead = x_bits.shape[:-1]
    q = np.empty(lead + (c // 2,), dtype=np.uint8)
    sf = np.empty(lead + (c // 16,), dtype=np.uint8)
    rc = lib().orc_quantize_with_scale(_p(x_bits), b, r, c, _p(g), _p(q), _p(sf), nthreads)
    if rc != 0:
        raise ValueError("oracle quantize_with_scale: bad shape, bad g or non-finite input")
    return q, sf


def dequantize(q: np.ndarray, sf: np.ndarray, g: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Returns bf16 bit patterns (uint16) with q's leading shape and cols = 2*q.shape[-1]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    c = q.shape[-1] * 2
    if q.ndim == 2:
        b, r = 1, q.shape[0]
    else:
        b, r = q.shape[0], q.shape[1]
    if sf.shape != q.shape[:-1] + (c // 16,):
        raise ValueError("oracle dequantize: scales must match the codes' rows, cols/16")
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float32).reshape(b))
    y = np.empty(q.shape[:-1] + (c,), dtype=np.uint16)
    rc = lib().orc_dequantize(_p(q), _p(sf), _p(g), b, r, c, _p(y), nthreads)
    if rc != 0:
        raise ValueError("oracle dequantize: bad shape")
    return y


def dequantize_f64_unscaled(q: np.ndarray, sf: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Exact fp64 E2M1(code)*s per element (tensor scale NOT applied), [rows][cols]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    rows = int(np.prod(q.shape[:-1])) if q.ndim > 1 else 1
    c = q.shape[-1] * 2
    if sf.size != rows * (c // 16):
        raise ValueError("oracle dequantize_f64: scales must match the codes' rows, cols/16")
    y = np.empty(q.shape[:-1] + (c,), dtype=np.float64)
    rc = lib().orc_dequantize_f64_unscaled(_p(q), _p(sf), rows, c, _p(y), nthreads)
    if rc != 0:
        raise ValueError("oracle dequantize_f64: bad shape")
    return y


# ---------------------------------------------------------------- KV cache
def kv_encode(x_new: np.ndarray, g_lh: np.ndarray, nthreads: int = 0):
    """Encode new K (or V) tokens for the cache.

    x_new: bf16 bits [layers][n][kv_heads][head_dim]; g_lh: float32 [layers][kv_heads].
    Each (layer, head, token) head_dim vector is one row of head_dim/16 blocks,
    quantized with that (layer, head)'s caller-supplied tensor scale.
    Returns (q [layers][kv_heads][n][head_dim/2], sf [layers][kv_heads][n][head_dim/16]).
    """
    L, n, H, D = x_new.shape
    xt = np.ascontiguousarray(np.transpose(x_new, (0, 2, 1, 3))).reshape(L * H, n, D)
    q, sf = quantize_with_scale(xt, np.asarray(g_lh, dtype=np.float32).reshape(L * H), nthreads)
    return q.reshape(L, H, n, D // 2), sf.reshape(L, H, n, D // 16)


def kv_read(q: np.ndarray, sf: np.ndarray, g_lh: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Dequantize cache slices q [L][H][n][D/2], sf [L][H][n][D/16] -> bf16 bits [L][H][n][D]."""
    L, H, n, D2 = q.shape
    y = dequantize(q.reshape(L * H, n, D2), sf.reshape(L * H, n, D2 // 8),
                   np.asarray(g_lh, dtype=np.float32).reshape(L * H), nthreads)
    return y.reshape(L, H, n, 2 * D2)


def bf16_bits_to_f64(x_bits: np.ndarray) -> np.ndarray:
    return (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_qk_f64(q_bits: np.ndarray, kq: np.ndarray, ksf: np.ndarray, k_g: np.ndarray) -> np.ndarray:
    """fp64 decode-step logits.

    q_bits [L][Hq][D] bf16 bits; kq [L][H][n][D/2]; ksf [L][H][n][D/16]; k_g [L][H].
    logits[l][hq][t] = sum_d q[l][hq][d] * Khat[l][hq // (Hq/H)][t][d], with
    Khat = E2M1(code) * s * g exactly in fp64.  Returns float64 [L][Hq][n].
    """
    L, Hq, D = q_bits.shape
    _, H, n, _ = kq.shape
    grp = Hq // H
    qd = bf16_bits_to_f64(q_bits)
    out = np.empty((L, Hq, n), dtype=np.float64)
    for l in range(L):
        for h in range(H):
            khat = dequantize_f64_unscaled(kq[l, h], ksf[l, h]) * float(k_g[l, h])
            out[l, h * grp:(h + 1) * grp, :] = qd[l, h * grp:(h + 1) * grp, :] @ khat.T
    return out


def decode_attention_f64(q_bits, kq, ksf, k_g, vq, vsf, v_g, scale) -> np.ndarray:
    """fp64 decode-step attention over the NVFP4 cache (decoding re-reads the
    cache every step: theddari.com, "What is FP4 quantization? KV cache in 4
    bits", section "how does 4-bit KV change inference cost").

    For each layer l and query head hq (KV head hq // (Hq/H)):
      s_t = scale * q . Khat_t,  p = softmax_t(s),  out = sum_t p_t Vhat_t,
    with Khat, Vhat the exact fp64 dequantized values.  Returns [L][Hq][D].
    """
    logits = decode_qk_f64(q_bits, kq, ksf, k_g) * float(scale)
    L, Hq, n = logits.shape
    H, D = kq.shape[1], kq.shape[3] * 2
    grp = Hq // H
    out = np.empty((L, Hq, D), dtype=np.float64)
    for l in range(L):
        for h in range(H):
            vhat = dequantize_f64_unscaled(vq[l, h], vsf[l, h]) * float(v_g[l, h])
            s = logits[l, h * grp:(h + 1) * grp]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[l, h * grp:(h + 1) * grp] = (p @ vhat) / p.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------- GEMM
def gemm_f64(a_q, a_sf, a_g, b_q, b_sf, b_g, rows=None) -> np.ndarray:
    """fp64 block-scaled GEMM  C[m][n] = gA*gB * sum_k deq(A)[m][k] * deq(B)[n][k].

    deq() is the exact fp64 E2M1(code)*s; every product is exact in fp64.
    `rows` optionally restricts to a subset of A's rows (sampled checks).
    """
    if rows is not None:
        a_q = a_q[rows]
        a_sf = a_sf[rows]
    A = dequantize_f64_unscaled(a_q, a_sf)
    B = dequantize_f64_unscaled(b_q, b_sf)
    return (float(a_g) * float(b_g)) * (A @ B.T)


def grouped_gemm_f64(a_q, a_sf, a_g, b_q, b_sf, b_g, offsets) -> np.ndarray:
    """fp64 grouped GEMM of MoE expert linears (iwan.kr, "NVIDIA shrank GLM-5.2
    to 4 bits", section 1: weights and activations of the experts are NVFP4).

    Rows [offsets[e], offsets[e+1]) of A are the tokens routed to expert e;
    each such row is multiplied by expert e's weight b[e] ([N][K]):
      C[m][n] = gA * gB[e] * sum_k deq(A)[m][k] * deq(B_e)[n][k].
    Rows outside every expert's range stay zero.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    M, N = a_q.shape[0], b_q.shape[1]
    C = np.zeros((M, N), dtype=np.float64)
    for e in range(b_q.shape[0]):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            C[r0:r1] = gemm_f64(a_q[r0:r1], a_sf[r0:r1], a_g, b_q[e], b_sf[e], b_g[e])
    return C


# ---------------------------------------------------------------- MXFP4
# 32-value blocks with one power-of-two (E8M0) scale and no tensor scale
# (iwan.kr, "NVIDIA shrank GLM-5.2 to 4 bits", section 3; theddari.com, "What
# is FP4 quantization? KV cache in 4 bits", format comparison table).  The
# exponent rule is the published Microscaling definition; see nvfp4_oracle.c.
def e8m0_value(byte: int) -> float:
    return lib().orc_e8m0_value(int(byte))


def mx_block_scale(bamax: float) -> int:
    return lib().orc_mx_block_scale(float(bamax))


def mx_decode_element(code: int, sbyte: int) -> float:
    return lib().orc_mx_decode_element(int(code), int(sbyte))


def mx_quantize(x_bits: np.ndarray, nthreads: int = 0):
    """x_bits: uint16 bf16 bit patterns [rows][cols] (cols % 32 == 0).
    Returns (q [rows][cols/2] u8, sf [rows][cols/32] u8)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    sf = np.empty((rows, cols // 32), dtype=np.uint8)
    if lib().orc_mx_quantize(_p(x), rows, cols, _p(q), _p(sf), nthreads) != 0:
        raise ValueError("mx_quantize: bad shape or non-finite input")
    return q, sf


def mx_dequantize(q: np.ndarray, sf: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Returns bf16 bit patterns [rows][cols], cols = 2 * q.shape[1]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    rows, cols = q.shape[0], 2 * q.shape[1]
    if sf.shape != (rows, cols // 32):
        raise ValueError("mx_dequantize: scales must be [rows][cols/32]")
    y = np.empty((rows, cols), dtype=np.uint16)
    if lib().orc_mx_dequantize(_p(q), _p(sf), rows, cols, _p(y), nthreads) != 0:
        raise ValueError("mx_dequantize: bad shape")
    return y


def mx_dequantize_f64(q: np.ndarray, sf: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Exact fp64 E2M1(code) * 2^X of every element, [rows][cols]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    rows, cols = q.shape[0], 2 * q.shape[1]
    if sf.shape != (rows, cols // 32):
        raise ValueError("mx_dequantize_f64: scales must be [rows][cols/32]")
    y = np.empty((rows, cols), dtype=np.float64)
    if lib().orc_mx_dequantize_f64(_p(q), _p(sf), rows, cols, _p(y), nthreads) != 0:
        raise ValueError("mx_dequantize_f64: bad shape")
    return y


def mx_gemm_f64(a_q, a_sf, b_q, b_sf, rows=None) -> np.ndarray:
    """fp64 MXFP4 GEMM  C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k] (both
    K-major, exact fp64 dequantization, library matmul).  `rows` optionally
    restricts to a subset of A's rows."""
    if rows is not None:
        a_q = a_q[rows]
        a_sf = a_sf[rows]
    return mx_dequantize_f64(a_q, a_sf) @ mx_dequantize_f64(b_q, b_sf).T


# ---------------------------------------------------------------- training variants
# 16x16 2D weight scales, random Hadamard transform of Wgrad inputs and
# stochastic rounding of gradients (axbrief.com, "NVFP4: how NVIDIA
# pre-trained a 12B model on 10 trillion tokens", section "Four stabilizers
# for training: from RHT to stochastic rounding"); the readings are spelled
# out in nvfp4_oracle.c.
COLWISE, TWO_D, RHT, SR = 1, 2, 4, 8


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.empty(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def e2m1_encode_sr(y: float, u16: int) -> int:
    return lib().orc_e2m1_encode_sr(float(y), int(u16))


def rht16(v, signs: int) -> np.ndarray:
    """fp32 RHT of one 16-value block: H16 (s .* v) / 4 by the fast
    Walsh-Hadamard stages h = 1, 2, 4, 8."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(16)).copy()
    lib().orc_rht16(_p(a), int(signs))
    return a


def quantize_ex(x_bits: np.ndarray, variant: int, signs: int = 0, seed: int = 0, offset: int = 0):
    """Variant quantize of bf16 bits [rows][cols] or [batch][rows][cols].
    Returns (q, sf, g); with COLWISE the outputs describe x^T
    ([batch][cols][rows/2], [batch][cols][rows/16])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    b, r, c = x.shape
    R, C = (c, r) if variant & COLWISE else (r, c)
    q = np.empty((b, R, C // 2), dtype=np.uint8)
    sf = np.empty((b, R, C // 16), dtype=np.uint8)
    g = np.empty(b, dtype=np.float32)
    rc = lib().orc_quantize_ex(_p(x), b, r, c, variant, signs, seed, offset, _p(q), _p(sf), _p(g))
    if rc == -2:
        raise ValueError("quantize_ex: 2D scaling and RHT are not combined")
    if rc != 0:
        raise ValueError("quantize_ex: bad shape or non-finite input")
    return (q[0], sf[0], g) if squeeze else (q, sf, g)
