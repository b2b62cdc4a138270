"""GPU parity: MXFP4 quantize / dequantize (bit-exact) and the MXFP4 GEMM on
the block-scaled MFMA (relative Frobenius error <= 1e-5 against fp64)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, bits, from_bits, np_, rel_frobenius

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")
TOL = 1e-5


def _mixed(rows, cols, seed):
    """Per-block magnitudes from 2^-140 to 2^100 (clamped exponents, bf16
    subnormals), zeros, signed zeros, exact ties, and values between 6 and 8
    times the block scale (saturation)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, cols))
    blk = 2.0 ** rng.integers(-140, 100, (rows, cols // 32)).astype(np.float64)
    z = z * blk.repeat(32, axis=1)
    z[rng.random((rows, cols)) < 0.02] = 0.0
    z[rng.random((rows, cols)) < 0.01] = -0.0
    # a few blocks of exact grid values and midpoints: 5 (tie 4|6), 7.5 (saturates), 0.25 (tie 0|0.5)
    for r in range(0, rows, 7):
        row = np.array([7.5, 5.0, 0.25, 2.5, -3.5, 1.25, 0.75, -7.0] * 4)
        z[r, :32] = row * 2.0 ** (r % 40 - 20)
    return np.clip(z, -3e38, 3e38)


@pytest.mark.parametrize("rows,cols,seed", [(1, 32, 1), (7, 96, 2), (64, 2048, 3), (13, 7168, 4), (3, 64, 5),
                                            (1000, 160, 6)])
def test_mx_quantize_matches_oracle(rows, cols, seed):
    print("case: mx quantize", rows, cols, seed, flush=True)
    x = torch.from_numpy(_mixed(rows, cols, seed)).to(torch.bfloat16).cuda()
    q = Guarded((rows, cols // 2), torch.uint8)
    sf = Guarded((rows, cols // 32), torch.uint8)
    nv.mxfp4_quantize(x, out=(q.view, sf.view))
    torch.cuda.synchronize()
    q.check()
    sf.check()
    wq, wsf = oracle.mx_quantize(bits(x))
    np.testing.assert_array_equal(np_(sf.view), wsf)
    np.testing.assert_array_equal(np_(q.view), wq)


def test_mx_quantize_batched_leading_dims():
    x = torch.from_numpy(_mixed(24, 256, 9)).to(torch.bfloat16).cuda().reshape(2, 3, 4, 256)
    q, sf = nv.mxfp4_quantize(x)
    torch.cuda.synchronize()
    wq, wsf = oracle.mx_quantize(bits(x.reshape(24, 256)))
    np.testing.assert_array_equal(np_(q).reshape(24, 128), wq)
    np.testing.assert_array_equal(np_(sf).reshape(24, 8), wsf)


def test_mx_dequantize_every_code_and_scale_byte():
    """Every code nibble under every scale byte 0..255 (subnormal, overflow to
    inf, NaN for 255) against the oracle's bf16 bits."""
    codes = np.arange(16, dtype=np.uint8)
    q = np.tile((codes[0::2] | (codes[1::2] << 4)).reshape(1, 8), (256, 2))       # [256][16] = 32 values per row
    sf = np.arange(256, dtype=np.uint8).reshape(256, 1)
    y = Guarded((256, 32), torch.bfloat16)
    nv.mxfp4_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(sf).cuda(), out=y.view)
    torch.cuda.synchronize()
    y.check()
    got = bits(y.view)
    want = oracle.mx_dequantize(q, sf)
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_w = (want & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal(nan_g, nan_w)
    np.testing.assert_array_equal(got[~nan_w], want[~nan_w])


@pytest.mark.parametrize("rows,cols", [(1, 32), (33, 224), (512, 7168)])
def test_mx_dequantize_random_bytes(rows, cols):
    rng = np.random.default_rng(rows + cols)
    q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    sf = rng.integers(60, 200, (rows, cols // 32), dtype=np.uint8)
    y = nv.mxfp4_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(sf).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y), oracle.mx_dequantize(q, sf))


def test_mx_round_trip_of_the_experts_tensor():
    """The 64 x 2048 x 7168 experts tensor: quantize and dequantize on the GPU,
    every code, scale byte and dequantized value against the oracle."""
    print("case: mx experts 64x2048x7168 seed 102", flush=True)
    x = synth.experts(device="cuda")
    q, sf = nv.mxfp4_quantize(x)
    y = nv.mxfp4_dequantize(q, sf)
    torch.cuda.synchronize()
    wq, wsf = oracle.mx_quantize(bits(x.reshape(-1, 7168)))
    assert np.array_equal(np_(q.reshape(-1, 3584)), wq), "codes"
    assert np.array_equal(np_(sf.reshape(-1, 224)), wsf), "scale bytes"
    assert np.array_equal(bits(y.reshape(-1, 7168)), oracle.mx_dequantize(wq, wsf)), "dequantized values"


def test_mx_rejects_bad_shapes():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        nv.mxfp4_quantize(x)
    L = nv.lib()
    assert L.nvfp4_mxfp4_gemm(None, None, None, None, 4, 4, 48, None, None) == -1      # K % 32
    assert L.nvfp4_mxfp4_quantize(None, 0, 64, None, None, None) == 0                  # empty: no-op


def _mx_quantized(x):
    """x in MXFP4 on the GPU and by the oracle.  The bytes must agree, and the
    expected GEMM is then computed from the oracle's encoding alone."""
    q, sf = nv.mxfp4_quantize(x)
    oq, osf = oracle.mx_quantize(bits(x))
    assert np.array_equal(np_(q), oq) and np.array_equal(np_(sf), osf), "GPU MXFP4 bytes differ from the oracle's"
    return (q, sf), (oq, osf)


def _mx_operands(M, N, K, seed, sa=1.0, sb=1.0):
    gen = torch.Generator().manual_seed(seed)
    a = (torch.randn((M, K), generator=gen) * sa).to(torch.bfloat16).cuda()
    b = (torch.randn((N, K), generator=gen) * sb).to(torch.bfloat16).cuda()
    (aq, asf), oa = _mx_quantized(a)
    (bq, bsf), ob = _mx_quantized(b)
    return aq, asf, bq, bsf, oa, ob


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (64, 96, 96), (300, 257, 544), (1, 1, 32), (512, 384, 2048),
                                   (130, 70, 7168), (256, 512, 4096)])
def test_mx_gemm_matches_oracle(M, N, K):
    print("case: mx gemm", M, N, K, flush=True)
    aq, asf, bq, bsf, oa, ob = _mx_operands(M, N, K, M * 5 + N + K)
    c = Guarded((M, N), torch.float32)
    nv.mxfp4_gemm(aq, asf, bq, bsf, out=c.view)
    torch.cuda.synchronize()
    c.check()
    want = oracle.mx_gemm_f64(oa[0], oa[1], ob[0], ob[1])
    err = rel_frobenius(np_(c.view), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


@pytest.mark.parametrize("K", [2048, 2080])
def test_mx_gemm_every_block_scale_and_code(K):
    """Raw codes and scale bytes that differ block by block (each K step's 8
    blocks carry different exponents), against fp64; K = 2080 ends in a
    ragged step."""
    print("case: mx gemm raw bytes K", K, flush=True)
    rng = np.random.default_rng(K)
    M, N = 96, 80
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = (100 + (np.arange(M * (K // 32)).reshape(M, K // 32) * 5) % 50).astype(np.uint8)
    bsf = (110 + (np.arange(N * (K // 32)).reshape(N, K // 32) * 3) % 40).astype(np.uint8)
    dev = [torch.from_numpy(t).cuda() for t in (aq, asf, bq, bsf)]
    c = nv.mxfp4_gemm(*dev)
    torch.cuda.synchronize()
    want = oracle.mx_gemm_f64(aq, asf, bq, bsf)
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


def test_mx_gemm_picks_single_elements_exactly():
    """Each column of B selects one element of A (code 1.0 at scale 2^0), so
    C[m][n] = E2M1(A[m][k_n]) * 2^X exactly: a per-element pin of the
    operand layout, the nibble order and the scale byte selection."""
    rng = np.random.default_rng(17)
    M, K, N = 64, 1024, 128
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asf = (112 + (np.arange(M * (K // 32)).reshape(M, K // 32) * 7) % 30).astype(np.uint8)
    ks = np.array([8 * n + (n % 8) for n in range(N)])
    bq = np.zeros((N, K // 2), np.uint8)
    bsf = np.full((N, K // 32), 127, np.uint8)
    for n, k in enumerate(ks):
        bq[n, k // 2] = 0x2 << (4 * (k % 2))        # E2M1 code 2 = 1.0
    dev = [torch.from_numpy(t).cuda() for t in (aq, asf, bq, bsf)]
    c = np_(nv.mxfp4_gemm(*dev))
    torch.cuda.synchronize()
    want = oracle.mx_dequantize_f64(aq, asf)[:, ks]
    np.testing.assert_array_equal(c.astype(np.float64), want)


def test_mx_gemm_k_zero_gives_zeros():
    aq = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    c = torch.full((64, 32), 7.0, device="cuda")
    nv.mxfp4_gemm(aq, aq, aq[:32], aq[:32], out=c)
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


def test_mx_gemm_full_size():
    """A [8192 x 7168] x B [2048 x 7168]^T from N(0,1) in MXFP4, the benchmarked
    shape: every element of C against fp64."""
    print("case: mx gemm 8192x2048x7168 seed 105", flush=True)
    a, b = synth.gemm_operands(device="cuda")
    (aq, asf), oa = _mx_quantized(a)
    (bq, bsf), ob = _mx_quantized(b)
    c = nv.mxfp4_gemm(aq, asf, bq, bsf)
    torch.cuda.synchronize()
    want = oracle.mx_gemm_f64(oa[0], oa[1], ob[0], ob[1])
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"
