"""GPU parity: block-scaled NVFP4 x NVFP4 GEMM against the fp64 oracle
(relative Frobenius error <= 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bits, np_, rel_frobenius

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")
TOL = 1e-5


def _operands(M, N, K, seed, scale_a=1.0, scale_b=1.0):
    gen = torch.Generator().manual_seed(seed)
    a = (torch.randn((M, K), generator=gen) * scale_a).to(torch.bfloat16).cuda()
    b = (torch.randn((N, K), generator=gen) * scale_b).to(torch.bfloat16).cuda()
    return a, b


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (64, 96, 160), (130, 257, 48), (256, 256, 1024),
                                   (1, 1, 16), (300, 70, 7168), (512, 384, 2048)])
def test_gemm_small(M, N, K):
    print("case: gemm", M, N, K, flush=True)
    a, b = _operands(M, N, K, M * 7 + N * 3 + K)
    aq, asf, ag = nv.quantize(a)
    bq, bsf, bg = nv.quantize(b)
    c = nv.gemm(aq, asf, ag, bq, bsf, bg)
    torch.cuda.synchronize()
    want = oracle.gemm_f64(np_(aq), np_(asf), np_(ag)[0], np_(bq), np_(bsf), np_(bg)[0])
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


def test_gemm_scales_and_outliers():
    a, b = _operands(256, 192, 512, 3, 1e-3, 40.0)
    a[:, 7] *= 300
    aq, asf, ag = nv.quantize(a)
    bq, bsf, bg = nv.quantize(b)
    c = nv.gemm(aq, asf, ag, bq, bsf, bg)
    torch.cuda.synchronize()
    want = oracle.gemm_f64(np_(aq), np_(asf), np_(ag)[0], np_(bq), np_(bsf), np_(bg)[0])
    assert rel_frobenius(np_(c), want) <= TOL


def test_gemm_k_zero_gives_zeros():
    aq = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    asf = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    c = torch.full((64, 32), 7.0, device="cuda")
    nv.gemm(aq, asf, g, aq[:32], asf[:32], g, out=c)
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


def test_gemm_full_size_sampled_rows():
    """A [8192 x 7168] x B [2048 x 7168]^T from N(0,1): 96 sampled rows of C
    (all 2048 columns) against fp64."""
    print("case: gemm 8192x2048x7168 seed 105", flush=True)
    a, b = synth.gemm_operands(device="cuda")
    aq, asf, ag = nv.quantize(a)
    bq, bsf, bg = nv.quantize(b)
    c = nv.gemm(aq, asf, ag, bq, bsf, bg)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(8192, 96, replace=False))
    want = oracle.gemm_f64(np_(aq), np_(asf), np_(ag)[0], np_(bq), np_(bsf), np_(bg)[0], rows=rows)
    err = rel_frobenius(np_(c[torch.from_numpy(rows).cuda()]), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"
