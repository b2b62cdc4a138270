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


def _quantized(x):
    """x quantized on the GPU and by the oracle.  The bytes must agree, and the
    expected GEMM is then computed from the oracle's encoding alone."""
    q, sf, g = nv.quantize(x)
    oq, osf, og = oracle.quantize(bits(x))
    assert np.array_equal(np_(q), oq) and np.array_equal(np_(sf), osf), "GPU codes differ from the oracle's"
    assert np.array_equal(np_(g).view(np.uint32), og.view(np.uint32)), "GPU tensor scale differs from the oracle's"
    return (q, sf, g), (oq, osf, og)


def _operands(M, N, K, seed, scale_a=1.0, scale_b=1.0):
    gen = torch.Generator().manual_seed(seed)
    a = (torch.randn((M, K), generator=gen) * scale_a).to(torch.bfloat16).cuda()
    b = (torch.randn((N, K), generator=gen) * scale_b).to(torch.bfloat16).cuda()
    return a, b


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (64, 96, 160), (130, 257, 48), (256, 256, 1024), (96, 200, 576),
                                   (64, 64, 320), (1, 1, 16), (300, 70, 7168), (512, 384, 2048)])
def test_gemm_small(M, N, K):
    print("case: gemm", M, N, K, flush=True)
    a, b = _operands(M, N, K, M * 7 + N * 3 + K)
    (aq, asf, ag), oa = _quantized(a)
    (bq, bsf, bg), ob = _quantized(b)
    c = nv.gemm(aq, asf, ag, bq, bsf, bg)
    torch.cuda.synchronize()
    want = oracle.gemm_f64(oa[0], oa[1], oa[2][0], ob[0], ob[1], ob[2][0])
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


def test_gemm_scales_and_outliers():
    a, b = _operands(256, 192, 512, 3, 1e-3, 40.0)
    a[:, 7] *= 300
    (aq, asf, ag), oa = _quantized(a)
    (bq, bsf, bg), ob = _quantized(b)
    c = nv.gemm(aq, asf, ag, bq, bsf, bg)
    torch.cuda.synchronize()
    want = oracle.gemm_f64(oa[0], oa[1], oa[2][0], ob[0], ob[1], ob[2][0])
    assert rel_frobenius(np_(c), want) <= TOL


def test_gemm_k_zero_gives_zeros():
    aq = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    asf = torch.zeros((64, 0), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, device="cuda")
    c = torch.full((64, 32), 7.0, device="cuda")
    nv.gemm(aq, asf, g, aq[:32], asf[:32], g, out=c)
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


def test_gemm_full_size():
    """A [8192 x 7168] x B [2048 x 7168]^T from N(0,1), the benchmarked shape:
    every element of C against the fp64 product of the oracle's encoding."""
    print("case: gemm 8192x2048x7168 seed 105", flush=True)
    a, b = synth.gemm_operands(device="cuda")
    (aq, asf, ag), oa = _quantized(a)
    (bq, bsf, bg), ob = _quantized(b)
    c = nv.gemm(aq, asf, ag, bq, bsf, bg)
    torch.cuda.synchronize()
    want = oracle.gemm_f64(oa[0], oa[1], oa[2][0], ob[0], ob[1], ob[2][0])
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


@pytest.mark.parametrize("K", [2048, 2032])
def test_gemm_every_scale_byte(K):
    """Raw operands that walk every block-scale byte 0x00..0x7E (subnormal
    E4M3 scales included) and every code nibble, against fp64; K = 2032 is
    not a multiple of the 64-wide K step."""
    print("case: gemm scale-byte sweep K", K, flush=True)
    rng = np.random.default_rng(K)
    M, N = 96, 80
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asf = ((np.arange(M * (K // 16)).reshape(M, K // 16) * 5) % 127).astype(np.uint8)
    bsf = ((np.arange(N * (K // 16)).reshape(N, K // 16) * 3 + 11) % 127).astype(np.uint8)
    ag = np.array([1.0], np.float32)
    bg = np.array([0.5], np.float32)
    dev = [torch.from_numpy(t).cuda() for t in (aq, asf, ag, bq, bsf, bg)]
    c = nv.gemm(*dev)
    torch.cuda.synchronize()
    want = oracle.gemm_f64(aq, asf, 1.0, bq, bsf, 0.5)
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


def test_gemm_picks_single_elements_exactly():
    """B selects one element of A per column (code 1.0, scale byte 0x38 = 1.0,
    gB = 1), so C[m][n] = E2M1(A[m][k_n]) * s(A) exactly: a per-element pin of
    the in-kernel decode for every scale byte and code nibble."""
    rng = np.random.default_rng(7)
    M, K, N = 128, 2048, 128
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    asf = ((np.arange(M * (K // 16)).reshape(M, K // 16) * 7 + 1) % 127).astype(np.uint8)
    ks = np.array([16 * n + (n % 16) for n in range(N)])
    bq = np.zeros((N, K // 2), np.uint8)
    bsf = np.zeros((N, K // 16), np.uint8)
    for n, k in enumerate(ks):
        bq[n, k // 2] = 0x2 << (4 * (k % 2))        # E2M1 code 2 = 1.0
        bsf[n, k // 16] = 0x38                      # E4M3 1.0
    one = np.array([1.0], np.float32)
    dev = [torch.from_numpy(t).cuda() for t in (aq, asf, one, bq, bsf, one)]
    c = np_(nv.gemm(*dev))
    torch.cuda.synchronize()
    want = oracle.dequantize_f64_unscaled(aq, asf)[:, ks]
    np.testing.assert_array_equal(c.astype(np.float64), want)


def _experts_and_routing(E, N, K, counts, seed):
    gen = torch.Generator().manual_seed(seed)
    M = int(sum(counts))
    a = torch.randn((M, K), generator=gen).to(torch.bfloat16).cuda()
    w = (torch.randn((E, N, K), generator=gen) * torch.linspace(0.5, 4.0, E).view(E, 1, 1)).to(torch.bfloat16).cuda()
    (aq, asf, ag), oa = _quantized(a)
    (bq, bsf, bg), ob = _quantized(w)             # one tensor scale per expert
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32).cuda()
    return aq, asf, ag, bq, bsf, bg, offsets, oa, ob


@pytest.mark.parametrize("K", [2048, 2032])
def test_grouped_gemm_against_oracle_and_dense(K):
    """Ragged routing (empty experts, a single-row expert, experts spanning
    several 256-row tiles) against the fp64 oracle, and bit-identical to one
    dense nvfp4_gemm per expert slice."""
    print("case: grouped gemm K", K, flush=True)
    counts = [300, 0, 1, 513, 0, 77, 256, 2]
    E, N = len(counts), 96
    aq, asf, ag, bq, bsf, bg, offsets, oa, ob = _experts_and_routing(E, N, K, counts, K + 5)
    c = nv.grouped_gemm(aq, asf, ag, bq, bsf, bg, offsets)
    torch.cuda.synchronize()
    off = np_(offsets)
    want = oracle.grouped_gemm_f64(oa[0], oa[1], oa[2][0], ob[0], ob[1], ob[2], off)
    err = rel_frobenius(np_(c), want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        # fresh (16-byte aligned) copies of the expert's rows: K/2 need not be a multiple of 16
        d = nv.gemm(aq[r0:r1].clone(), asf[r0:r1].clone(), ag, bq[e], bsf[e], bg[e:e + 1].clone())
        torch.cuda.synchronize()
        assert torch.equal(c[r0:r1], d), f"expert {e} differs from the dense GEMM of its rows"


def test_grouped_gemm_full_size_sampled_rows():
    """The benchmarked MoE shape: 16384 tokens routed top-8 over 64 experts
    [2048 x 7168] (131072 routed rows, seeded uniform routing, activations and
    experts as the bench draws them).  Both operands' encodings are checked
    in full against the oracle; 512 sampled rows of C (all 2048 columns, each
    against its expert's weight) against fp64."""
    print("case: grouped gemm 131072 rows x 64 experts", flush=True)
    T, E, top, N, K = 16384, 64, 8, 2048, 7168
    gen = torch.Generator().manual_seed(106)
    choice = torch.rand((T, E), generator=gen).argsort(dim=1)[:, :top]
    counts = torch.bincount(choice.flatten(), minlength=E)
    off = np.concatenate([[0], np.cumsum(counts.numpy())]).astype(np.int32)
    M = int(off[-1])
    a = synth.activations(tokens=M, channels=K, seed=107, device="cuda")
    (aq, asf, ag), oa = _quantized(a)
    del a
    w = synth.experts(E, N, K, device="cuda")
    (bq, bsf, bg), ob = _quantized(w)
    del w
    c = nv.grouped_gemm(aq, asf, ag, bq, bsf, bg, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(11).choice(M, 512, replace=False))
    got = np_(c[torch.from_numpy(rows).cuda()])
    want = np.empty_like(got, dtype=np.float64)
    expert = np.searchsorted(off, rows, side="right") - 1
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        want[sel] = oracle.gemm_f64(oa[0], oa[1], oa[2][0], ob[0][e], ob[1][e], ob[2][e], rows=rows[sel])
    err = rel_frobenius(got, want)
    assert err <= TOL, f"rel Frobenius {err:.3e}"


def test_grouped_gemm_offsets_past_m_are_clamped():
    """A last offset beyond M is clamped to M: rows inside A are still right."""
    counts = [40, 90]
    aq, asf, ag, bq, bsf, bg, offsets, oa, ob = _experts_and_routing(2, 64, 512, counts, 9)
    offsets[2] = 130 + 1000
    c = nv.grouped_gemm(aq, asf, ag, bq, bsf, bg, offsets)
    torch.cuda.synchronize()
    want = oracle.grouped_gemm_f64(oa[0], oa[1], oa[2][0], ob[0], ob[1], ob[2],
                                   np.array([0, 40, 130], np.int32))
    assert rel_frobenius(np_(c), want) <= TOL
