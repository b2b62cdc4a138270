"""GPU parity: the training-recipe quantize variants (column-wise operand
layout, 16x16 2D scales, random Hadamard transform, stochastic rounding),
bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, bits, from_bits, np_

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")

VARIANTS = [0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13]


def _x(shape, seed, wide=False):
    gen = torch.Generator().manual_seed(seed)
    z = torch.randn(shape, generator=gen)
    if wide:                                             # per-row magnitudes over a wide range
        z = z * torch.exp2(torch.randint(-30, 30, shape[:-1] + (1,), generator=gen).float())
    z.view(-1)[::97] = 0.0
    z.view(-1)[5::211] = -0.0
    return z.to(torch.bfloat16).cuda()


def _check(x, variant, signs=0xB5E1, seed=0x1234_5678_9ABC, offset=17):
    print("case: quantize_ex variant", variant, tuple(x.shape), flush=True)
    q, sf, g = nv.quantize_ex(x, variant, rht_signs=signs, seed=seed, offset=offset)
    torch.cuda.synchronize()
    wq, wsf, wg = oracle.quantize_ex(bits(x), variant, signs=signs, seed=seed, offset=offset)
    np.testing.assert_array_equal(np_(g).reshape(-1), np.asarray(wg).reshape(-1))
    np.testing.assert_array_equal(np_(sf).reshape(wsf.shape), wsf)
    np.testing.assert_array_equal(np_(q).reshape(wq.shape), wq)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [(32, 64), (48, 80), (16, 16), (3, 64, 128), (64, 1040)])
def test_variants_match_oracle(variant, shape):
    _check(_x(shape, sum(shape) + variant, wide=len(shape) == 3), variant)


@pytest.mark.parametrize("variant", [0, 4, 8, 12])
def test_rowwise_variants_any_row_count(variant):
    _check(_x((40, 96), 5), variant)


@pytest.mark.parametrize("variant", [1, 3, 5, 9, 11, 13])
@pytest.mark.parametrize("shape", [(272, 528), (528, 48), (2, 800, 1056), (256, 512)])
def test_colwise_variants_over_several_row_blocks(variant, shape):
    """COLWISE output is written per block of 256 input rows x 512 columns:
    shapes with a ragged last block (rows % 256 = 16 or 32), output rows of
    codes that start only 8-byte aligned (rows % 32 = 16), a ragged column
    band, and one exact block."""
    _check(_x(shape, sum(shape) * 3 + variant, wide=len(shape) == 3), variant)


@pytest.mark.parametrize("variant", [2, 3])
@pytest.mark.parametrize("shape", [(5, 48, 1040), (2, 512, 7168), (1, 16, 16), (7, 32, 4096), (2, 400, 80),
                                   (3, 128, 512), (2, 256, 1024), (1, 128, 192)])
def test_2d_single_launch_shapes(shape, variant):
    """2D (row-major or transposed outputs) runs as one launch
    when a tensor's 16 x 8 strips fit on the chip: strip rows that cross
    workgroup boundaries (cols = 1040), 64 workgroups per tensor, a single
    tile, a batch of 7, and strip blocks cut by the tensor's edge in both
    directions (400 x 80: 25 strip rows, 10 strip columns); per-tensor
    magnitudes span 60 binades.  The transposed layout stages its scale
    bytes through LDS when every 8 x 8 block of strips is whole: a
    workgroup's blocks in 8 column bands (128 x 512), alternating between two
    bands (256 x 1024), and 3 blocks in the last workgroup's 8 (128 x 192)."""
    _check(_x(shape, sum(shape) * 5 + variant, wide=True), variant)


@pytest.mark.parametrize("variant", [2, 3])
def test_2d_ignores_stale_workspace_contents(variant):
    """The single-launch 2D path clears its exchange words itself: a
    workspace full of 0xFF bytes gives the same bytes as a fresh one."""
    x = _x((3, 64, 512), 31, wide=True)
    wsb = nv.lib().nvfp4_quantize_ex_workspace_bytes(3)
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda")
    a = nv.quantize_ex(x, variant, workspace=ws)
    b = nv.quantize_ex(x, variant, workspace=ws)
    c = nv.quantize_ex(x, variant)
    torch.cuda.synchronize()
    for u, v, w in zip(a, b, c):
        assert torch.equal(u, w) and torch.equal(v, w)


@pytest.mark.parametrize("variant", [2, 3])
def test_2d_too_large_for_one_launch(variant):
    """A 4096 x 7168 tensor has twice the strips the chip holds, so 2D
    takes the two-pass path; same bytes as the oracle."""
    print("case: 2D 4096x7168 (two-pass), variant", variant, flush=True)
    _check(_x((4096, 7168), 41 + variant), variant)


@pytest.mark.parametrize("variant", [2, 3])
def test_2d_experts_full_size(variant):
    """2D scales on the 64 x [2048 x 7168] expert weights (the single-launch
    path at its full size), row-major and transposed outputs, every byte
    against the oracle."""
    print("case: 2D experts 64x2048x7168, variant", variant, flush=True)
    x = synth.experts(device="cuda")
    q, sf, g = nv.quantize_ex(x, variant)
    torch.cuda.synchronize()
    wq, wsf, wg = oracle.quantize_ex(bits(x), variant, signs=0, seed=0, offset=0)
    assert np.array_equal(np_(g).reshape(-1).view(np.uint32), np.asarray(wg, dtype=np.float32).reshape(-1).view(np.uint32))
    assert np.array_equal(np_(sf).reshape(wsf.shape), wsf)
    assert np.array_equal(np_(q).reshape(wq.shape), wq)


def test_variant_zero_equals_plain_quantize():
    x = _x((2, 128, 256), 6, wide=True)
    q, sf, g = nv.quantize_ex(x, 0)
    q0, sf0, g0 = nv.quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(sf, sf0) and torch.equal(g, g0)


def test_sr_seed_and_offset_change_the_draws():
    x = _x((64, 256), 7)
    a = nv.quantize_ex(x, nv.VAR_SR, seed=1)[0]
    b = nv.quantize_ex(x, nv.VAR_SR, seed=2)[0]
    c = nv.quantize_ex(x, nv.VAR_SR, seed=1, offset=1)[0]
    d = nv.quantize_ex(x, nv.VAR_SR, seed=1)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, d) and not torch.equal(a, b) and not torch.equal(a, c)


def _every_magnitude_blocks(reps, seed):
    """bf16 bit patterns [reps + 1][cols]: row 0 holds 2688 in a block of its
    own, so the tensor scale is exactly 1; every other block holds 6.0 and 15
    of the finite bf16 magnitudes in [0, 6] (all of them across a row), with
    random signs, so its E4M3 scale is exactly 1 and each value's quotient is
    the value itself."""
    mags = np.arange(0, 0x40C1, dtype=np.uint16)                  # +0 .. 6.0, every finite bf16
    nblk = -(-mags.size // 15)
    body = np.zeros((nblk, 16), dtype=np.uint16)
    body[:, 0] = 0x40C0                                           # 6.0
    flat = np.zeros(nblk * 15, dtype=np.uint16)
    flat[:mags.size] = mags
    body[:, 1:] = flat.reshape(nblk, 15)
    cols = 16 * (nblk + 1)
    rng = np.random.default_rng(seed)
    x = np.zeros((reps + 1, cols), dtype=np.uint16)
    x[0, 0] = 0x4528                                              # 2688
    for r in range(1, reps + 1):
        rows = body[rng.permutation(nblk)].reshape(-1)
        x[r, 16:] = rows | (rng.integers(0, 2, rows.size, dtype=np.uint16) << 15)
    return x


@pytest.mark.parametrize("variant", [nv.VAR_SR, nv.VAR_COLWISE | nv.VAR_SR])
def test_sr_decision_every_bf16_magnitude(variant):
    """Stochastic rounding of every finite bf16 magnitude up to 6 as the
    quotient itself (tensor and block scales exactly 1), 64 draws each: all
    three regimes of the rule (below 0.5, [0.5, 1), the binades from 1), the
    grid points themselves, and ties between the draw and the fraction
    (draws that are multiples of 1024 against 8-bit mantissas); every byte
    against the oracle."""
    if variant & nv.VAR_COLWISE:                                  # blocks run down the columns
        xb = np.ascontiguousarray(_every_magnitude_blocks(63, 2024).T)
    else:
        xb = _every_magnitude_blocks(64, 2024)
    x = from_bits(xb)
    print("case: SR every bf16 magnitude, variant", variant, tuple(x.shape), flush=True)
    _check(x, variant, signs=0, seed=0x5EED, offset=3)
    q, sf, g = nv.quantize_ex(x, variant, seed=0x5EED, offset=3)
    torch.cuda.synchronize()
    assert float(np_(g).reshape(-1)[0]) == 1.0


def test_outputs_stay_in_bounds():
    x = _x((48, 80), 8)
    for variant in (1, 2, 3, 13):
        R, C = (80, 48) if variant & 1 else (48, 80)
        q = Guarded((R, C // 2), torch.uint8)
        sf = Guarded((R, C // 16), torch.uint8)
        g = Guarded((1,), torch.float32)
        nv.quantize_ex(x, variant, out=(q.view, sf.view, g.view))
        torch.cuda.synchronize()
        q.check()
        sf.check()
        g.check()


def test_rejected_combinations():
    x = _x((32, 64), 9)
    with pytest.raises(nv.NVFP4Error):
        nv.quantize_ex(x, nv.VAR_2D | nv.VAR_RHT)
    with pytest.raises(nv.NVFP4Error):
        nv.quantize_ex(_x((24, 64), 9), nv.VAR_COLWISE)
    with pytest.raises(nv.NVFP4Error):
        nv.quantize_ex(x, 16)
    with pytest.raises(nv.NVFP4Error):
        nv.quantize_ex(x, nv.VAR_RHT, rht_signs=1 << 16)


def test_2d_weight_and_its_transpose_agree():
    """One 2048 x 7168 expert weight: 2D scaling of W and of W^T (COLWISE)
    give transposed codes and scales, and both match the oracle."""
    w = synth.experts(1, 2048, 7168, device="cuda")[0]
    print("case: 2D expert weight 2048x7168", flush=True)
    q, sf, g = nv.quantize_ex(w, nv.VAR_2D)
    qt, sft, gt = nv.quantize_ex(w, nv.VAR_2D | nv.VAR_COLWISE)
    torch.cuda.synchronize()
    wq, wsf, wg = oracle.quantize_ex(bits(w), oracle.TWO_D)
    np.testing.assert_array_equal(np_(q), wq)
    np.testing.assert_array_equal(np_(sf), wsf)
    assert np_(g)[0] == wg[0] == np_(gt)[0]
    nib = lambda a: np.stack([a & 15, a >> 4], axis=-1).reshape(a.shape[0], -1)
    np.testing.assert_array_equal(nib(np_(qt)), nib(np_(q)).T)
    np.testing.assert_array_equal(np_(sft)[::16], np_(sf)[::16].T)


@pytest.mark.parametrize("variant", [nv.VAR_SR, nv.VAR_COLWISE | nv.VAR_RHT | nv.VAR_SR])
def test_sr_variants_on_the_activations_full_size(variant):
    """The benchmarked training variants on the full 16384 x 7168 activations
    (RHT signs 0x6A3C, SR seed 77): row-wise SR, and the Wgrad operand
    quantized along the tokens (COLWISE) with RHT and SR; every byte against
    the oracle."""
    a = synth.activations(device="cuda")
    _check(a, variant, signs=0x6A3C, seed=77, offset=0)
