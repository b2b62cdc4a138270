"""GPU parity: nvfp4_quantize / quantize_with_scale / dequantize against the
CPU oracle, bit for bit (codes, scale bytes, tensor scales, bf16 output)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Guarded, bits, bf16_from_floats, from_bits, np_

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")
FLAGS = ["two_kernel", "fused"]


def assert_quantize_matches(x_gpu, flags="two_kernel", label=""):
    xb = bits(x_gpu)
    q, sf, g = nv.quantize(x_gpu, flags=flags)
    torch.cuda.synchronize()
    assert not torch.isnan(g).any(), f"{label}: persistent launch reported a wait timeout"
    oq, osf, og = oracle.quantize(xb)
    assert np.array_equal(np_(g).view(np.uint32), og.view(np.uint32)), f"{label}: g {np_(g)} vs {og}"
    bad = np.argwhere(np_(sf) != osf)
    assert bad.size == 0, f"{label}: scale byte mismatch at {bad[:5].tolist()}"
    bad = np.argwhere(np_(q) != oq)
    assert bad.size == 0, f"{label}: code mismatch at {bad[:5].tolist()}"
    y = nv.dequantize(q, sf, g)
    oy = oracle.dequantize(oq, osf, og)
    assert np.array_equal(bits(y), oy), f"{label}: dequant mismatch"
    return q, sf, g


@pytest.mark.parametrize("flags", FLAGS)
def test_single_tensor_1024x1024(flags):
    print("case: single 1024x1024 N(0,1) seed 101", flags, flush=True)
    x = synth.single(device="cuda")
    assert_quantize_matches(x, flags, "single")


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (7, 16 * 33), (1, 16 * 4099), (257, 160), (2, 5, 7168)])
def test_ragged_shapes(shape):
    print("case: ragged", shape, flush=True)
    g = torch.Generator().manual_seed(sum(shape))
    x = (torch.randn(shape, generator=g) * 3).to(torch.bfloat16).cuda()
    for fl in FLAGS:
        assert_quantize_matches(x, fl, f"ragged {shape} {fl}")


def _edge_tensors():
    out = {}
    out["all_zero"] = [[0.0] * 64]
    out["signed_zeros"] = [[0.0, -0.0] * 32]
    out["single_nonzero"] = [[0.0] * 37 + [-3.25] + [0.0] * 26]
    out["tiny_amax_subnormal_bf16"] = [[9.2e-41, -1e-40, 5e-39, 0.0] * 16]
    out["huge"] = [[3.3e38, -3.0e38, 1e30, -1.0] * 16]
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    ties = []
    for j in (-9, -4, 0, 3, 7):
        ties += [6.0 * 2 ** j] + [m * 2 ** j for m in mids] + [-m * 2 ** j for m in mids] + [-0.0]
    out["ties_g1"] = [ties + [2688.0] + [0.0] * 15]
    out["e4m3_tie"] = [[6.375] + [0.0] * 15 + [2688.0] + [0.0] * 15]
    out["subnormal_scales"] = [[6 * 1.6 * 2.0 ** -9, 1e-3, 6 * 2.0 ** -10, 2e-3] * 4 + [2688.0] + [0.0] * 15]
    out["wide_range"] = [[2.0 ** e * (1 if e % 2 else -1) for e in range(-60, 4)]]
    return out


@pytest.mark.parametrize("name", sorted(_edge_tensors()))
def test_edge_tensors(name):
    print("case: edge", name, flush=True)
    x = bf16_from_floats(_edge_tensors()[name])
    for fl in FLAGS:
        assert_quantize_matches(x, fl, f"{name} {fl}")


def _sweep_input(g_value, seed):
    """Blocks covering every bf16 magnitude below each block's max, for every
    block-scale byte reachable with tensor scale g."""
    rng = np.random.default_rng(seed)
    rows = []
    allmag = np.arange(0, 0x7F80, dtype=np.uint16)
    allf = (allmag.astype(np.uint32) << 16).view(np.float32)
    for sbyte in range(1, 0x7F):
        s = oracle.e4m3_value(sbyte)
        bam = np.float32(6.0 * s * g_value)
        bam_bits = oracle.f32_to_bf16_array(np.array([bam], dtype=np.float32))[0]
        lim = int(bam_bits)
        if lim == 0 or lim >= 0x7F80:
            continue
        mags = allmag[:lim + 1]
        if mags.size > 4000:            # all of the top 2^11 patterns, a random sample below
            top = mags[-2048:]
            rest = rng.choice(mags[:-2048], 1952, replace=False)
            mags = np.concatenate([top, rest])
        signs = (rng.random(mags.size) < 0.5).astype(np.uint16) << 15
        vals = mags | signs
        pad = (-vals.size) % 15
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 15)
        blk = np.concatenate([np.full((vals.shape[0], 1), bam_bits, dtype=np.uint16), vals], axis=1)
        rows.append(blk.reshape(-1))
    return np.concatenate(rows)


@pytest.mark.parametrize("g_value", [np.float32(0.0123), np.float32(1.0), np.float32(3.7e-5),
                                     np.float32(2.0 ** -100), np.float32(1e30)])
def test_scale_by_magnitude_sweep(g_value):
    """quantize_with_scale: for every E4M3 scale byte, blocks holding (nearly) every
    bf16 magnitude up to the block max -- exercises the reciprocal fast path,
    the danger-magnitude fix-ups and the fully exact path."""
    print("case: sweep g", float(g_value), flush=True)
    flat = _sweep_input(float(g_value), 17)
    cols = 16 * 64
    flat = np.concatenate([flat, np.zeros((-flat.size) % cols, dtype=np.uint16)])
    xb = flat.reshape(1, -1, cols)
    x = from_bits(xb)
    gt = torch.tensor([g_value], dtype=torch.float32, device="cuda")
    q, sf = nv.quantize_with_scale(x, gt)
    torch.cuda.synchronize()
    oq, osf = oracle.quantize_with_scale(xb, np.array([g_value], dtype=np.float32))
    bad = np.argwhere(np_(sf) != osf)
    assert bad.size == 0, f"scale mismatch at {bad[:5].tolist()}"
    bad = np.argwhere(np_(q) != oq)
    assert bad.size == 0, f"code mismatch at {bad[:5].tolist()}: got {np_(q)[tuple(bad[0])]:#x} want {oq[tuple(bad[0])]:#x}"
    y = nv.dequantize(q, sf, gt)
    assert np.array_equal(bits(y), oracle.dequantize(oq, osf, np.array([g_value], dtype=np.float32)))


def test_batch_distinct_magnitudes_and_guards():
    print("case: batch of 5 tensors with different magnitudes, guarded outputs", flush=True)
    b, r, c = 5, 33, 256
    gen = torch.Generator().manual_seed(5)
    x = torch.randn((b, r, c), generator=gen)
    x *= torch.tensor([1e-20, 1e-3, 1.0, 40.0, 1e25]).view(b, 1, 1)
    x[2] = 0.0
    x = x.to(torch.bfloat16).cuda()
    for fl in FLAGS:
        qg = Guarded((b, r, c // 2), torch.uint8)
        sg = Guarded((b, r, c // 16), torch.uint8)
        gg = Guarded((b,), torch.float32)
        nv.quantize(x, flags=fl, out=(qg.view, sg.view, gg.view))
        yg = Guarded((b, r, c), torch.bfloat16)
        nv.dequantize(qg.view, sg.view, gg.view, out=yg.view)
        torch.cuda.synchronize()
        for gd in (qg, sg, gg, yg):
            gd.check()
        oq, osf, og = oracle.quantize(bits(x))
        assert np.array_equal(np_(gg.view), og)
        assert np.array_equal(np_(sg.view), osf) and np.array_equal(np_(qg.view), oq)
        assert np.array_equal(bits(yg.view), oracle.dequantize(oq, osf, og))


def test_quantize_with_scale_equals_quantize():
    x = synth.single(device="cuda", rows=256, cols=512)
    q, sf, g = nv.quantize(x)
    q2, sf2 = nv.quantize_with_scale(x, g)
    assert torch.equal(q, q2) and torch.equal(sf, sf2)


def test_deterministic_reruns():
    x = synth.activations(tokens=512, channels=7168, device="cuda")
    a = nv.quantize(x)
    b = nv.quantize(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_experts_full_size_sampled():
    """64 x [2048 x 7168] expert weights (N(0,0.02), 0.1% x50 outliers): all
    64 tensor scales checked; codes, scales and dequant of 3 experts checked in full."""
    print("case: experts 64x2048x7168 seed 102", flush=True)
    x = synth.experts(device="cuda")
    ws = nv.make_workspace(64, 2048, 7168)
    for fl in FLAGS:
        q, sf, g = nv.quantize(x, flags=fl, workspace=ws)
        y = nv.dequantize(q, sf, g)
        torch.cuda.synchronize()
        amax = x.float().abs().amax(dim=(1, 2)).cpu().numpy()
        og_all = np.array([oracle.global_scale(a) for a in amax], dtype=np.float32)
        assert np.array_equal(np_(g), og_all)
        for e in (0, 31, 63):
            xb = bits(x[e])
            oq, osf, og = oracle.quantize(xb)
            assert og[0] == np_(g)[e]
            assert np.array_equal(np_(sf[e]), osf), f"expert {e} scales"
            assert np.array_equal(np_(q[e]), oq), f"expert {e} codes"
            assert np.array_equal(bits(y[e]), oracle.dequantize(oq, osf, og)), f"expert {e} dequant"
        del q, sf, y
    del x


def test_activations_full_size():
    """16384 x 7168 activations, 0.5 * Student-t(3) with 8 channels x30, in full."""
    print("case: activations 16384x7168 seed 103", flush=True)
    x = synth.activations(device="cuda")
    xb = bits(x)
    oq, osf, og = oracle.quantize(xb)
    for fl in FLAGS:
        q, sf, g = nv.quantize(x, flags=fl)
        torch.cuda.synchronize()
        assert np_(g)[0] == og[0]
        assert np.array_equal(np_(sf), osf)
        assert np.array_equal(np_(q), oq)
        del q, sf


def test_fused_workspace_is_left_clean():
    """The persistent launch restores its counters to zero: many back-to-back
    calls on one workspace, with different batch sizes, all give the two-kernel bytes."""
    gen = torch.Generator().manual_seed(21)
    ws = nv.make_workspace(8, 64, 512)
    for it, b in enumerate([8, 3, 8, 1, 5] * 3):
        x = (torch.randn((b, 64, 512), generator=gen) * (it + 1)).to(torch.bfloat16).cuda()
        a = nv.quantize(x, flags="fused", workspace=ws[:nv.workspace_bytes(b, 64, 512)])
        r = nv.quantize(x, flags="two_kernel")
        for u, v in zip(a, r):
            assert torch.equal(u, v), f"iteration {it}"
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:nv.workspace_bytes(8, 64, 512) - 8 * 2048 * 4]).item() == 0
