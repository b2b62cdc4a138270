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


# Tensor scales of the conversion sweeps: round values, inexact decimals,
# extremes whose block divisors reach the top and bottom of the fp32 range.
SWEEP_G = [np.float32(v) for v in (0.0123, 1.0, 3.7e-5, 2.0 ** -100, 1e30, 1.0 / 3.0, 0.1, 7.77e-12)]
ALL_MAGS = np.arange(0, 0x7F80, dtype=np.uint16)          # every finite bf16 magnitude, +0 included


def _bf16_value(bits16):
    return float((np.uint32(bits16) << np.uint32(16)).view(np.float32))


def _largest_bamax_per_scale(g_value, cap=0x7F7F):
    """For tensor scale g: each block-scale byte reachable with g, with the
    largest bf16 magnitude (<= cap) whose block takes that byte (the oracle
    decides which byte a block amax maps to)."""
    out = {}
    for m in range(0, cap + 1):
        s = oracle.block_scale(_bf16_value(m), float(g_value))
        out[s] = m                                      # ascending m: the last one wins
    return out


def _element_sweep_input(g_value, seed, cap=0x7F7F):
    """Blocks that put every finite bf16 magnitude up to the block amax (both
    signs drawn at random) through the element quotient and the E2M1
    conversion, for every block-scale byte reachable with tensor scale g.
    The block amax rotates over the 16 positions."""
    rng = np.random.default_rng(seed)
    rows = []
    blk = 0
    for sbyte, bam in sorted(_largest_bamax_per_scale(g_value, cap).items()):
        mags = ALL_MAGS[:bam + 1]
        signs = (rng.random(mags.size) < 0.5).astype(np.uint16) << 15
        vals = mags | signs
        vals = np.concatenate([vals, np.zeros((-vals.size) % 15, dtype=np.uint16)]).reshape(-1, 15)
        n = vals.shape[0]
        out = np.empty((n, 16), dtype=np.uint16)
        pos = (blk + np.arange(n)) % 16
        for i in range(n):
            out[i] = np.insert(vals[i], pos[i], np.uint16(bam))
        blk += n
        rows.append(out.reshape(-1))
    return np.concatenate(rows)


def _pad_rows(flat, cols=1024):
    flat = np.concatenate([flat, np.zeros((-flat.size) % cols, dtype=np.uint16)])
    return flat.reshape(1, -1, cols)


def _check_with_scale(xb, g_value, what):
    x = from_bits(xb)
    gt = torch.tensor([g_value], dtype=torch.float32, device="cuda")
    q, sf = nv.quantize_with_scale(x, gt)
    torch.cuda.synchronize()
    oq, osf = oracle.quantize_with_scale(xb, np.array([g_value], dtype=np.float32))
    bad = np.argwhere(np_(sf) != osf)
    assert bad.size == 0, f"{what}: scale mismatch at {bad[:5].tolist()}"
    bad = np.argwhere(np_(q) != oq)
    assert bad.size == 0, f"{what}: code mismatch at {bad[:5].tolist()}: got {np_(q)[tuple(bad[0])]:#x} " \
                          f"want {oq[tuple(bad[0])]:#x}"
    y = nv.dequantize(q, sf, gt)
    assert np.array_equal(bits(y), oracle.dequantize(oq, osf, np.array([g_value], dtype=np.float32))), \
        f"{what}: dequantize mismatch"


@pytest.mark.parametrize("g_value", SWEEP_G)
def test_element_conversion_sweep(g_value):
    """quantize_with_scale, reachable domain of the element path: for every
    E4M3 scale byte reachable with tensor scale g, blocks holding every finite
    bf16 magnitude up to the block amax.  Every quotient RN32(|x| / RN32(s g))
    the encode can form with this g goes through the fp64 reciprocal and the
    hardware E2M1 conversion, and every code through the dequantize."""
    print("case: element sweep g", float(g_value), flush=True)
    xb = _pad_rows(_element_sweep_input(g_value, 17))
    _check_with_scale(xb, g_value, f"g={float(g_value)}")


@pytest.mark.parametrize("g_value", SWEEP_G)
def test_block_scale_conversion_sweep(g_value):
    """quantize_with_scale, reachable domain of the block-scale path: one
    block per finite bf16 magnitude as its amax (the rest of the block drawn
    below it), so the E4M3 conversion sees every quotient RN32(bamax /
    RN32(6 g)) that tensor scale g allows."""
    print("case: block-scale sweep g", float(g_value), flush=True)
    rng = np.random.default_rng(29)
    n = ALL_MAGS.size
    fill = (rng.random((n, 15)) * (ALL_MAGS.astype(np.float64)[:, None] + 1)).astype(np.uint16)
    fill = np.minimum(fill, ALL_MAGS[:, None]) | ((rng.random((n, 15)) < 0.5).astype(np.uint16) << 15)
    pos = np.arange(n) % 16
    blocks = np.empty((n, 16), dtype=np.uint16)
    for i in range(n):
        blocks[i] = np.insert(fill[i], pos[i], ALL_MAGS[i] | (np.uint16(i & 1) << 15))
    _check_with_scale(_pad_rows(blocks.reshape(-1)), g_value, f"g={float(g_value)}")


@pytest.mark.parametrize("flags", FLAGS)
def test_element_sweep_through_tensor_amax(flags):
    """The element sweep for g = 1 through nvfp4_quantize itself (amax pass,
    tensor scale, both launch modes): block amaxes capped at 2688 and one
    block holding 2688, so RN32(amax / 2688) = 1."""
    print("case: element sweep through the tensor amax", flags, flush=True)
    flat = _element_sweep_input(np.float32(1.0), 31, cap=0x4528)        # 0x4528 = bf16(2688)
    amax_blk = np.zeros(16, dtype=np.uint16)
    amax_blk[5] = 0x4528
    xb = _pad_rows(np.concatenate([flat, amax_blk]))
    q, sf, g = assert_quantize_matches(from_bits(xb), flags, f"sweep {flags}")
    assert np_(g)[0] == np.float32(1.0)


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


def test_experts_full_size():
    """64 x [2048 x 7168] expert weights (N(0,0.02), 0.1% x50 outliers), the
    headline workload: tensor scales, codes, scale bytes and dequantized values
    of all 64 experts, both launch modes, bit for bit against one oracle pass."""
    print("case: experts 64x2048x7168 seed 102", flush=True)
    x = synth.experts(device="cuda")
    oq, osf, og = oracle.quantize(bits(x))
    oy = oracle.dequantize(oq, osf, og)
    ws = nv.make_workspace(64, 2048, 7168)
    for fl in FLAGS:
        q, sf, g = nv.quantize(x, flags=fl, workspace=ws)
        y = nv.dequantize(q, sf, g)
        torch.cuda.synchronize()
        assert np.array_equal(np_(g).view(np.uint32), og.view(np.uint32)), f"{fl}: tensor scales"
        for e in range(64):
            assert np.array_equal(np_(sf[e]), osf[e]), f"{fl}: expert {e} scales"
            assert np.array_equal(np_(q[e]), oq[e]), f"{fl}: expert {e} codes"
            assert np.array_equal(bits(y[e]), oy[e]), f"{fl}: expert {e} dequant"
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


def _chunk_elems():
    """Elements one FUSED on-chip pass holds for a tensor too large for the
    chip: one workgroup per CU x 512 threads x 14 half blocks of 8."""
    return torch.cuda.get_device_properties(0).multi_processor_count * 512 * 14 * 8


# (chunks, which chunk holds the planted maximum, batch): every pass-2 tail
# (nc mod 3), the maximum in a streamed chunk, the staged chunk nc-4 and
# each register-held chunk, and tensors of two and three chunks (read once).
BIG_CASES = [(2, 0, 1), (2, 1, 3), (3, 2, 1), (3, 0, 2), (4, 0, 1), (5, 0, 1), (5, 3, 2), (6, 2, 1), (7, 6, 1),
             (8, 5, 1)]


@pytest.mark.parametrize("nc,hot,batch", BIG_CASES)
def test_big_tensor_chunks(nc, hot, batch):
    """Tensors of 2..8 on-chip chunks (the single-launch path for tensors
    larger than the chip), ragged last chunk, guarded outputs."""
    cols = 7168
    elems = (nc - 1) * _chunk_elems() + 3 * cols * 37   # the last chunk partly filled
    rows = -(-elems // cols)
    print(f"case: big tensor nc={nc} hot={hot} batch={batch} rows={rows}", flush=True)
    gen = torch.Generator().manual_seed(1000 + 10 * nc + hot)
    x = (torch.randn((batch, rows, cols), generator=gen) * 2).to(torch.bfloat16)
    flat = x.view(batch, -1)
    pos = min(hot * _chunk_elems() + 12345, rows * cols - 1)
    flat[0, pos] = 3.0e4
    if batch > 1:
        flat[1, 77] = -5.0e5
    x = x.cuda()
    qg = Guarded((batch, rows, cols // 2), torch.uint8)
    sg = Guarded((batch, rows, cols // 16), torch.uint8)
    gg = Guarded((batch,), torch.float32)
    nv.quantize(x, flags="fused", out=(qg.view, sg.view, gg.view))
    torch.cuda.synchronize()
    for gd in (qg, sg, gg):
        gd.check()
    oq, osf, og = oracle.quantize(bits(x))
    assert np.array_equal(np_(gg.view).view(np.uint32), og.view(np.uint32)), f"g {np_(gg.view)} vs {og}"
    bad = np.argwhere(np_(sg.view) != osf)
    assert bad.size == 0, f"scale byte mismatch at {bad[:5].tolist()}"
    bad = np.argwhere(np_(qg.view) != oq)
    assert bad.size == 0, f"code mismatch at {bad[:5].tolist()}"


def test_streaming_fused_over_2gib():
    """A 65536 x 16384 tensor (2 GiB of bf16) is past the 32-bit offsets of
    the single-launch kernels, so FUSED runs the streaming kernel (pass 1 of
    tensor t beside pass 2 of tensor t-1); bit for bit against the oracle."""
    print("case: streaming fused, 65536x16384", flush=True)
    x = synth.normal((1, 65536, 16384), 1.5, seed=777, device="cuda")
    q, sf, g = nv.quantize(x, flags="fused")
    torch.cuda.synchronize()
    oq, osf, og = oracle.quantize(bits(x))
    assert np.array_equal(np_(g).view(np.uint32), og.view(np.uint32))
    assert np.array_equal(np_(sf), osf)
    assert np.array_equal(np_(q), oq)


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
