"""GPU tests of the boundary's error paths: the bounded waits of the FUSED
quantize (forced to give up from the host, so every kernel still runs to its
end) are reported by nvfp4_quantize_status, and the binding rejects tensors
whose shapes do not match the sizes it would pass to the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bits, np_

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")


class _WaitLimit:
    """Sets the co-resident kernels' poll limit for a block, restoring it after."""

    def __init__(self, polls):
        self.polls = polls

    def __enter__(self):
        self.prev = nv.set_wait_limit(self.polls)
        return self

    def __exit__(self, *exc):
        nv.set_wait_limit(self.prev)
        return False


@pytest.mark.parametrize("shape", [(5, 256, 1024), (1, 8192, 7168), (1, 65536, 16384)])
def test_fused_wait_timeout_is_reported(shape):
    """With a poll limit of 0 every wait of the FUSED launch gives up at once
    (the on-chip kernel for the first shape, the big-tensor one for the
    second, the streaming one for the third: 2 GiB of bf16).  A
    tensor whose amax was still being gathered when its workgroups had to
    wait gets NaN for g; one whose maxima had all arrived
    when they were polled keeps its exact g.  At least one tensor waits (the
    first: nothing is published before the launch), and
    nvfp4_quantize_status reports ETIMEOUT once.  The same workspace then
    gives the two-kernel bytes."""
    print("case: fused timeout", shape, flush=True)
    gen = torch.Generator().manual_seed(61)
    x = torch.randn(shape, generator=gen).to(torch.bfloat16).cuda()
    ws = nv.make_workspace(*shape)
    with _WaitLimit(0):
        _, _, g = nv.quantize(x, flags="fused", workspace=ws)
        torch.cuda.synchronize()
    nan = torch.isnan(g)
    assert nan[0], "the first tensor's wait gave up: its g must be NaN"
    _, _, g2 = nv.quantize(x, flags="two_kernel")
    assert torch.equal(g[~nan], g2[~nan]), "tensors that did not wait keep their exact g"
    with pytest.raises(nv.NVFP4Error) as err:
        nv.quantize_status(ws)
    assert err.value.status == nv.ETIMEOUT
    assert nv.quantize_status(ws)                     # reported once, then clear
    a = nv.quantize(x, flags="fused", workspace=ws)
    r = nv.quantize(x, flags="two_kernel")
    assert nv.quantize_status(ws)
    for u, v in zip(a, r):
        assert torch.equal(u, v)
    oq, osf, og = oracle.quantize(bits(x))
    assert np.array_equal(np_(a[2]), og) and np.array_equal(np_(a[0]), oq) and np.array_equal(np_(a[1]), osf)


def test_quantize_ex_2d_timeout_is_reported():
    """The single-launch 2D quantize of nvfp4_quantize_ex reports a wait that
    gave up through nvfp4_quantize_status on its own workspace."""
    gen = torch.Generator().manual_seed(62)
    x = torch.randn((2, 256, 512), generator=gen).to(torch.bfloat16).cuda()
    ws = torch.empty(nv.lib().nvfp4_quantize_ex_workspace_bytes(2), dtype=torch.uint8, device="cuda")
    oq, osf, og = oracle.quantize_ex(bits(x), nv.VAR_2D)
    with _WaitLimit(0):
        _, _, g = nv.quantize_ex(x, nv.VAR_2D, workspace=ws)
        torch.cuda.synchronize()
    # the first tensor's amax is a blocking wait, which gives up at once;
    # later tensors' maxima may already be complete in the polled slots
    gh = np_(g)
    assert np.isnan(gh[0])
    assert np.array_equal(gh[~np.isnan(gh)], og[~np.isnan(gh)])
    with pytest.raises(nv.NVFP4Error) as err:
        nv.quantize_status(ws)
    assert err.value.status == nv.ETIMEOUT
    q, sf, g = nv.quantize_ex(x, nv.VAR_2D, workspace=ws)
    assert nv.quantize_status(ws)
    assert np.array_equal(np_(g), og) and np.array_equal(np_(q), oq) and np.array_equal(np_(sf), osf)


def test_binding_rejects_mismatched_shapes():
    """Every shape the binding derives a size from is checked before a launch."""
    dev = "cuda"
    x = torch.zeros((2, 8, 64), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((2, 8, 32), dtype=torch.uint8, device=dev)
    sf = torch.zeros((2, 8, 4), dtype=torch.uint8, device=dev)
    g = torch.ones(2, device=dev)
    bad = [
        lambda: nv.quantize(x, out=(q[:, :7].contiguous(), sf, g)),
        lambda: nv.quantize(x, out=(q, sf[:1], g)),
        lambda: nv.quantize(x, out=(q, sf, g[:1])),
        lambda: nv.quantize_with_scale(x, g, out=(q, sf[:, :, :3].contiguous())),
        lambda: nv.dequantize(q, sf[:, :4], g),
        lambda: nv.dequantize(q, sf, g[:1]),
        lambda: nv.dequantize(q, sf, g, out=torch.zeros((2, 8, 62), dtype=torch.bfloat16, device=dev)),
    ]
    cache = nv.KVCache(2, 2, 64, 32, torch.ones(4), torch.ones(4), device=dev)
    kn = torch.zeros((2, 4, 2, 64), dtype=torch.bfloat16, device=dev)
    bad += [
        lambda: cache.append(0, kn, kn[:, :, :1].contiguous()),
        lambda: cache.append(0, kn[:1].contiguous(), kn[:1].contiguous()),
        lambda: cache.append(0, kn[..., :32].contiguous(), kn[..., :32].contiguous()),
        lambda: cache.decode_qk(torch.zeros((1, 4, 64), dtype=torch.bfloat16, device=dev), 8),
        lambda: cache.decode_qk(torch.zeros((2, 4, 32), dtype=torch.bfloat16, device=dev), 8),
        lambda: cache.decode_qk(torch.zeros((2, 4, 64), dtype=torch.bfloat16, device=dev), 8,
                                out=torch.zeros((2, 4, 7), device=dev)),
        lambda: cache.decode_attention(torch.zeros((3, 4, 64), dtype=torch.bfloat16, device=dev), 8, 0.1),
        lambda: cache.decode_attention(torch.zeros((2, 4, 64), dtype=torch.bfloat16, device=dev), 8, 0.1,
                                       out=torch.zeros((2, 4, 32), device=dev)),
        lambda: cache.read(0, 2, 0, 8, k_out=torch.zeros((2, 2, 7, 64), dtype=torch.bfloat16, device=dev)),
    ]
    aq = torch.zeros((64, 256), dtype=torch.uint8, device=dev)
    asf = torch.zeros((64, 32), dtype=torch.uint8, device=dev)
    one = torch.ones(1, device=dev)
    bad += [
        lambda: nv.gemm(aq, asf, one, aq[:, :128].contiguous(), asf, one),
        lambda: nv.gemm(aq, asf[:, :16].contiguous(), one, aq, asf, one),
        lambda: nv.gemm(aq, asf, one, aq, asf[:32], one),
        lambda: nv.gemm(aq, asf, torch.ones(2, device=dev), aq, asf, one),
        lambda: nv.gemm(aq, asf, one, aq, asf, one, out=torch.zeros((64, 32), device=dev)),
        lambda: nv.grouped_gemm(aq, asf, one, aq.view(2, 32, 256), asf[:32].contiguous(), one.repeat(2),
                                torch.tensor([0, 32, 64], dtype=torch.int32, device=dev)),
        lambda: nv.quantize_ex(x, nv.VAR_2D, out=(q[:, :4].contiguous(), sf, g)),
        lambda: nv.mxfp4_quantize(x, out=(q, sf)),
        lambda: nv.mxfp4_dequantize(q, sf[:, :, :2].contiguous(), out=torch.zeros((2, 8, 32), dtype=torch.bfloat16,
                                                                                 device=dev)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
            pytest.fail(f"call {i} was accepted")
    torch.cuda.synchronize()
