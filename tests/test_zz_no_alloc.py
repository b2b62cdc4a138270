"""GPU test of nvfp4_quantize_noalloc through the C ABI: its outputs equal
nvfp4_quantize's (same inputs, caller workspace) bit for bit, on consecutive
calls on the library's shared scratch, each with a smaller input than the
last, in both launch modes; and a batch above the scratch limit is rejected before
any launch."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

nv = pytest.importorskip("nvfp4_block_scaled_06_amd")


def _input(shape, seed):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=gen) * torch.linspace(0.01, 50.0, shape[0]).view(-1, 1, 1)
    return x.to(torch.bfloat16).cuda()


@pytest.mark.parametrize("flags", ["fused", "two_kernel"])
def test_noalloc_matches_quantize_on_consecutive_calls(flags):
    print("case: noalloc", flags, flush=True)
    # the streaming FUSED kernel (a tensor too large to hold on chip), then the
    # on-chip one, then a smaller input again on the same scratch
    for shape, seed in (((1, 8192, 2048), 70), ((9, 512, 2048), 71), ((3, 64, 256), 72)):
        x = _input(shape, seed)
        got = nv.quantize_noalloc(x, flags=flags)
        want = nv.quantize(x, flags=flags)
        torch.cuda.synchronize()
        for u, v, what in zip(got, want, ("codes", "scale bytes", "tensor scales")):
            assert torch.equal(u, v), f"{flags} {shape}: {what} differ"


def test_noalloc_rejects_batch_above_scratch():
    L = nv.lib()
    x = torch.zeros((102, 1, 16), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((102, 1, 8), dtype=torch.uint8, device="cuda")
    sf = torch.zeros((102, 1, 1), dtype=torch.uint8, device="cuda")
    g = torch.zeros(102, device="cuda")
    st = L.nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), 102, 1, 16, ctypes.c_void_p(q.data_ptr()),
                                  ctypes.c_void_p(sf.data_ptr()), ctypes.c_void_p(g.data_ptr()), 1, None)
    assert st == -3                                    # NVFP4_EWORKSPACE
    assert L.nvfp4_quantize_workspace_bytes(101, 1, 16) <= 1 << 20 < L.nvfp4_quantize_workspace_bytes(102, 1, 16)
