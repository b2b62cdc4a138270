"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random tensors; it holds none of the NVFP4 method's
arithmetic, so both the HIP path and the CPU oracle may consume its output.
Values are drawn with torch's seeded generator on the requested device and
rounded to bf16 (round-to-nearest-even).  The oracle always receives a host
copy of the very tensor the kernels consumed, so both sides see identical
bits whichever device drew them.

Workloads (sizes from the five configurations the library is measured on):
  single    1024 x 1024, N(0,1)
  experts   E x [2048 x 7168], N(0, 0.02), each entry independently x50
            with probability 0.001 (outliers); one tensor scale per expert
  acts      tokens x 7168, 0.5 * Student-t(nu=3), 8 random channels x30
  kv        K/V chunks [32 layers][256 tokens][8 heads][128 dims], N(0,1),
            decode query [32][32 q-heads][128], N(0,1)
  gemm      A [8192 x 7168], B [2048 x 7168], N(0,1)
"""
import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std=1.0, seed=0, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def single(seed=101, device="cpu", rows=1024, cols=1024) -> torch.Tensor:
    return normal((rows, cols), 1.0, seed, device)


def experts(n_experts=64, rows=2048, cols=7168, seed=102, device="cpu") -> torch.Tensor:
    """[E][rows][cols] bf16: N(0, 0.02) with Bernoulli(0.001) entries scaled by 50."""
    g = _gen(seed, device)
    out = torch.empty((n_experts, rows, cols), dtype=torch.bfloat16, device=device)
    for e in range(n_experts):           # per expert keeps peak fp32 scratch small
        x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32).mul_(0.02)
        mask = torch.rand((rows, cols), generator=g, device=device) < 0.001
        x[mask] *= 50.0
        out[e].copy_(x.to(torch.bfloat16))
        del x, mask
    return out


def activations(tokens=16384, channels=7168, seed=103, device="cpu") -> torch.Tensor:
    """[tokens][channels] bf16: 0.5 * Student-t(3) = 0.5 * z / sqrt(chi2_3 / 3); 8 channels x30."""
    g = _gen(seed, device)
    z = torch.randn((tokens, channels), generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros_like(z)
    for _ in range(3):
        w = torch.randn((tokens, channels), generator=g, device=device, dtype=torch.float32)
        chi2.addcmul_(w, w)
        del w
    t = z.div_(chi2.div_(3.0).sqrt_()).mul_(0.5)
    del chi2
    cols = torch.randperm(channels, generator=g, device=device)[:8]
    t[:, cols] *= 30.0
    return t.to(torch.bfloat16)


def kv_chunk(chunk: int, layers=32, tokens=256, kv_heads=8, head_dim=128, seed=104, device="cpu"):
    """One appended chunk: (K, V) bf16 [layers][tokens][kv_heads][head_dim], N(0,1).

    Chunk c draws from its own stream (seed, c) so chunks can be made in any order."""
    g = _gen(seed * 1_000_003 + 7919 * (chunk + 1), device)
    k = torch.randn((layers, tokens, kv_heads, head_dim), generator=g, device=device).to(torch.bfloat16)
    v = torch.randn((layers, tokens, kv_heads, head_dim), generator=g, device=device).to(torch.bfloat16)
    return k, v


def kv_query(layers=32, q_heads=32, head_dim=128, seed=104, device="cpu") -> torch.Tensor:
    return normal((layers, q_heads, head_dim), 1.0, seed * 1_000_003 + 1, device)


def gemm_operands(M=8192, N=2048, K=7168, seed=105, device="cpu"):
    g = _gen(seed, device)
    a = torch.randn((M, K), generator=g, device=device).to(torch.bfloat16)
    b = torch.randn((N, K), generator=g, device=device).to(torch.bfloat16)
    return a, b


def to_bits(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns on the host."""
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
