"""Helpers shared by the GPU parity tests (host-side marshalling only)."""
import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_from_floats(values, device="cuda") -> torch.Tensor:
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).to(device)


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_frobenius(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / den) if den > 0 else float(np.linalg.norm(got))


class Guarded:
    """An output buffer with sentinel bytes on both sides; check() verifies the
    kernels wrote nothing outside the view."""
    PAD = 256

    def __init__(self, shape, dtype, device="cuda", fill=0x5A):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((n + 2 * self.PAD,), fill, dtype=torch.uint8, device=device)
        self.fill = fill
        self.n = n
        self.view = self.raw[self.PAD:self.PAD + n].view(dtype).view(shape)

    def check(self):
        r = self.raw.cpu().numpy()
        assert np.all(r[:self.PAD] == self.fill), "write before the output buffer"
        assert np.all(r[self.PAD + self.n:] == self.fill), "write past the output buffer"
