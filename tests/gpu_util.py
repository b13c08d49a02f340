"""Helpers shared by the GPU parity tests (conversion between torch and numpy)."""

import numpy as np
import torch

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def packed_host(p):
    """(qweight uint32, scales fp16, zeros uint8) of a PackedLinear, on the host."""
    return host(p.qweight).view(np.uint32), host(p.scales), host(p.zeros)


def flags_tensor():
    return torch.zeros(1, dtype=torch.int32, device=DEV)
