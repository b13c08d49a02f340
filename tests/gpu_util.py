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


CANARY = 0x5A  # byte pattern of the guard tail


def guarded(shape, dtype, tail_bytes=4096):
    """An output tensor of `shape` followed, in the same allocation, by a tail of guard
    bytes; returns (tensor, check) where check() asserts that the tail is untouched (no
    kernel wrote past the end of its output)."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((n + tail_bytes,), CANARY, dtype=torch.uint8, device=DEV)
    out = buf[:n].view(dtype).view(*shape)

    def check():
        tail = host(buf[n:])
        assert np.all(tail == CANARY), f"output overrun: {np.count_nonzero(tail != CANARY)} guard bytes changed"
    return out, check


def guarded_packed(awq, N, K, group=128, w_bit=4):
    """A PackedLinear whose three tensors each carry a guard tail; returns (packed, check)."""
    G = K // group
    zcols = G if w_bit == 8 else (G + 1) // 2
    qw, c1 = guarded((N, K * w_bit // 32), torch.int32)
    sc, c2 = guarded((N, G), torch.float16)
    zb, c3 = guarded((N, zcols), torch.uint8)

    def check():
        c1(), c2(), c3()
    return awq.PackedLinear(qw, sc, zb, N, K, group, w_bit), check
