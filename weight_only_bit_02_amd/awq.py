"""Thin PyTorch binding of the AWQ W4A16 C ABI (argument marshalling only).

torch provides device memory and the current stream; every step of the path runs in
the library's HIP kernels. Each function checks that its tensors live on the GPU,
have the expected dtype and are contiguous (a host pointer handed to a kernel would
fault the device), allocates outputs, and raises AwqError on a non-OK status.
"""

from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _abi

GROUP = 128          # default group size; 64 and 32 are also supported


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class PackedLinear:
    """Packed 4-bit weight of one [N][K] linear: codes, fp16 group scales, zero nibbles."""
    qweight: torch.Tensor  # int32 [N][K w_bit / 32] (3, 4 or 8-bit codes): the bits of uint32 words
    scales: torch.Tensor   # fp16 [N][G], G = K / group
    zeros: torch.Tensor    # uint8 [N][ceil(G/2)] (3/4-bit: two per byte) or [N][G] (8-bit)
    N: int
    K: int
    group: int = GROUP
    w_bit: int = 4

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.qweight, self.scales, self.zeros))


def alloc_packed(N: int, K: int, device, group: int = GROUP, w_bit: int = 4) -> PackedLinear:
    G = K // group
    zcols = G if w_bit == 8 else (G + 1) // 2
    return PackedLinear(
        torch.empty((N, K * w_bit // 32), dtype=torch.int32, device=device),
        torch.empty((N, G), dtype=torch.float16, device=device),
        torch.empty((N, zcols), dtype=torch.uint8, device=device), N, K, group, w_bit)


def quantize_pack(W: torch.Tensor, s: torch.Tensor | None = None, flags: torch.Tensor | None = None,
                  out: PackedLinear | None = None, clip_idx: torch.Tensor | None = None,
                  clip_steps: int = 200, zero_point: bool = True,
                  group_size: int = GROUP, w_bit: int = 4) -> PackedLinear:
    """awq_quantize_pack: 4-bit group-wise quantization of W * diag(s) (s = None: plain
    RTN; groups of group_size = 128 or 64 channels); with clip_idx (uint8 [N][K/group],
    clip_search's output), awq_quantize_pack_clipped; zero_point=False: symmetric codes
    (same packed format, every zero 8); w_bit=8 or 3: 8- or 3-bit codes."""
    lib = _abi.load()
    _need(W, torch.float16, "W")
    if W.dim() != 2:
        raise ValueError("W must be [N][K]")
    N, K = W.shape
    if s is not None:
        _need(s, torch.float16, "s")
        if s.shape != (K,):
            raise ValueError("s must be [K]")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    p = out if out is not None else alloc_packed(N, K, W.device, group_size, w_bit)
    for name, t, dt in (("qweight", p.qweight, torch.int32), ("scales", p.scales, torch.float16),
                        ("zeros", p.zeros, torch.uint8)):
        _need(t, dt, name)
    if p.N != N or p.K != K or p.group != group_size or p.w_bit != w_bit:
        raise ValueError("output packed buffers have the wrong shape, group size or width")
    cfg = _abi.config(zero_point=int(zero_point), group_size=group_size, w_bit=w_bit)
    if clip_idx is not None:
        _need(clip_idx, torch.uint8, "clip_idx")
        if clip_idx.shape != (N, K // group_size):
            raise ValueError("clip_idx must be [N][K/group]")
    _abi.check("awq_quantize_pack_clipped", lib.awq_quantize_pack_clipped(
        _ptr(W), N, K, _ptr(s), _ptr(clip_idx), clip_steps, C.byref(cfg), _ptr(p.qweight),
        _ptr(p.scales), _ptr(p.zeros), _ptr(flags), _stream()))
    return p


def clip_search(X: torch.Tensor, W: torch.Tensor, s: torch.Tensor | None = None,
                clip_steps: int = 200, n_shrink: int = 100, flags: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, zero_point: bool = True,
                group_size: int = GROUP, w_bit: int = 4):
    """awq_clip_search: per group, the index of the best shrink ratio (uint8 [N][K/group])
    and its error (fp64 [N][K/group]); ratio r_i = (clip_steps - i) / clip_steps, i < n_shrink."""
    lib = _abi.load()
    _need(X, torch.float16, "X")
    _need(W, torch.float16, "W")
    T, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("X and W disagree on K")
    if s is not None:
        _need(s, torch.float16, "s")
        if s.shape != (K,):
            raise ValueError(f"s must have shape ({K},)")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    cfg = _abi.config(zero_point=int(zero_point), group_size=group_size, w_bit=w_bit)
    nbytes = int(lib.awq_clip_search_workspace_size(T, N, K, n_shrink, C.byref(cfg)))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=X.device)
    _need(workspace, torch.uint8, "workspace")
    G = K // group_size
    idx = torch.empty((N, G), dtype=torch.uint8, device=X.device)
    err = torch.empty((N, G), dtype=torch.float64, device=X.device)
    _abi.check("awq_clip_search", lib.awq_clip_search(
        _ptr(X), T, _ptr(W), N, K, _ptr(s), clip_steps, n_shrink, C.byref(cfg), _ptr(idx),
        _ptr(err), _ptr(workspace), workspace.numel(), _ptr(flags), _stream()))
    return idx, err


def activation_stats(X: torch.Tensor, flags: torch.Tensor | None = None) -> torch.Tensor:
    """awq_activation_stats: fp64 [K] mean |x| per input channel."""
    lib = _abi.load()
    _need(X, torch.float16, "X")
    T, K = X.shape
    act = torch.empty(K, dtype=torch.float64, device=X.device)
    ws_bytes = lib.awq_activation_stats_workspace_size(T, K)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=X.device)
    if flags is not None:
        _need(flags, torch.int32, "flags")
    _abi.check("awq_activation_stats", lib.awq_activation_stats(
        _ptr(X), T, K, _ptr(act), _ptr(ws), ws_bytes, _ptr(flags), _stream()))
    return act


def candidate_scales(act: torch.Tensor, n_grid: int = 20) -> torch.Tensor:
    """awq_candidate_scales: fp16 [n_grid][K], row i = fp16(max(act, 2^-14)^(i/n_grid))."""
    lib = _abi.load()
    _need(act, torch.float64, "act")
    K = act.shape[0]
    out = torch.empty((n_grid, K), dtype=torch.float16, device=act.device)
    cfg = _abi.config(n_grid)
    _abi.check("awq_candidate_scales", lib.awq_candidate_scales(
        _ptr(act), K, C.byref(cfg), _ptr(out), _stream()))
    return out


@dataclass
class SearchResult:
    s_best: torch.Tensor    # fp16 [K]
    best_idx: torch.Tensor  # int32 [1] (device)
    err: torch.Tensor       # fp64 [n_grid]
    s_grid: torch.Tensor    # fp16 [n_grid][K]


class SearchWorkspace:
    """Reusable device scratch for awq_search_scales (sized by the library's query)."""

    def __init__(self, T: int, N: int, K: int, device, n_grid: int = 20):
        lib = _abi.load()
        cfg = _abi.config(n_grid)
        self.nbytes = lib.awq_search_workspace_size(T, N, K, C.byref(cfg))
        if self.nbytes == 0:
            raise ValueError("unsupported search shape")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)


def search_scales(X: torch.Tensor, W: torch.Tensor, n_grid: int = 20,
                  workspace: SearchWorkspace | None = None, flags: torch.Tensor | None = None,
                  out: SearchResult | None = None, zero_point: bool = True,
                  group_size: int = GROUP, w_bit: int = 4) -> SearchResult:
    """awq_search_scales: grid search of s = mean|x|^alpha minimizing the output error."""
    lib = _abi.load()
    _need(X, torch.float16, "X")
    _need(W, torch.float16, "W")
    T, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("X and W disagree on K")
    dev = W.device
    if out is None:
        out = SearchResult(torch.empty(K, dtype=torch.float16, device=dev),
                           torch.empty(1, dtype=torch.int32, device=dev),
                           torch.empty(n_grid, dtype=torch.float64, device=dev),
                           torch.empty((n_grid, K), dtype=torch.float16, device=dev))
    _need(out.s_best, torch.float16, "out.s_best")
    _need(out.best_idx, torch.int32, "out.best_idx")
    _need(out.err, torch.float64, "out.err")
    _need(out.s_grid, torch.float16, "out.s_grid")
    if (out.s_best.shape != (K,) or out.best_idx.numel() < 1 or out.err.shape != (n_grid,)
            or out.s_grid.shape != (n_grid, K)):
        raise ValueError("out buffers have the wrong shapes for this search")
    ws = workspace if workspace is not None else SearchWorkspace(T, N, K, dev, n_grid)
    if ws.buf.numel() < int(lib.awq_search_workspace_size(
            T, N, K, C.byref(_abi.config(n_grid, zero_point=int(zero_point), group_size=group_size,
                                         w_bit=w_bit)))):
        raise ValueError("search workspace is too small for this shape")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    cfg = _abi.config(n_grid, zero_point=int(zero_point), group_size=group_size, w_bit=w_bit)
    _abi.check("awq_search_scales", lib.awq_search_scales(
        _ptr(X), T, _ptr(W), N, K, C.byref(cfg), _ptr(out.s_best), _ptr(out.best_idx),
        _ptr(out.err), _ptr(out.s_grid), _ptr(ws.buf), ws.nbytes, _ptr(flags), _stream()))
    return out


_KERNELS = {"auto": _abi.KERNEL_AUTO, "gemv": _abi.KERNEL_GEMV, "gemm": _abi.KERNEL_GEMM,
            "skinny": _abi.KERNEL_SKINNY, "gemm_wide": _abi.KERNEL_GEMM_WIDE}


def linear_w4a16(X: torch.Tensor, w: PackedLinear, kernel: str = "auto",
                 out: torch.Tensor | None = None, flags: torch.Tensor | None = None) -> torch.Tensor:
    """awq_linear_w4a16: Y[M][N] = X[M][K] deq(W)^T in fp16 with fp32 accumulation.
    flags (int32 [1] on the GPU, optional): NONFINITE_INPUT is OR-ed in when X or the group
    scales hold an Inf or a NaN."""
    lib = _abi.load()
    _need(X, torch.float16, "X")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    M, K = X.shape
    if K != w.K:
        raise ValueError("X and the packed weight disagree on K")
    Y = out if out is not None else torch.empty((M, w.N), dtype=torch.float16, device=X.device)
    _need(Y, torch.float16, "Y")
    if Y.shape != (M, w.N):
        raise ValueError("Y has the wrong shape")
    cfg = _abi.config(group_size=w.group, w_bit=w.w_bit)
    _abi.check("awq_linear_w4a16_ex", lib.awq_linear_w4a16_ex(
        _ptr(X), M, _ptr(w.qweight), _ptr(w.scales), _ptr(w.zeros), w.N, K, C.byref(cfg),
        _ptr(Y), _ptr(flags), _KERNELS[kernel], _stream()))
    return Y


def linear_w4a16_gated_silu(X: torch.Tensor, w: PackedLinear, kernel: str = "auto",
                            out: torch.Tensor | None = None,
                            flags: torch.Tensor | None = None) -> torch.Tensor:
    """awq_linear_w4a16_gated_silu: Y[M][N/2] = SiLU(X deq(W_gate)^T) * (X deq(W_up)^T),
    where w packs the gate rows [0, N/2) and the up rows [N/2, N) (fused MLP module).
    flags as for linear_w4a16."""
    lib = _abi.load()
    _need(X, torch.float16, "X")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    M, K = X.shape
    if K != w.K:
        raise ValueError("X and the packed weight disagree on K")
    if w.N % 2:
        raise ValueError("a gate|up weight has an even number of rows")
    Y = out if out is not None else torch.empty((M, w.N // 2), dtype=torch.float16, device=X.device)
    _need(Y, torch.float16, "Y")
    if Y.shape != (M, w.N // 2):
        raise ValueError("Y has the wrong shape")
    cfg = _abi.config(group_size=w.group, w_bit=w.w_bit)
    _abi.check("awq_linear_w4a16_gated_silu_ex", lib.awq_linear_w4a16_gated_silu_ex(
        _ptr(X), M, _ptr(w.qweight), _ptr(w.scales), _ptr(w.zeros), w.N, K, C.byref(cfg),
        _ptr(Y), _ptr(flags), _KERNELS[kernel], _stream()))
    return Y


def apply_inverse_scale(A: torch.Tensor, s: torch.Tensor, axis: int, out: torch.Tensor | None = None,
                        flags: torch.Tensor | None = None) -> torch.Tensor:
    """awq_apply_inverse_scale: fp16(A / s) along columns (axis 1, activations or a norm
    weight) or rows (axis 0, the previous linear's weight); out may be A (in place)."""
    lib = _abi.load()
    _need(A, torch.float16, "A")
    _need(s, torch.float16, "s")
    if flags is not None:
        _need(flags, torch.int32, "flags")
    A2 = A.reshape(1, -1) if A.dim() == 1 else A
    if A2.dim() != 2:
        raise ValueError("A must be 1-D or 2-D")
    rows, cols = A2.shape
    if s.numel() != (cols if axis == 1 else rows):
        raise ValueError("s has the wrong length for this axis")
    Y = out if out is not None else torch.empty_like(A)
    _need(Y, torch.float16, "out")
    if Y.shape != A.shape:
        raise ValueError("out has the wrong shape")
    _abi.check("awq_apply_inverse_scale", lib.awq_apply_inverse_scale(
        _ptr(A), rows, cols, _ptr(s), axis, _ptr(Y), _ptr(flags) if flags is not None else None,
        _stream()))
    return Y


def gemv_max_m() -> int:
    return int(_abi.load().awq_gemv_max_m())
