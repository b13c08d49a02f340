"""ctypes view of libawq_mi355x.so (the C ABI declared in include/awq.h).

Loading fails loudly when the library has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libawq_mi355x.so")

AWQ_OK = 0
STATUS_NAMES = {0: "AWQ_OK", 1: "AWQ_ERR_NULL_POINTER", 2: "AWQ_ERR_BAD_SHAPE",
                3: "AWQ_ERR_UNSUPPORTED", 4: "AWQ_ERR_MISALIGNED", 5: "AWQ_ERR_WORKSPACE",
                6: "AWQ_ERR_HIP", 7: "AWQ_ERR_SCRATCH_LIMIT"}

FLAG_NONFINITE_INPUT = 1
FLAG_SCALE_CLAMPED = 2
FLAG_OVERFLOW = 8

NOALLOC_SCRATCH_BYTES = 32 << 20  # AWQ_NOALLOC_SCRATCH_BYTES

KERNEL_AUTO, KERNEL_GEMV, KERNEL_GEMM, KERNEL_SKINNY, KERNEL_GEMM_WIDE = 0, 1, 2, 3, 4


class AwqConfig(C.Structure):
    _fields_ = [("w_bit", C.c_int32), ("group_size", C.c_int32), ("zero_point", C.c_int32),
                ("n_grid", C.c_int32)]


P = C.c_void_p
I64 = C.c_int64
CFG = C.POINTER(AwqConfig)

# name -> (restype, argtypes); every name here is exported by the library
SIGNATURES = {
    "awq_quantize_pack": (C.c_int, [P, I64, I64, P, CFG, P, P, P, P, P]),
    "awq_quantize_pack_clipped": (C.c_int, [P, I64, I64, P, P, C.c_int32, CFG, P, P, P, P, P]),
    "awq_clip_search_workspace_size": (C.c_size_t, [I64, I64, I64, C.c_int32, CFG]),
    "awq_clip_search": (C.c_int, [P, I64, P, I64, I64, P, C.c_int32, C.c_int32, CFG, P, P, P,
                                  C.c_size_t, P, P]),
    "awq_activation_stats_workspace_size": (C.c_size_t, [I64, I64]),
    "awq_activation_stats": (C.c_int, [P, I64, I64, P, P, C.c_size_t, P, P]),
    "awq_candidate_scales": (C.c_int, [P, I64, CFG, P, P]),
    "awq_search_workspace_size": (C.c_size_t, [I64, I64, I64, CFG]),
    "awq_search_scales": (C.c_int, [P, I64, P, I64, I64, CFG, P, P, P, P, P, C.c_size_t, P, P]),
    "awq_search_scales_noalloc": (C.c_int, [P, I64, P, I64, I64, CFG, P, P, P, P, P, P]),
    "awq_linear_w4a16": (C.c_int, [P, I64, P, P, P, I64, I64, CFG, P, P, P]),
    "awq_linear_w4a16_ex": (C.c_int, [P, I64, P, P, P, I64, I64, CFG, P, P, C.c_int, P]),
    "awq_linear_w4a16_gated_silu": (C.c_int, [P, I64, P, P, P, I64, I64, CFG, P, P, P]),
    "awq_linear_w4a16_gated_silu_ex": (C.c_int, [P, I64, P, P, P, I64, I64, CFG, P, P, C.c_int, P]),
    "awq_apply_inverse_scale": (C.c_int, [P, I64, I64, P, C.c_int32, P, P, P]),
    "awq_gemv_max_m": (C.c_int32, []),
    # calibration probes (include/awq_peaks.h)
    "awq_peak_read_stream": (C.c_int, [P, C.c_size_t, P, C.c_int32, P]),
    "awq_peak_mfma": (C.c_int, [I64, P, C.c_int32, P]),
    "awq_status_string": (C.c_char_p, [C.c_int]),
}

_LIB = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Loads the HIP library (once). Raises if it is missing: the product has no other path."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(
            f"libawq_mi355x.so not found at {path}; build it first "
            "(python -m weight_only_bit_02_amd.build_lib)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def config(n_grid: int = 20, w_bit: int = 4, group_size: int = 128, zero_point: int = 1) -> AwqConfig:
    return AwqConfig(w_bit, group_size, zero_point, n_grid)


class AwqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        msg = lib.awq_status_string(status).decode()
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != AWQ_OK:
        raise AwqError(fn, status)
