"""Builds libawq_mi355x.so (hand-written HIP for gfx950) in-tree with hipcc.

Usage: python -m weight_only_bit_02_amd.build_lib   (or build() from Python)
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libawq_mi355x.so")

SOURCES = [  # the slowest units (GEMM instantiations, the searches) first: they bound the build
    "gemm_i3_plain.hip", "gemm_i3_gated.hip", "gemm_i3_plain_g32.hip", "gemm_i3_gated_g32.hip",
    "gemm_i8_plain.hip", "gemm_i8_gated.hip", "gemm_i4_plain.hip", "gemm_i4_gated.hip",
    "gemm_i4_plain_g32.hip", "gemm_i4_gated_g32.hip", "search.hip", "gemm_wide.hip", "gemv.hip", "gemv_mfma.hip",
    "gemv8.hip", "gemv3.hip", "quant_pack.hip", "stats.hip", "fold.hip", "check.hip", "peaks.hip", "gemm.hip", "awq_abi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions anywhere (plain fp32 only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32: correctly rounded division, denormals kept, no fast-math
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    "-I", INCLUDE, "-I", CSRC,
]


# Units whose results must be bit-exact against the oracle's step-by-step fp32 / fp64
# arithmetic (the group quantizer, the statistic, the candidate scales, the fold): no
# contraction of a multiply and an add into an FMA anywhere in them, not only inside the
# functions that say so with a pragma.
EXACT_UNITS = {"quant_pack.hip", "stats.hip", "search.hip", "fold.hip", "check.hip"}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = ["-ffp-contract=off"] if src in EXACT_UNITS else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature and says so; keep the rest
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if any(l.strip() for l in lines):
            print("\n".join(lines), file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compiles every HIP source for gfx950 and links the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
