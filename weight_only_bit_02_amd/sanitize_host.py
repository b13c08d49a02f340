"""Host-side sanitizer build of the C ABI's argument validation.

Compiles awq_abi.hip with AddressSanitizer and UndefinedBehaviorSanitizer on its host pass
only (the device code is built as usual), links it with the other objects of the normal
build (_build/, from build_lib.build()) and the driver tests/sanitize/abi_host_checks.cpp,
and runs the driver: every entry point is called with arguments it must reject before
enqueuing anything, so no GPU is used.

Usage: python -m weight_only_bit_02_amd.sanitize_host   (returns the driver's exit code)
"""

from __future__ import annotations

import os
import subprocess
import sys

from . import build_lib

LLVM = os.environ.get("ROCM_LLVM", "/opt/rocm/llvm/bin")
OUT = os.path.join(build_lib.BUILD, "sanitize")
DRIVER = os.path.join(build_lib.ROOT, "tests", "sanitize", "abi_host_checks.cpp")
SAN = ["address", "undefined"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build() -> str:
    """Builds the sanitized driver executable and returns its path (needs the objects of a
    normal build in _build/)."""
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in build_lib.SOURCES:
        if src == "awq_abi.hip":
            continue
        o = os.path.join(build_lib.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(o):
            raise FileNotFoundError(f"{o}: run build_lib.build() first")
        objs.append(o)
    abi = os.path.join(OUT, "awq_abi_san.o")
    host_san = []
    for s in SAN:  # host pass only: device code is never built with a sanitizer
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    _run([build_lib.HIPCC, *build_lib.FLAGS, *host_san, "-Xarch_host", "-fno-sanitize-recover=undefined",
          "-Xarch_host", "-g", "-c", os.path.join(build_lib.CSRC, "awq_abi.hip"), "-o", abi])
    drv = os.path.join(OUT, "abi_host_checks.o")
    _run([os.path.join(LLVM, "clang++"), "-std=c++17", "-g", "-O1", f"-fsanitize={','.join(SAN)}",
          "-fno-sanitize-recover=undefined", "-I", build_lib.INCLUDE, "-c", DRIVER, "-o", drv])
    exe = os.path.join(OUT, "abi_host_checks")
    _run([os.path.join(LLVM, "clang++"), f"-fsanitize={','.join(SAN)}", drv, abi, *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    return exe


def run() -> subprocess.CompletedProcess:
    exe = build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


if __name__ == "__main__":
    r = run()
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    sys.exit(r.returncode)
