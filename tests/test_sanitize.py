"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU: every call is rejected before anything is enqueued).
The driver is tests/sanitize/abi_host_checks.cpp, built against a host-sanitized
awq_abi.hip by weight_only_bit_02_amd/sanitize_host.py. The oracle is plain Python and NumPy,
with no native code of its own to sanitize."""

import os
import shutil

import pytest

from weight_only_bit_02_amd import build_lib, sanitize_host


def test_host_validation_under_sanitizers():
    needed = [os.path.join(build_lib.BUILD, os.path.splitext(s)[0] + ".o")
              for s in build_lib.SOURCES if s != "awq_abi.hip"]
    if not all(os.path.exists(o) for o in needed) or not shutil.which(build_lib.HIPCC):
        pytest.skip("needs the objects of a normal build (build_lib.build()) and hipcc")
    r = sanitize_host.run()
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host validation ok" in r.stdout
