"""The host ABI tests again, against a build whose HOST code (argument
validation, workspace carving, planning, the host validator) is compiled
with AddressSanitizer; device code is built as usual.  Runs on the CPU.

The instrumented library resolves the sanitizer runtime from the
interpreter, which loads it first (LD_PRELOAD); leak checking is off
because the interpreter itself keeps allocations until exit."""
import glob
import os
import subprocess
import sys

import pytest

from mla_latent_kv_33_amd import build as mla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob(
        "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_under_host_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(mla_build.HIPCC):
        pytest.skip("no hipcc or sanitizer runtime")
    lib = str(tmp_path / "libmla_host_asan.so")
    host_asan = ["-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
    mla_build.build(lib=lib, extra_flags=host_asan)
    env = dict(os.environ, LD_PRELOAD=rt, MLA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi_host.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = proc.stdout + proc.stderr
    assert proc.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
