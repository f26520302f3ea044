"""The C ABI's host-side validation under AddressSanitizer.

The library is rebuilt with the host half of every source instrumented (the sanitizer flag is
given to the host pass only; device code is built as usual), loaded into a fresh interpreter with
the sanitizer runtime preloaded, and the ctypes checks of tests/test_abi_host.py run against it:
every validation path (null pointers, shapes, pitches, alignments, descriptor arrays, status
strings, workspace queries) must complete without a sanitizer report. No kernel is launched.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    for clang in ("/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if clang and os.path.exists(clang):
            r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


@pytest.mark.skipif(_asan_runtime() is None or shutil.which("hipcc") is None
                    and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc or the AddressSanitizer runtime is not available")
def test_host_validation_under_address_sanitizer(tmp_path):
    sys.path.insert(0, ROOT)
    from fp8_blockwise_quantization_amd import build as b

    lib = str(tmp_path / "libfp8rl_asan.so")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    b.build(extra_flags=host_asan, out_path=lib)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms  # the host code is instrumented
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), FP8RL_TEST_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"), "-k",
                        "not python_binding"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
