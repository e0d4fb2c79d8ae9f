"""The C ABI's host code under AddressSanitizer (CPU only): the library is
rebuilt with the host half of api.hip instrumented, and the host-side ABI
tests (argument and capacity checks, context life cycle, buffer sizing, the
no-allocation entry point's refusals) run against it in a subprocess with
the sanitizer runtime preloaded. Any invalid read or write in the host code
they reach fails the run."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_abi_tests_pass_under_address_sanitizer():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the clang sanitizer runtime is not available")
    sys.path.insert(0, ROOT)
    from block_discrete_diffusion_dg_amd import build
    lib = build.build_asan()
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_init" in nm or "__asan_report" in nm, "the host code is not instrumented"
    env = dict(os.environ, DG_LIB_PATH=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in res.stderr
