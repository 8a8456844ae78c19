"""The host-side ABI tests again, against a build whose host code (mj_host.cpp,
mj_noalloc.hip's host pass) carries AddressSanitizer and
UndefinedBehaviorSanitizer: plan arithmetic, argument validation and
workspace sizing without out-of-bounds accesses, overflows or other
undefined behaviour.  CPU only; needs hipcc and the device objects of the
normal build (``__graft_entry__.build()``)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _san_env(lib, runtime):
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, PAGED_FP8_DECODE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


@pytest.fixture(scope="module")
def sanitized():
    from paged_fp8_decode_amd import build as B
    if not os.path.exists(B.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc is not installed")
    if not all(os.path.exists(os.path.join(B.BUILD, s + ".o")) for s in B.HIP_SOURCES):
        pytest.skip("no device objects: run __graft_entry__.build() first")
    return B.build_host_sanitized(), B.asan_runtime()


def test_sanitized_library_is_the_one_loaded(sanitized):
    lib, runtime = sanitized
    code = ("import paged_fp8_decode_amd as m; m.lib(); "
            "maps = open('/proc/self/maps').read(); "
            f"assert {os.path.basename(lib)!r} in maps and 'libmj.so' not in maps, 'wrong library'; "
            "assert 'libclang_rt.asan' in maps, 'no sanitizer runtime'; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_san_env(lib, runtime), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_abi_host_suite_under_asan_ubsan(sanitized):
    lib, runtime = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_host.py", "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=_san_env(lib, runtime), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
