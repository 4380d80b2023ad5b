"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of libseer whose capi.cpp (validation, workspace sizing, launch
geometry) is compiled with -fsanitize=address,undefined on the host side,
linked with the regular kernel objects, and runs the host-side C-ABI tests
(tests/test_capi_cpu.py) against it in a child process that preloads the
sanitizer runtime.  Any sanitizer report fails the run (halt_on_error).
No GPU is used: every call in those tests fails validation before a launch.
"""

import os
import subprocess
import sys

import pytest

from block_sparse_attention_29_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_capi_host_layer_is_sanitizer_clean():
    try:
        lib = B.build_host_sanitized()
        rt = B.sanitizer_runtime()
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"no sanitizer toolchain: {e}")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # the child confirms that the sanitizer runtime and the sanitized library are the ones loaded
    probe = ("import ctypes, sys; sys.path.insert(0, %r); "
             "from block_sparse_attention_29_amd import seer; l = seer.load(%r); "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); "
             "maps = open('/proc/self/maps').read(); assert %r in maps; print('probe ok')"
             % (ROOT, lib, os.path.basename(lib)))
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "probe ok" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_capi_cpu.py"), "--seer-lib", lib],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
