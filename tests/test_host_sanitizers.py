"""AddressSanitizer and UndefinedBehaviorSanitizer on the library's host code
(CPU only: no kernel is launched).

Argument validation, size queries, workspace checks and error reporting of
the C ABI are host code in api.hip.  That file is rebuilt with both
sanitizers on its host pass only (the device code is compiled as usual),
linked with the other objects of the ordinary build, loaded under the ASan
runtime in a child process, and driven through every host-side check of
tests/test_abi.py.  A sanitizer report aborts the child, which fails this
test.
"""
import glob
import os
import subprocess
import sys

import pytest

from nvfp4_block_scaled_03_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# Host pass only: each -fsanitize option follows -Xarch_host.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _object(src: str, out_dir: str, extra=()) -> str:
    """The ordinary build's object for ``src`` when it is current, else a fresh one."""
    obj = os.path.join(B.BUILD, src.replace(".hip", ".o"))
    path = os.path.join(B.CSRC, src)
    if not extra and os.path.exists(obj) and os.path.getmtime(obj) >= os.path.getmtime(path):
        return obj
    obj = os.path.join(out_dir, src.replace(".hip", ".o"))
    B._run([B.HIPCC, *B.FLAGS, *extra, "-c", path, "-o", obj], False)
    return obj


def test_host_code_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(B.HIPCC):
        pytest.skip("no hipcc or no ASan runtime")
    objs = [_object(src, str(tmp_path), SAN if src == "api.hip" else ()) for src in B.SOURCES]
    lib = str(tmp_path / "libnvfp4moe_san.so")
    B._run([B.HIPCC, "--offload-arch=" + B.ARCH, "-shared", "-fPIC", *SAN[:4], "-o", lib, *objs], False)
    env = dict(os.environ, LD_PRELOAD=rt, NVFP4_MOE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "passed" in r.stdout and "skipped" not in r.stdout.splitlines()[-1], report
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, report
