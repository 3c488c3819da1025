"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code: the
CPU oracle (oracle.c) and the library's host side (argument checks,
workspace sizing, plans, the C ABI; its device code is unchanged and never
runs here).  The oracle's pins and the ABI checks then run against those
builds in a child process with the sanitizer runtime preloaded; any report
fails the child (halt_on_error)."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-shared-libasan", "-g"]

CHILD = r"""
import sys
root, lib, olib = sys.argv[1:4]
sys.path[:0] = [root, root + "/tests"]
import oracle
oracle._LIBPATH = olib
import tree_verification_best_amd as tv
tv.LIBPATH = lib
import pytest
files = ["tests/test_abi_cpu.py", "tests/test_oracle_build.py", "tests/test_oracle_accept.py",
         "tests/test_oracle_numerics.py", "tests/test_oracle_check.py",
         "tests/test_oracle_expand.py", "tests/test_oracle_budget.py"]
sys.exit(pytest.main(["-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] +
                     [root + "/" + f for f in files]))
"""


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_host_code_under_asan_ubsan():
    rt = _runtime()
    if rt is None or not os.path.exists(CLANG):
        pytest.skip("clang's shared sanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    import oracle.build as ob
    import tree_verification_best_amd.build as lb
    with tempfile.TemporaryDirectory() as tmp:
        olib = ob.build(lib=os.path.join(tmp, "liboracle_san.so"), cc=CLANG, flags=SAN)
        lib = lb.build(lib=os.path.join(tmp, "libtreeverify_san.so"),
                       objdir=os.path.join(tmp, "obj"), host_flags=SAN)
        env = dict(os.environ, LD_PRELOAD=rt,
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
                   LD_LIBRARY_PATH="/opt/rocm/llvm/lib:" + os.environ.get("LD_LIBRARY_PATH", ""))
        r = subprocess.run([sys.executable, "-c", CHILD, ROOT, lib, olib], env=env,
                           capture_output=True, text=True, timeout=900)
        tail = (r.stdout + r.stderr)[-4000:]
        assert r.returncode == 0, tail
        assert "ERROR: AddressSanitizer" not in r.stderr, tail
        assert "runtime error:" not in r.stderr, tail
