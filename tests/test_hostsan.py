"""The library's host code (argument checks, workspace and size arithmetic, launch set-up) under
AddressSanitizer and UndefinedBehaviorSanitizer: every CPU-side ABI test of test_abi.py runs
against a host-sanitized copy of the library (newton_schulz_matrix_muon_amd.build.build_hostsan:
the host pass rebuilt with the sanitizers around the built library's own GPU binary) in a child
process that preloads the ASan runtime. Any sanitizer report fails the test. The copy is for
the CPU only: the test skips on a machine with a GPU device node."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

CHILD = r"""
import ctypes, inspect, sys
sys.path[:0] = [{root!r}, {tests!r}]
from newton_schulz_matrix_muon_amd import ops
lib = ops.declare(ctypes.CDLL({path!r}))
ops._LIB = lib          # the binding's helpers use this copy (and never import torch)
import test_abi
ran = []
for name, fn in sorted(vars(test_abi).items()):
    if name.startswith("test_") and list(inspect.signature(fn).parameters) == ["L"]:
        fn(lib)
        ran.append(name)
print("ran", len(ran), " ".join(ran), flush=True)
"""


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_tests_under_host_sanitizers():
    from newton_schulz_matrix_muon_amd import build as b
    if os.path.exists("/dev/kfd"):
        pytest.skip("the host-sanitized copy runs on the CPU only")
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime under /opt/rocm/llvm")
    if not os.path.exists(b.LIB):
        pytest.skip("the library is not built")
    if not os.path.exists(b.HOSTSAN_LIB) or os.path.getmtime(b.HOSTSAN_LIB) < os.path.getmtime(b.LIB):
        b.build_hostsan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, tests=TESTS, path=b.HOSTSAN_LIB)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    ran = [l for l in r.stdout.splitlines() if l.startswith("ran ")]
    assert ran and int(ran[0].split()[1]) >= 10, out[-2000:]
