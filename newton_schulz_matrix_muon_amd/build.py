"""Build libmuon_ns.so in-tree with hipcc for gfx950 (no JIT cache, no torch extension).

Usage: python -m newton_schulz_matrix_muon_amd.build [-v] [--hostsan]
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmuon_ns.so")
SOURCES = ["muon_ns.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


BUILD = os.path.join(ROOT, "_build")
HOSTSAN_LIB = os.path.join(BUILD, "libmuon_ns_hostsan.so")


def llvm_tool(name: str) -> str:
    cand = os.path.join("/opt/rocm/llvm/bin", name)
    return cand if os.path.exists(cand) else name


def build_hostsan(verbose: bool = False) -> str:
    """A copy of the library whose host code (argument checks, workspace arithmetic, launch
    set-up) is built with AddressSanitizer and UndefinedBehaviorSanitizer, for CPU-side tests.
    Its device code is the built library's own GPU binary (its .hip_fatbin section), so only
    the host pass is compiled here; no device code is instrumented. Load it only in a process
    that preloads the ASan runtime, and never on a GPU."""
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is missing: run build() first")
    os.makedirs(BUILD, exist_ok=True)
    fatbin = os.path.join(BUILD, "muon_ns_gfx950.hipfb")
    r = subprocess.run([llvm_tool("llvm-objcopy"), "-O", "binary", "--only-section=.hip_fatbin", LIB, fatbin],
                       capture_output=True, text=True)
    if r.returncode != 0 or not os.path.getsize(fatbin):
        raise RuntimeError("could not extract the GPU binary:\n" + r.stderr)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"]
    tmp = HOSTSAN_LIB + ".tmp"
    cmd = [hipcc(), *flags, "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc (host sanitizers) failed:\n" +
                           "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l))
    os.replace(tmp, HOSTSAN_LIB)
    return HOSTSAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--hostsan" in sys.argv:
        print(build_hostsan(verbose="-v" in sys.argv))
