"""Builds libentq.so (HIP kernels for gfx950 + host C++) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libentq.so")

SOURCES = ["entq_decode.hip", "entq_decode_gemv.hip", "entq_decode_gemm.hip",
           "entq_decode_tiles.hip", "entq_decode_adaptive.hip", "entq_plan.cpp", "entq_encode.cpp", "entq_encode_dev.hip"]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc") or ""):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libentq")


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
            # packed fp32 forms stay off on this hardware: plain float code only
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wall"]


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES], "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libentq build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose:
        print(r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def asm(out: str, source: str = "entq_decode.hip") -> str:
    """Device assembly of one source into the file `out` (for inspection)."""
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    cmd = [hipcc(), *compile_flags(), "--cuda-device-only", "-S", "-o", out,
           os.path.join(CSRC, source)]
    subprocess.check_call(cmd)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
