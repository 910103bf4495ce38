"""Build libsegkv.so for gfx950 with hipcc, in-tree.

The library is the C ABI declared in include/segkv.h: host code
(csrc/segkv_host.cpp) and HIP kernels (csrc/*.hip, one file per kernel
family, sharing csrc/kernels_common.h).  Packed fp32 instructions are
disabled for the device code (-packed-fp32-ops).
"""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libsegkv.so")
KERNEL_SOURCES = ["scatter.hip", "prefill.hip", "prefill_variants.hip", "score.hip", "decode.hip", "merge.hip"]
SOURCES = [os.path.join(CSRC, "segkv_host.cpp")] + [os.path.join(CSRC, f) for f in KERNEL_SOURCES]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libsegkv")


def build_command(out: str = LIB_PATH) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wl,--no-undefined",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC] + SOURCES + ["-o", out]


def build(verbose: bool = False) -> str:
    """Compile libsegkv.so (always recompiles).  Returns its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag and says so
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("building libsegkv failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
