"""Build libsdpa03.so in-tree with hipcc for gfx950.

    python -m scaled_dot_product_03_amd.build

compiles the HIP kernels and the C-ABI layer into
``scaled_dot_product_03_amd/libsdpa03.so``.  Every call recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libsdpa03.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "api.cpp"]

# Packed fp32 VALU instructions are kept out of the device code; hipcc's
# host pass does not know the feature and says so, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_command(out_path: str = LIB_PATH, extra=()) -> list:
    return [
        HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        *DEVICE_FLAGS,
        "-I", os.path.join(ROOT, "include"),
        "-x", "hip",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out_path, *extra,
    ]


def build_library(verbose: bool = True) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-q" not in sys.argv))
