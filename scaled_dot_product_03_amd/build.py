"""Build libsdpa03.so in-tree with hipcc for gfx950.

    python -m scaled_dot_product_03_amd.build

compiles the HIP kernels and the C-ABI layer into
``scaled_dot_product_03_amd/libsdpa03.so``, one hipcc process per source
file.  Every call recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libsdpa03.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn_fwd.hip", "attn_fwd_bf16.hip", "attn_fwd_f16.hip", "attn_fwd_f32.hip", "attn_bwd.hip",
           "api.cpp"]

# Packed fp32 VALU instructions are kept out of the device code; hipcc's
# host pass does not know the feature and says so, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def object_command(source: str, out_path: str, extra=()) -> list:
    """hipcc command that compiles one source of the library to an object."""
    return [
        HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        *DEVICE_FLAGS,
        "-I", os.path.join(ROOT, "include"),
        "-x", "hip", "-c", os.path.join(CSRC, source),
        "-o", out_path, *extra,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build_library(verbose: bool = True, out_path: str = LIB_PATH, extra=()) -> str:
    """Compile every source (in parallel, one hipcc per file) and link
    ``out_path``; ``extra`` goes to every compile (e.g. -D overrides)."""
    with tempfile.TemporaryDirectory(prefix="sdpa03_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            for f in [pool.submit(_run, object_command(s, o, extra), verbose)
                      for s, o in zip(SOURCES, objs)]:
                f.result()
        tmp = out_path + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build_library(verbose="-q" not in sys.argv))
