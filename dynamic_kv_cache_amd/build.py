"""Build step of the HIP library: one hipcc invocation for gfx950.

Produces ``dynamic_kv_cache_amd/libfastocr.so`` in-tree from the sources in
``dynamic_kv_cache_amd/csrc`` and the public header in ``include/``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libfastocr.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["kernels.hip", "probe.hip", "static_scratch.hip", "fastocr_api.cpp"]
ARCH = os.environ.get("FASTOCR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked at $HIPCC, /opt/rocm/bin/hipcc, PATH)")


def command(out_path: str = LIB_PATH, extra=()) -> list:
    return [
        hipcc(),
        "-O3",
        "-std=c++17",
        f"--offload-arch={ARCH}",
        "-fPIC",
        "-shared",
        # packed fp32 VALU forms stay off; plain fp32 code is scheduled instead
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
        "-o", out_path,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-ldl",
        *extra,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always, even if a built copy exists)."""
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    stderr = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{stderr}")
    if verbose and stderr.strip():
        print(stderr, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
