"""Build libclear_attn.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libclear_attn.so")

SOURCES = ["clear_attn.cpp", "tilemap_host.cpp", "tilemap_device.hip", "attn_fwd.hip", "attn_bwd.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Code-generation flags of the device code (part of what the kernels are).
DEVICE_FLAGS = [
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # branches on wavefront-uniform values stay plain scalar branches: the CFG
    # structurizer would otherwise join them through flow blocks whose
    # conditions it carries as 64-bit lane masks (scalar work on every chunk)
    "-Xarch_device", "-mllvm=-structurizecfg-skip-uniform-regions=true",
]


# sources the forward attention kernel is compiled and launched from (launch
# configuration included); with the device code-generation flags they key the
# committed profile figures, which hold only while both are unchanged
FWD_KERNEL_SOURCES = ("dit_circular_local_amd/csrc/attn_fwd.hip", "dit_circular_local_amd/csrc/attn_common.h",
                      "dit_circular_local_amd/csrc/clear_internal.h", "dit_circular_local_amd/csrc/tile_geom.h",
                      "include/clear_attn.h", "dit_circular_local_amd/csrc/clear_attn.cpp")


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed: edits to
    comments leave the hash (and the compiled kernel) unchanged."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """16 hex digits of SHA-256 over the forward kernel's sources (code only)
    and the device flags."""
    import hashlib

    h = hashlib.sha256()
    for name in FWD_KERNEL_SOURCES:
        with open(os.path.join(ROOT, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    h.update(" ".join(DEVICE_FLAGS).encode())
    return h.hexdigest()[:16]


def build_command(out: str = LIB):
    return [
        HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # warnings are errors (unused parameters aside: engines share signatures)
        "-Wall", "-Wextra", "-Wno-unused-parameter", "-Wno-unused-function", "-Werror",
        *DEVICE_FLAGS,
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libclear_attn.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    if verbose and r.stderr:
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
