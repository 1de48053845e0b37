"""Builds libmixer.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m heterogeneous_attention_mixer_amd.build`` (always recompiles).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmixer.so")
SOURCES = [os.path.join(CSRC, f)
           for f in ("attn_prefill.hip", "attn_prefill_dma.hip", "mixer_api.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("kernels.h", "device_common.h")] + [
    os.path.join(ROOT, "include", "mixer.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def build(extra_flags=None, out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP/C++ source into ``out`` (atomically replaced)."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, out)
    return out


def needs_build() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
