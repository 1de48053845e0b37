"""Builds libmixer.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m heterogeneous_attention_mixer_amd.build`` (always recompiles).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmixer.so")
SOURCES = [os.path.join(CSRC, f)
           for f in ("attn_prefill.hip", "attn_prefill_dma.hip", "mfma_ceiling.hip",
                     "mixer_api.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("kernels.h", "device_common.h")] + [
    os.path.join(ROOT, "include", "mixer.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# Per-source flags. The bf16 kernel is compiled without NaN semantics (no NaN reaches a
# value it uses), which lets fmaxf chains become plain v_max3_f32; the host API, whose
# argument checks test for NaN, keeps IEEE semantics.
SOURCE_FLAGS = {"attn_prefill_dma.hip": ["-fno-honor-nans"]}
# Sources whose kernels must build with no register spills and no scratch: their key loops
# issue tile loads the compiler does not track and wait on them with counted waits, which a
# spill (a counted scratch access) inside the loop would break. The compiler's resource
# remarks are read for them on every build.
NO_SPILL = ("attn_prefill_dma.hip",)
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
NOISE = "is not a recognized feature for this target"


def spilling_kernels(remarks: str) -> list:
    """(kernel, what) for every kernel whose resource remarks report a vector-register spill
    or a non-zero scratch size. Scalar registers spilled with no scratch went to lanes of a
    vector register (register moves, no memory access) and pass."""
    bad = []
    name = None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+(VGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and name and int(m.group(2)) != 0:
            bad.append((name, f"{m.group(1)} {m.group(2)}"))
    return bad


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    remarks = [ln for ln in msgs if "kernel-resource-usage" in ln]
    msgs = [ln for ln in msgs if "kernel-resource-usage" not in ln]
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return "\n".join(remarks)


def build(extra_flags=None, out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP/C++ source (each with its own flags) and link ``out``
    (atomically replaced)."""
    objs = []
    with tempfile.TemporaryDirectory(prefix="mixer_build_") as tmpdir:
        for src in SOURCES:
            base = os.path.basename(src)
            obj = os.path.join(tmpdir, base + ".o")
            remarks = _run([HIPCC, *FLAGS, *SOURCE_FLAGS.get(base, []),
                            *(RESOURCE_REMARKS if base in NO_SPILL else []),
                            *(extra_flags or []), "-c", src, "-o", obj], verbose)
            if base in NO_SPILL:
                bad = spilling_kernels(remarks)
                if bad:
                    raise RuntimeError(f"{base}: kernels spill vector registers or use "
                                       f"scratch, which the untracked tile loads do not "
                                       f"allow: {bad}")
            objs.append(obj)
        tmp = out + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def needs_build() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
