"""Builds libpsb.so in-tree with hipcc for gfx950.

    python -m packed_sequence_block_amd.build

Every HIP source is compiled with packed-fp32 ops disabled (the code relies on
plain fp32 VALU arithmetic) and linked with the host-only ABI file into one
shared library next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpsb.so")

HIP_SOURCES = ["boundary.hip", "schedule.hip", "attn_fwd.hip", "attn_bwd.hip"]
CPP_SOURCES = ["capi.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no NaN semantics needed (inputs are finite); lets fmaxf map to v_max3_f32
    # without canonicalizing every operand
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpsb")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if lines:
        print("\n".join(lines), file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compiles every source and links ``libpsb.so``; returns its path."""
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in HIP_SOURCES + CPP_SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc, "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-x", "c++", "-c",
                   os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host launch stub went missing fails here, not at load time
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
