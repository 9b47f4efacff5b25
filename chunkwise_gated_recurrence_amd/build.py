"""Build libgtrgla.so (HIP for gfx950) in-tree with hipcc.

    python -m chunkwise_gated_recurrence_amd.build [-v]

Objects go to chunkwise_gated_recurrence_amd/_build/, the library to
chunkwise_gated_recurrence_amd/libgtrgla.so, and the benchmark's streaming
ceiling kernel to libgtrgla_ceiling.so. Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libgtrgla.so")
CEILING_PATH = os.path.join(PKG, "libgtrgla_ceiling.so")
ARCH = "gfx950"

SOURCES = ["gla_generic.hip", "gla_fused.hip", "gla_gate.hip", "sswiglu.hip", "gtr_gla_api.cpp",
           "sswiglu_api.cpp", "gtr_gla_noalloc.hip", "gla_span.hip"]

# Packed fp32 instructions are turned off for every HIP translation unit.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# Per-source additions. The Spatial SwiGLU up kernel keeps 22 MFMA accumulators
# across its K loop; in their accumulation-register form the register allocator
# rotates them with about 120 accvgpr moves per K step, more vector-ALU issue
# than the step's MFMA time. The VGPR form keeps each accumulator in place.
SOURCE_FLAGS = {
    "sswiglu.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgtrgla)")


def build(verbose: bool = False, extra_flags: List[str] | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = COMMON_FLAGS + list(extra_flags or [])
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [cc, "-c", os.path.join(CSRC, src), "-o", obj] + flags + SOURCE_FLAGS.get(src, [])
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature name: harmless
        text = "\n".join(l for l in text.splitlines()
                         if "is not a recognized feature for this target" not in l)
        if text.strip() and (verbose or p.returncode):
            print(f"--- {src}\n{text}", file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    # the benchmark's streaming ceiling, a library of its own
    tmp = CEILING_PATH + ".tmp"
    cmd = [cc, "-shared", os.path.join(CSRC, "stream_ceiling.hip"), "-o", tmp] + flags
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, CEILING_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB_PATH)
