"""Build libnvfp4_router.so for gfx950 with hipcc (in-tree, next to this file)."""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4_router.so")
SOURCES = ["router_api.hip", "quantize.hip", "gate.hip", "gate_mfma_e4.hip", "gate_mfma_e8.hip", "gate_mfma_e16.hip", "gate_mfma_e24.hip", "gate_mfma_e32.hip", "gate_decode.hip", "gate_batch.hip", "probe.hip", "lmhead.hip", "grouped.hip"]

COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 arithmetic stays off: hipcc would otherwise form
    # v_pk_{add,mul,fma}_f32 from plain float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def build(verbose=False, extra_flags=()):
    """Compile every HIP source (one hipcc process each, in parallel) and link
    the shared library; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        cmd = [hipcc()] + COMPILE_FLAGS + list(extra_flags) + ["-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), s))
        objs.append(obj)
    failed = [s for p, s in procs if p.wait() != 0]
    if failed:
        raise RuntimeError("hipcc failed on " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
