"""Build the HIP library ``libps.so`` for gfx950 in-tree.

hipcc compiles the kernels and the host-side C ABI (planner, entry points)
into one shared library next to this file. Packed-fp32 instruction
selection is switched off for the device code.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libps.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["ps_capi.cpp", "ps_plan.cpp", "ps_kernels.hip", "ps_rope.hip", "ps_spec.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] + DEVICE if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"]
        cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    failed = []
    for src, p in zip(SOURCES, procs):
        _, err = p.communicate()
        msgs = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
        if msgs and (verbose or p.returncode):
            print("\n".join(msgs), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
