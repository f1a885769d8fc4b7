"""Builds libolk.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run ``python -m transformer_attention_fwd_amd.build_lib``; the library lands
next to this file, where the binding loads it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libolk.so")
ARCH = "gfx950"

# Packed-FP32 VALU instructions are kept out of the generated code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-unused-result"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [hipcc(), *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for s, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature name; harmless
        text = "\n".join(l for l in text.splitlines()
                         if "is not a recognized feature for this target" not in l)
        if text.strip() and (verbose or pr.returncode):
            print(text, file=sys.stderr)
        if pr.returncode:
            failed.append(s)
    if failed:
        raise RuntimeError("hipcc failed on: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    # --no-undefined: a kernel the host pass dropped (its launch stub missing)
    # fails here instead of when the library is loaded
    subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
