"""Build libkda (the HIP kernels and the C ABI) for gfx950 into this package directory.

    python -m gated_delta_rule_59_amd.build

hipcc compiles every source under csrc/ and links one shared library, libkda.so.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libkda.so")
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if p.returncode != 0:
        sys.stderr.write(text)
        raise RuntimeError(f"hipcc failed for {src}")
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
