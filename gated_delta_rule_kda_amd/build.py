"""Build libkda.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m gated_delta_rule_kda_amd.build

Every compile also builds the host side, so this runs on a machine without a
GPU.  Flags: -O3, C++17, gfx950 only, packed fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ into libkda.so (always recompiles)."""
    objs = []
    procs = []
    flags = ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in sources():
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc()] + flags + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that warning is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f) for f in failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
