"""Build the gfx950 shared library ``libdts_moe.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdts_moe.so")
SRC = os.path.join(PKG, "csrc", "moe.hip")
ARCH = os.environ.get("DTS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-fp32 VALU forms stay off (a known-fragile instruction family)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def sources():
    csrc = os.path.join(PKG, "csrc")
    return sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                  if f.endswith((".hip", ".hpp"))) + [os.path.join(ROOT, "include", "moe.h")]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in sources())


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
