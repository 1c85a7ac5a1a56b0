"""Build the gfx950 shared library ``libdts_moe.so`` in-tree with hipcc.

Each kernel family sits in a translation unit of its own (csrc/*.hip); the
units compile in parallel to objects under ``_build/`` and are linked into one
shared library.  ``--resource-usage`` also writes the compiler's per-kernel
register / scratch report and fails the build if a persistent kernel spills
to scratch memory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdts_moe.so")
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
ARCH = os.environ.get("DTS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms stay off (a known-fragile instruction family)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def units():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".hpp"))) + [os.path.join(ROOT, "include", "moe.h")]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _clean(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def _obj(src: str) -> str:
    return os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")


def _up_to_date(src: str) -> bool:
    """An object is current when it is newer than its unit and every header
    (each unit includes most of them)."""
    obj = _obj(src)
    if not os.path.exists(obj):
        return False
    t = os.path.getmtime(obj)
    deps = [src] + [s for s in sources() if s.endswith(".hpp")]
    if os.path.basename(src) == "moe.hip":           # the only unit with the C header
        deps.append(os.path.join(ROOT, "include", "moe.h"))
    return all(os.path.getmtime(d) <= t for d in deps)


def _compile(src: str, remarks: bool):
    obj = _obj(src)
    cmd = [_hipcc()] + HIPCC_FLAGS + ["-c", src, "-o", obj]
    if remarks:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return src, obj, r.returncode, _clean(r.stdout)


def parse_resource_usage(text: str):
    """Per-kernel VGPRs, AGPRs, scratch bytes/lane and occupancy from the
    compiler's kernel-resource-usage remarks."""
    out = {}
    name = None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        if name is None:
            continue
        for key, pat in (("vgprs", r"remark:\s+VGPRs: (\d+)"), ("agprs", r"remark:\s+AGPRs: (\d+)"),
                         ("scratch", r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)"),
                         ("sgprs", r"remark:\s+TotalSGPRs: (\d+)")):
            m = re.search(pat, line)
            if m:
                out[name][key] = int(m.group(1))
    return out


def build(verbose: bool = False, resource_usage: bool = False, jobs: int = 0,
          force: bool = True) -> str:
    """Compile every unit (force) or only the out-of-date ones, then link."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = units()
    if not force and not resource_usage:
        todo = [s for s in srcs if not _up_to_date(s)]
        if verbose:
            print("out of date: %s" % [os.path.basename(s) for s in todo], flush=True)
        objs_all = [_obj(s) for s in srcs]
        srcs = todo
    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 1))
    if verbose:
        print("hipcc %s -c <unit> (%d units, %d in parallel)" % (" ".join(HIPCC_FLAGS), len(srcs), jobs),
              flush=True)
    objs = []
    report = []
    if srcs:
        with cf.ThreadPoolExecutor(max_workers=jobs or len(srcs)) as ex:
            for src, obj, rc, out in ex.map(lambda s: _compile(s, resource_usage), srcs):
                if rc != 0:
                    raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(src), out))
                objs.append(obj)
                report.append(out)
    if not force and not resource_usage:
        objs = objs_all
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + _clean(r.stdout))
    os.replace(tmp, LIB)
    if resource_usage:
        usage = parse_resource_usage("\n".join(report))
        spills = {k: v for k, v in usage.items()
                  if ("k_dynamic" in k or "k_static" in k) and v.get("scratch", 0) > 0}
        for k, v in sorted(usage.items()):
            print("%-44s vgpr %3d agpr %3d sgpr %3d scratch %4d occ %d" % (
                k, v.get("vgprs", -1), v.get("agprs", -1), v.get("sgprs", -1),
                v.get("scratch", -1), v.get("occupancy", -1)))
        if spills:
            raise RuntimeError("persistent kernels spill to scratch: %s" % sorted(spills))
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in sources())


if __name__ == "__main__":
    ru = "--resource-usage" in sys.argv
    print(build(verbose=True, resource_usage=ru, force="--incremental" not in sys.argv))
    sys.exit(0)
