"""Host-only checks (no GPU): the C ABI library loads and exports every
function include/moe.h declares, the ctypes mirror matches the C struct
layout, descriptor validation, and the analysis helpers against the worked
examples printed on the pages."""
import ctypes
import json
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def abi():
    from dynamic_task_scheduling_amd import _abi
    from dynamic_task_scheduling_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    return _abi


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(abi):
    names = declared_functions()
    assert set(names) == set(abi.EXPORTS)
    L = abi.lib()
    for n in names:
        assert hasattr(L, n), n
    # also visible as dynamic symbols of the shared object
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB if hasattr(abi, "LIB") else
                          os.path.join(ROOT, "dynamic_task_scheduling_amd", "libdts_moe.so")],
                         stdout=subprocess.PIPE, text=True).stdout
    for n in names:
        assert re.search(r"\bT %s\b" % n, out), n


def test_struct_layout_matches_header(abi, tmp_path):
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(moe_desc), sizeof(moe_weights),
         sizeof(moe_routing), sizeof(moe_info), offsetof(moe_desc, trace),
         offsetof(moe_desc, timeout_ms), offsetof(moe_info, workspace_bytes),
         offsetof(moe_desc, flags));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    vals = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    exp = [ctypes.sizeof(abi.Desc), ctypes.sizeof(abi.Weights), ctypes.sizeof(abi.Routing),
           ctypes.sizeof(abi.Info), abi.Desc.trace.offset, abi.Desc.timeout_ms.offset,
           abi.Info.workspace_bytes.offset, abi.Desc.flags.offset]
    assert vals == exp


def _desc(abi, **kw):
    d = abi.Desc()
    base = dict(T=128, d=4096, E=8, k=2, f=14336, e_begin=0, e_end=0, n_shared=0, f_shared=0,
                dtype=1, mode=0, split_policy=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_workspace_size_and_validation(abi):
    L = abi.lib()
    ok = L.moe_workspace_size(ctypes.byref(_desc(abi)))
    # holds at least Xp [T*k, d] and H [T*k, f] in bf16
    assert ok >= 2 * 256 * (4096 + 14336)
    bad = [dict(k=9), dict(k=3, E=2), dict(d=100), dict(f=200), dict(E=300), dict(T=-1),
           dict(e_begin=5, e_end=3), dict(n_shared=1, f_shared=100), dict(dtype=7),
           dict(mode=5), dict(split_k=9), dict(claim_batch=9), dict(claim_batch=-1),
           dict(flags=abi.FLAG_LOCAL_QUEUES | abi.FLAG_XCD_AFFINITY),
           dict(flags=abi.FLAG_LOCAL_QUEUES | abi.FLAG_CONT_PRIORITY)]
    for b in bad:
        assert L.moe_workspace_size(ctypes.byref(_desc(abi, **b))) == 0, b
    # bigger problems need more workspace
    assert L.moe_workspace_size(ctypes.byref(_desc(abi, T=256))) > ok


def test_strerror(abi):
    assert abi.strerror(0) == "ok"
    assert "watchdog" in abi.strerror(5)
    assert abi.strerror(12345) == "unknown error"


def test_layer_rejects_bad_arguments_without_gpu(abi):
    """Argument errors are returned before anything touches the device."""
    L = abi.lib()
    d = _desc(abi)
    rc = L.moe_layer(ctypes.byref(d), None, None, None, None, None, 0, None)
    assert rc == 2   # workspace missing is detected first (before any HIP call)
    d.k = 99
    assert L.moe_layer(ctypes.byref(d), None, None, None, None, None, 0, None) == 1


GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_worked_examples.json")))


@pytest.mark.parametrize("case", GOLD["wave_tail"])
def test_wave_tail_matches_pages(case):
    from dynamic_task_scheduling_amd.analysis import wave_tail
    r = wave_tail(case["slots"], case["blocks"])
    assert r["waves"] == 2
    assert r["last_wave_blocks"] == case["last_wave_blocks"]
    assert r["idle_slots"] == case["idle_slots"]


def test_speedup_formulas_match_pages():
    from dynamic_task_scheduling_amd.analysis import amdahl, idle_bound
    for c in GOLD["amdahl"]:
        assert abs(amdahl(c["r"], c["s"]) - c["speedup"]) <= c["tol"]
    for c in GOLD["idle_bound"]:
        assert abs(idle_bound(c["alpha"]) - c["bound"]) <= c["tol"]
    for c in GOLD["composition"]:
        assert abs(sum(c["parts"]) - c["total"]) <= 1e-12
        assert abs(1.0 / c["total"] - c["speedup"]) <= c["tol"]


def test_overlap_efficiency_limits():
    from dynamic_task_scheduling_amd.analysis import overlap_efficiency
    assert overlap_efficiency(10.0, 10.0, 4.0) == 1.0   # shorter stream fully hidden
    assert overlap_efficiency(14.0, 10.0, 4.0) == 0.0   # fully serialised
