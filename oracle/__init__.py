"""CPU oracle for one Mixture-of-Experts layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and the two share no code: the oracle is plain C in
``moe_oracle.c`` (fp64 arithmetic, ascending-index sums, no blocking), loaded
here through ctypes.

The functions follow the layer stages the Weave pages list (router, top-k,
per-expert FFN, weighted merge: xxqk.cn/news/665650 section 1;
m.xxqk.cn/news/657744 section 1.1) with the formulas written out in the
header comment of ``moe_oracle.c``.

Inputs are numpy arrays.  bf16 tensors are passed as their raw ``uint16``
bit patterns and widened exactly inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
            "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.oracle_logits.argtypes = [ci, ci, ci, vp, ci, vp, ci, vp, vp]
        lib.oracle_logits.restype = None
        lib.oracle_route.argtypes = [ci, ci, ci, ci, ci, vp, vp, vp, vp, vp,
                                     vp, vp, vp]
        lib.oracle_route.restype = ci
        lib.oracle_moe_rows.argtypes = [ci] * 9 + [vp, ci] + [vp] * 6 + [
            ci, vp, vp, vp, ci, vp, vp]
        lib.oracle_moe_rows.restype = None
        lib.oracle_moe_layer.argtypes = [ci] * 9 + [vp, ci] + [vp] * 6 + [
            ci, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_moe_layer.restype = None
        lib.oracle_residual_rmsnorm.argtypes = [ci, ci, vp, vp, vp, ctypes.c_double, vp, vp]
        lib.oracle_residual_rmsnorm.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ci
        _lib = lib
    return _lib


def _arr(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_of(a) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs must be float32 or bf16 bits as uint16, got %s" % a.dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def logits(x, wr, bias=None) -> np.ndarray:
    """Router logits [T,E] fp32: fp64 sum over ascending i, bias last."""
    lib = _load()
    x = _arr(x)
    wr = _arr(wr)
    T, d = x.shape
    E = wr.shape[1]
    assert wr.shape[0] == d
    b = None if bias is None else _arr(bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib.oracle_logits(T, d, E, _ptr(x), _dtype_of(x), _ptr(wr), _dtype_of(wr),
                      _ptr(b), _ptr(out))
    return out


def route(lg, k: int, e_begin: int = 0, e_end: int | None = None) -> dict:
    """Expert choice, weights, counts, offsets and stable positions."""
    lib = _load()
    lg = _arr(lg, np.float32)
    T, E = lg.shape
    if e_end is None:
        e_end = E
    E_loc = e_end - e_begin
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    counts = np.empty(E_loc, np.int32)
    offsets = np.empty(E_loc + 1, np.int32)
    perm = np.empty(max(T * k, 1), np.int32)
    slot_pos = np.empty((T, k), np.int32)
    rw = np.empty(max(T * k, 1), np.float64)
    R = lib.oracle_route(T, E, k, e_begin, e_end, _ptr(lg), _ptr(idx), _ptr(w),
                         _ptr(counts), _ptr(offsets), _ptr(perm),
                         _ptr(slot_pos), _ptr(rw))
    if R == -1:
        raise FloatingPointError("non-finite router logit")
    if R < 0:
        raise ValueError("bad routing arguments")
    return dict(idx=idx, w=w, counts=counts, offsets=offsets, perm=perm[:R],
                slot_pos=slot_pos, rw=rw[:R], R=R)


def _shared(ws):
    if ws is None:
        return 0, 0, None, None, None
    sg, su, sd = (_arr(a) for a in ws)
    return sg.shape[0], sg.shape[2], sg, su, sd


def moe_rows(x, wg, wu, wd, routing: dict, tokens, e_begin: int = 0,
             shared=None) -> np.ndarray:
    """y rows (float64) for the listed tokens, given routing from ``route``."""
    lib = _load()
    x = _arr(x)
    wg, wu, wd = _arr(wg), _arr(wu), _arr(wd)
    T, d = x.shape
    E_loc, _, f = wg.shape
    k = routing["idx"].shape[1]
    ns, fs, sg, su, sd = _shared(shared)
    if ns:
        assert _dtype_of(sg) == _dtype_of(wg)
    tok = _arr(np.asarray(tokens), np.int32)
    y = np.empty((tok.size, d), np.float64)
    lib.oracle_moe_rows(T, d, 0, k, f, e_begin, e_begin + E_loc, ns, fs,
                        _ptr(x), _dtype_of(x), _ptr(wg), _ptr(wu), _ptr(wd),
                        _ptr(sg), _ptr(su), _ptr(sd), _dtype_of(wg),
                        _ptr(_arr(routing["idx"], np.int32)),
                        _ptr(_arr(routing["w"], np.float64)),
                        _ptr(_arr(routing["slot_pos"], np.int32)), tok.size,
                        _ptr(tok), _ptr(y))
    return y


def moe_layer(x, wg, wu, wd, routing: dict, e_begin: int = 0,
              shared=None) -> np.ndarray:
    """Whole-layer y [T,d] float64 (explicit gather, per-expert FFN, combine)."""
    lib = _load()
    x = _arr(x)
    wg, wu, wd = _arr(wg), _arr(wu), _arr(wd)
    T, d = x.shape
    E_loc, _, f = wg.shape
    k = routing["idx"].shape[1]
    ns, fs, sg, su, sd = _shared(shared)
    R = int(routing["R"])
    O = np.empty((max(R, 1), d), np.float64)
    y = np.empty((T, d), np.float64)
    perm = _arr(routing["perm"], np.int32)
    if perm.size == 0:
        perm = np.zeros(1, np.int32)
    lib.oracle_moe_layer(T, d, 0, k, f, e_begin, e_begin + E_loc, ns, fs,
                         _ptr(x), _dtype_of(x), _ptr(wg), _ptr(wu), _ptr(wd),
                         _ptr(sg), _ptr(su), _ptr(sd), _dtype_of(wg),
                         _ptr(_arr(routing["idx"], np.int32)),
                         _ptr(_arr(routing["w"], np.float64)),
                         _ptr(_arr(routing["offsets"], np.int32)), _ptr(perm),
                         _ptr(_arr(routing["slot_pos"], np.int32)), _ptr(O),
                         _ptr(y))
    return y


def residual_rmsnorm(y, residual, gamma, eps: float):
    """h = residual + y and hn = RMSNorm(h) * gamma, both float64 [T,d]
    (the layer tail: residual add, then the next block's RMSNorm)."""
    lib = _load()
    y = _arr(y, np.float64)
    T, d = y.shape
    res = None if residual is None else _arr(residual, np.float32)
    g = _arr(gamma, np.float32)
    assert g.shape == (d,) and (res is None or res.shape == (T, d))
    h = np.empty((T, d), np.float64)
    hn = np.empty((T, d), np.float64)
    lib.oracle_residual_rmsnorm(T, d, _ptr(y), _ptr(res), _ptr(g), float(eps), _ptr(h), _ptr(hn))
    return h, hn


def full(x, wr, bias, wg, wu, wd, k: int, e_begin: int = 0, e_end=None,
         shared=None, logits_override=None):
    """Route and run the whole layer; returns (y, routing, logits)."""
    lg = logits(x, wr, bias) if logits_override is None else _arr(
        logits_override, np.float32)
    r = route(lg, k, e_begin, e_end)
    y = moe_layer(x, wg, wu, wd, r, e_begin, shared)
    return y, r, lg
