"""Independent numpy fp64 brute force used to pin the oracle (tests only).

It computes the layer a different way from the oracle: every expert is
applied densely to every token with numpy matmuls, the softmax is taken over
all E experts and renormalised over the chosen k, and the chosen outputs are
combined through a dense [T,E] weight mask.  Nothing here is shared with the
oracle's C code.
"""
import numpy as np


def widen(a):
    """fp32 stays fp32; bf16 bit patterns (uint16) become the exact fp32."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def topk_stable(logits32, k):
    """Indices of the k largest fp32 logits per row, ties to the lower index
    (numpy's stable sort on the negated values; -0.0 == +0.0 under <)."""
    neg = -logits32.astype(np.float64)
    order = np.argsort(neg, axis=1, kind="stable")
    return order[:, :k]


def softmax64(z):
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True)


def swiglu_dense(x64, wg64, wu64, wd64):
    g = x64 @ wg64
    u = x64 @ wu64
    h = g / (1.0 + np.exp(-g)) * u
    return h @ wd64


def moe_dense(x, wr, bias, wg, wu, wd, k, e_begin=0, e_end=None, shared=None,
              logits32=None):
    """Returns (y [T,d] fp64, idx [T,k], w [T,k] fp64, logits fp64)."""
    x64 = widen(x).astype(np.float64)
    wr64 = widen(wr).astype(np.float64)
    lg64 = x64 @ wr64
    if bias is not None:
        lg64 = lg64 + np.asarray(bias, np.float64)[None, :]
    if logits32 is None:
        logits32 = lg64.astype(np.float32)
    T, E = logits32.shape
    if e_end is None:
        e_end = E
    idx = topk_stable(logits32, k)
    p = softmax64(logits32.astype(np.float64))
    psel = np.take_along_axis(p, idx, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    mask = np.zeros((T, E), np.float64)
    np.put_along_axis(mask, idx, w, axis=1)
    y = np.zeros((T, x64.shape[1]), np.float64)
    wg64, wu64, wd64 = (widen(a).astype(np.float64) for a in (wg, wu, wd))
    for e in range(e_begin, e_end):
        out = swiglu_dense(x64, wg64[e - e_begin], wu64[e - e_begin],
                           wd64[e - e_begin])
        y += mask[:, e:e + 1] * out
    if shared is not None:
        sg, su, sd = (widen(a).astype(np.float64) for a in shared)
        for s in range(sg.shape[0]):
            y += swiglu_dense(x64, sg[s], su[s], sd[s])
    return y, idx, w, lg64
