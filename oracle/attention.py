"""Exact single-query attention (oracle side).

QEvict notes, section 4.1, Eq.(attention): a_t = softmax(q_t K_acc^T / sqrt(d)),
o_t = a_t V_acc over the keys/values currently accessible (full-precision
windows, dequantized quantized windows; evicted windows contribute nothing).
H2O page, section 1.1: the softmax is renormalized over the kept set D_t, so
dropping a position changes the denominator of every other weight.
GQA: query head h reads KV head floor(h / G), G = H_q / H_kv.
All arithmetic in float64.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray | None = None):
    """q [Hq, d]; k, v [Hkv, T, d]; mask [T] (True = accessible) or [Hkv, T].

    Returns (out [Hq, d], probs [Hq, T]); probabilities of masked positions
    are exactly 0."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hq, d = q.shape
    hkv, T, _ = k.shape
    G = hq // hkv
    qg = q.reshape(hkv, G, d)
    logits = np.matmul(qg, k.transpose(0, 2, 1)) / np.sqrt(d)        # [Hkv, G, T]
    if mask is not None:
        m = np.asarray(mask, bool)
        m = np.broadcast_to(m if m.ndim == 2 else m[None, :], (hkv, T))[:, None, :]
        logits = np.where(m, logits, -np.inf)
    mx = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - mx)
    p = e / e.sum(axis=-1, keepdims=True)
    out = np.matmul(p, v)                                               # [Hkv, G, d]
    return out.reshape(hq, d), p.reshape(hq, T)


def attend_bruteforce(q, k, v, mask=None):
    """The same definition with explicit loops and math.exp (tiny inputs)."""
    import math
    q = np.asarray(q, np.float64)
    hq, d = q.shape
    hkv, T, _ = np.shape(k)
    G = hq // hkv
    out = np.zeros((hq, d))
    probs = np.zeros((hq, T))
    for h in range(hq):
        g = h // G
        idx = [t for t in range(T) if mask is None or (np.ndim(mask) == 1 and mask[t]) or (np.ndim(mask) == 2 and mask[g][t])]
        ls = [sum(float(q[h, c]) * float(k[g][t][c]) for c in range(d)) / math.sqrt(d) for t in idx]
        mx = max(ls)
        ws = [math.exp(x - mx) for x in ls]
        z = sum(ws)
        for t, w in zip(idx, ws):
            probs[h, t] = w / z
            for c in range(d):
                out[h, c] += w / z * float(v[g][t][c])
    return out, probs
