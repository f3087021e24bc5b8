"""Independent re-derivations used to pin the oracle (tests only).

These are written from the definitions in a different form from the oracle:
the retained set as a closed form (sort every eligible token and keep the C
best) instead of a streaming heap, and attention as a dense T x T masked
softmax in float64 instead of per-row gathers.
"""
import math

import numpy as np


def closed_form_retained(r, s, w, C, i):
    """R_i = the C best of {j : s <= j <= i-w, r_j > 0.5} by (score desc, index asc)."""
    r = np.asarray(r, np.float32)
    elig = [j for j in range(s, i - w + 1) if j < len(r) and r[j] > np.float32(0.5)]
    elig.sort(key=lambda j: (-float(r[j]), j))
    return sorted(elig[:C])


def dense_mask(r, s, w, C, T):
    """Boolean [T, T] mask: row i may see key j."""
    m = np.zeros((T, T), bool)
    for i in range(T):
        for j in range(T):
            if j > i:
                continue
            if j < s or j >= i - w + 1:
                m[i, j] = True
        for j in closed_form_retained(r, s, w, C, i):
            m[i, j] = True
    return m


def dense_attention(q, k, v, masks):
    """float64 masked softmax. q [B,T,Hq,D], k/v [B,T,Hkv,D], masks [B,Hkv,T,T]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            logits = q[b, :, h, :] @ k[b, :, g, :].T / math.sqrt(D)
            logits = np.where(masks[b, g], logits, -np.inf)
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[b, :, h, :] = p @ v[b, :, g, :]
    return out
