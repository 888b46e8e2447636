"""Lookahead-mask attention, written as its definition (dense masked softmax).

"M7.3 - Lookahead Decoding", 0x04A and 0x07A: every current row attends the
whole committed prefix plus the current rows in its visibility set; the
dense packed-mask path applies that set as a mask over [prefix + Q] keys.

out[i, h] = sum_j softmax_j(q[i,h] . k[j, g(h)] / sqrt(dh) over allowed j) v[j, g(h)],
g(h) = h // (H / H_kv), computed in fp64.
"""
from __future__ import annotations

import numpy as np


def lookahead_attention(q, k_prefix, v_prefix, k_new, v_new, visible):
    """q [Q,H,dh]; k/v_prefix [Hkv,T,dh]; k/v_new [Q,Hkv,dh]; visible [Q,Q] bool -> [Q,H,dh] fp64."""
    q = np.asarray(q, np.float64)
    Qn, H, dh = q.shape
    Hkv = k_prefix.shape[0]
    T = k_prefix.shape[1]
    group = H // Hkv
    out = np.zeros((Qn, H, dh))
    allowed = np.concatenate([np.ones((Qn, T), bool), np.asarray(visible, bool)], axis=1)
    for h in range(H):
        g = h // group
        keys = np.concatenate([np.asarray(k_prefix[g], np.float64), np.asarray(k_new[:, g, :], np.float64)])
        vals = np.concatenate([np.asarray(v_prefix[g], np.float64), np.asarray(v_new[:, g, :], np.float64)])
        s = (q[:, h, :] @ keys.T) / np.sqrt(dh)
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vals
    return out
