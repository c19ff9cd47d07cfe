"""Textbook fp64 softmax attention (numpy), used only as an independent pin.

softmax(scale * Q K^T + mask) V with a causal mask, GQA by contiguous head
groups; nothing here knows about blocks, lists or 4-bit formats."""
import numpy as np


def softmax_attention(q, k, v, causal=True, sm_scale=None):
    """q [B,Hq,N,d], k/v [B,Hkv,N,d] float64 -> out [B,Hq,N,d] float64."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if sm_scale is None else sm_scale
    out = np.empty((B, Hq, N, d))
    for b in range(B):
        for h in range(Hq):
            g = h * Hkv // Hq
            s = scale * (q[b, h] @ k[b, g].T)
            if causal:
                s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[b, h] = (p @ v[b, g]) / p.sum(axis=1, keepdims=True)
    return out
