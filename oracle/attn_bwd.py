"""Backward of the attention (the *Attention kernels* table's ``attn_bwd`` row: a
gradient-checked backward pass on full fp16 state; the *Infrastructure* table's
autograd row: int8 attention made differentiable).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Reading R17.  The quantization of the forward has zero derivative almost everywhere, so
the differentiable int8 attention takes it as the identity (straight-through): the
backward is the gradient of exact attention

    O = softmax(s * Q K^T + mask) V     (s the softmax scale; causal: key j > query i
                                         masked; GQA: query head h reads kv head h/G)

at the fp16 inputs, contracted with the output gradient dO.  With P the softmax and
D_i = sum_d dO[i, d] O[i, d]:

    dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = s dS K,  dK = s dS^T Q,

and for GQA dK, dV of a kv head sum over the G query heads that read it.  Computed in
fp64 from the fp16 values.
"""

from __future__ import annotations

import numpy as np

from .attn_ref import default_softmax_scale


def attn_bwd_exact(q16, k16, v16, do16, causal=True, softmax_scale=None):
    """Gradients (dq, dk, dv) in fp64 of exact attention (R17) for dense BHSD inputs:
    ``q, do [B,Hq,S,D]``, ``k, v [B,Hkv,S,D]``."""
    q = np.asarray(q16, dtype=np.float64)
    k = np.asarray(k16, dtype=np.float64)
    v = np.asarray(v16, dtype=np.float64)
    do = np.asarray(do16, dtype=np.float64)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    s = np.float64(default_softmax_scale(D) if softmax_scale is None else np.float32(softmax_scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mask = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            logits = np.where(mask, s * (q[b, h] @ k[b, g].T), -np.inf)
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, g]
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            dsc = p * (dp - np.sum(do[b, h] * o, axis=1, keepdims=True))
            dq[b, h] = s * (dsc @ k[b, g])
            dk[b, g] += s * (dsc.T @ q[b, h])
    return dq, dk, dv
