"""Gradients of exact attention in float64 on the CPU: the oracle the GPU
backward pass is checked against. TEST INFRASTRUCTURE ONLY (see
oracle/__init__.py).

What is computed: for O = softmax(scale * Q K^T) V (the scaled dot-product
attention equation of the droidorbit FlashAttention-3 explainer, introduction)
with the causal mask key j <= query i when asked, and an upstream gradient dO
of the same shape as O, the gradients dQ, dK, dV of the scalar
sum(dO * O) with respect to Q, K and V. The pages name the backward pass
(QbitAI FlashAttention-3 article, benchmark section: forward and backward
timed separately) but do not write it out; this is the definition from the
chain rule through the softmax, written out with nothing fused or reordered:

    S = scale * Q K^T (masked entries -inf),  P = softmax over each row of S
    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)   (the softmax Jacobian)
    dQ = scale * dS K,   dK = scale * dS^T Q

The whole N x N matrices of one (batch, head) are formed; P comes from the
row maximum subtracted before the exponential, as in the forward oracle.

Optional `o`: the row term sum_k P_ik dP_ik equals sum_c dO_ic O_ic (the dot
product of row i of dO with row i of O = P V). A backward pass that is handed
the forward's stored output forms the term that second way, from the O it is
given; passing that O here evaluates the same formula with the same term, so
that the stored output's rounding is part of the reference rather than of the
error. With the exact O both ways agree (pinned in the tests).
"""
from __future__ import annotations

import numpy as np


def _probabilities(q, k, causal, scale):
    s = scale * (q @ k.T)
    if causal:
        n = s.shape[0]
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_backward(q, k, v, do, causal=False, scale=None, o=None):
    """Gradients of sum(dO * attention(Q, K, V)) over [B, H, N, d] inputs.

    Returns (dq, dk, dv), float64 [B, H, N, d]. `scale` defaults to 1/sqrt(d).
    With `o` ([B, H, N, d], a forward output), the row term is sum_c dO_ic O_ic.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    if o is not None:
        o = np.asarray(o, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            p = _probabilities(q[b, h], k[b, h], causal, scale)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            if o is None:
                row = (p * dp).sum(axis=1, keepdims=True)
            else:
                row = (do[b, h] * o[b, h]).sum(axis=1, keepdims=True)
            ds = p * (dp - row)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv
