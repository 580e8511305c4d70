"""Exact attention in float64 on the CPU: the oracle the GPU path is checked
against. TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed follows the plain definition the pages give:
  * softmax(Q K^T / sqrt(d)) V, the scaled dot-product attention equation
    (droidorbit FlashAttention-3 explainer, introduction and "The Memory
    Bottleneck": standard attention materialises S = Q K^T and
    P = softmax(S) and then multiplies by V).
  * the result of the tiled online-softmax method is the same as this global
    softmax (droidorbit explainer, "Mathematical Formulation: The Online
    Softmax Rescaling Trick"; FAQ on linear attention: FlashAttention is exact).
  * causal attention: query i attends key j only when j <= i (the dibro.site
    FlashAttention-3 post, "Contribuciones clave", causal attention without
    padding; the direction there is garbled, this is the reading used).
  * the per-row log-sum-exp of the scaled scores, natural logarithm, is
    returned beside O (not on the pages; the reading is LSE_i =
    log sum_j exp(S_ij)).
  * queries and keys of different lengths (decode: a few new queries against
    a long key/value cache, which FlashDecoding splits over the key length;
    droidorbit explainer, FAQ on FlashDecoding): the Nq queries are the last
    Nq positions of the Nk-long sequence, so with the causal mask query i
    attends keys j <= i + Nk - Nq (the pages do not say how the positions
    align; this is the reading for decode, where the new token comes last).

Nothing here is blocked, fused or reordered beyond the definition: each query
row's scores are formed whole, the row maximum is subtracted for a stable
exponential (the first of the three passes the explainer's "Mathematical
Formulation" section names), and the normalised row is multiplied by V. Rows
are processed a chunk at a time only to bound memory; every row is computed
from all of its keys.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024


def attention_rows(q_rows, k, v, rows, causal, scale):
    """Exact attention for selected query rows of one (batch, head).

    q_rows : float64 [R, d], the query vectors at sequence positions `rows`.
    k, v   : float64 [N, d].
    rows   : int array [R], the sequence position of each query row.
    Returns (o [R, d], lse [R]) in float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    n = k.shape[0]
    s = scale * (q_rows @ k.T)                          # [R, N] scores
    if causal:
        masked = np.arange(n)[None, :] > rows[:, None]  # key after query
        s = np.where(masked, -np.inf, s)
    m = s.max(axis=1, keepdims=True)                    # row maximum
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)                    # row normaliser
    p = e / z                                           # softmax row
    o = p @ v
    lse = m[:, 0] + np.log(z[:, 0])
    return o, lse


def attention(q, k, v, causal=False, scale=None):
    """Exact attention over [B, H, N, d] float64 tensors.

    Returns (o [B, H, N, d], lse [B, H, N]) in float64. `scale` defaults to
    1/sqrt(d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                rows = np.arange(r0, r1)
                o[b, h, r0:r1], lse[b, h, r0:r1] = attention_rows(
                    q[b, h, r0:r1], k[b, h], v[b, h], rows, causal, scale)
    return o, lse


def attention_kv(q, k, v, causal=False, scale=None):
    """Exact attention of [B, H, Nq, d] queries over [B, H, Nk, d] keys and
    values, the queries placed at positions Nk - Nq .. Nk - 1 (causal needs
    Nq <= Nk). Returns (o [B, H, Nq, d], lse [B, H, Nq]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if causal and Nq > Nk:
        raise ValueError("causal attention needs Nq <= Nk (every query sees a key)")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, Nq, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, ROW_CHUNK):
                r1 = min(Nq, r0 + ROW_CHUNK)
                rows = np.arange(r0, r1) + (Nk - Nq)
                o[b, h, r0:r1], lse[b, h, r0:r1] = attention_rows(
                    q[b, h, r0:r1], k[b, h], v[b, h], rows, causal, scale)
    return o, lse


def attention_sampled(q, k, v, samples, causal=False, scale=None):
    """Exact attention at sampled (b, h, i) positions only.

    samples : int array [S, 3] of (b, h, i).
    Returns (o [S, d], lse [S]).
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    samples = np.asarray(samples, dtype=np.int64)
    o = np.empty((len(samples), v.shape[-1]), dtype=np.float64)
    lse = np.empty(len(samples), dtype=np.float64)
    for idx, (b, h, i) in enumerate(samples):
        oi, li = attention_rows(np.asarray(q[b, h, i:i + 1], dtype=np.float64),
                                k[b, h], v[b, h], np.array([i]), causal, scale)
        o[idx] = oi[0]
        lse[idx] = li[0]
    return o, lse

