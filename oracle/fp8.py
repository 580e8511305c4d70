"""FP8 (OCP e4m3fn) encoding, block quantisation with optional random-sign
Hadamard rotation, and an FP8 attention emulator. TEST INFRASTRUCTURE ONLY
(see oracle/__init__.py).

Passages followed:
  * block-wise quantisation, one scale per block rather than one per tensor
    (QbitAI FlashAttention-3 article, FP8 section; dibro.site post,
    "Arquitectura y metodo": FP8 with per-block quantisation);
  * incoherent processing: Q and K are multiplied by a random orthogonal
    matrix, for example a Hadamard matrix, before quantising; the product
    Q K^T is unchanged because the matrix is orthogonal (FlashAttention-3 (HE),
    "3. FP8 with reduced quantisation error"; QbitAI article, FP8 section);
  * the per-tensor baseline uses one scale for the whole tensor (QbitAI
    article, FP8 accuracy test).

Readings where the pages are silent (each also listed in the design notes):
  * e4m3 is the OCP e4m3fn format: bias 7, 3 mantissa bits, largest finite
    value 448, no infinities, S.1111.111 is NaN.
  * a block is 128 consecutive sequence rows of one (batch, head), all d
    columns. The per-tensor variant uses one block for the whole tensor.
  * the rotation is M = diag(signs) H_d / sqrt(d) with H_d the Sylvester
    Hadamard matrix. The unnormalised product y = (x * signs) H_d is what is
    quantised (its entries are exact in float64 and, for these inputs,
    usually exact in float32); the 1/sqrt(d) is folded into the stored scale.
  * the block scale is s = amax / 448 with amax the largest magnitude of
    the block's (rotated) values, stored as a float32 (the exact quotient
    rounded once; s = 1 for an all-zero block, whose codes are all zero);
    the code of a value y is y / s, clamped to [-448, 448], rounded to the
    nearest e4m3 value with ties to the even code. y and y / s are taken in
    float64 (the rotated sums of bf16 inputs are exact there). The stored
    scale is s, or s / sqrt(d) rounded to float32 when rotated;
    dequantised value = e4m3 value * stored scale.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode(codes):
    """Value of each e4m3fn code (uint8) as float64, from the format's fields."""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# Non-negative finite values, codes 0x00..0x7E, increasing with the code.
_POS_VALUES = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x):
    """Round finite values with |x| <= 448 to e4m3fn codes, nearest value,
    ties to the even code (even mantissa). Returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode expects finite values within +-448")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 1, 0x7E)
    lo = hi - 1
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = code | (np.signbit(x).astype(np.int64) << 7)
    return code.astype(np.uint8)


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_d (entries +-1), d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_unnormalised(x, signs):
    """y = (x * signs) H_d along the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return (x * np.asarray(signs, dtype=np.float64)) @ hadamard(d)


def quantize(x, per_tensor=False, signs=None, block=BLOCK):
    """Block quantisation of a [B, H, N, d] tensor to e4m3fn.

    Returns (codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N/block)]).
    With per_tensor=True every entry of `scales` holds the one tensor scale.
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    y = rotate_unnormalised(x, signs) if signs is not None else x
    nblk = -(-N // block)
    amax = np.zeros((B, H, nblk), dtype=np.float64)
    for t in range(nblk):
        amax[:, :, t] = np.abs(y[:, :, t * block:(t + 1) * block, :]).max(axis=(2, 3))
    if per_tensor:
        amax[...] = amax.max()
    s = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)   # stored in float32
    s_rows = np.repeat(s.astype(np.float64), block, axis=2)[:, :, :N, None]
    t = np.clip(y / s_rows, -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(t)
    if signs is not None:
        stored = (s.astype(np.float64) / np.sqrt(d)).astype(np.float32)
    else:
        stored = s
    return codes, stored


def dequantize(codes, scales, block=BLOCK):
    """float64 values = e4m3 value * the stored scale of the row's block."""
    B, H, N, d = codes.shape
    s_rows = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=2)[:, :, :N, None]
    return e4m3_decode(codes) * s_rows


def fp8_attention_emulate(q_codes, k_codes, v_codes, sq, sk, sv, causal, scale,
                          p_scale=256.0, block=BLOCK, round_p=True):
    """Attention on dequantised FP8 operands with P rounded to e4m3.

    A prediction of the FP8 kernel's error, not a definition of the method
    and not a gate: S = scale * Qd Kd^T from the dequantised (and, if
    rotated, rotated) Q, K; P = exp(S - rowmax); the product P V is taken in
    e4m3 (QbitAI article, FP8 section), so P is multiplied by p_scale (to
    keep small probabilities out of e4m3's subnormal range) and rounded to
    e4m3; the row sum is taken over the same rounded values, i.e. over the
    probabilities the product used: O = sum_j Pq_j Vd_j / sum_j Pq_j.
    Without rounding (round_p=False) this is exact attention on the
    dequantised operands.
    """
    qd = dequantize(q_codes, sq, block)
    kd = dequantize(k_codes, sk, block)
    vd = dequantize(v_codes, sv, block)
    B, H, N, d = qd.shape
    o = np.empty_like(vd)
    for b in range(B):
        for h in range(H):
            s = scale * (qd[b, h] @ kd[b, h].T)
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            if round_p:
                pq = e4m3_decode(e4m3_encode(np.minimum(p * p_scale, E4M3_MAX))) / p_scale
            else:
                pq = p
            o[b, h] = (pq @ vd[b, h]) / pq.sum(axis=1, keepdims=True)
    return o
