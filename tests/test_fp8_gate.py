"""CPU checks of the FP8 kernel's tolerance (tests/fp8_gate.py): an fp64
emulation of the kernel's rounding of P (a reference maximum up to 2.75 log2
units below the row's, P * 2^6 * r rounded to e4m3 with the fold ratio r
of the key's block, the row sum over the same rounded values) stays inside
the bound on plain, zero-padded and widely spread V scales; planted mistakes
(the fold not undone, one bit less of mantissa for P, a dropped key tile)
leave it."""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs
from oracle import fp8
from tests.fp8_gate import fp8_gate, fp8_reference_and_bounds


def fold_ratios(sv_head, n, tile=64, window=4.0):
    """The V fold ratio of each key: the reference starts at the largest V
    block scale and moves to a tile's scale when the ratio leaves
    [2^-window, 1], tiles taken in key order."""
    ref = sv_head.max()
    r = np.empty(n)
    for j0 in range(0, n, tile):
        s = sv_head[j0 // 128]
        ratio = s / ref
        if ratio > 1 or ratio < 2.0 ** -window:
            ref, ratio = s, 1.0
        r[j0:j0 + tile] = ratio
    return r


def round_e4m3(x, drop_bit=False):
    x = np.minimum(x, 448.0)
    if drop_bit:   # a planted mistake: two mantissa bits instead of three
        e = np.floor(np.log2(np.maximum(x, 2.0 ** -6)))
        q = 2.0 ** (e - 2)
        return np.round(x / q) * q
    return fp8.e4m3_decode(fp8.e4m3_encode(x))


def emulate_kernel(qd, kd, vd, sv, causal, scale, seed, mistake=None):
    rng = np.random.default_rng(seed)
    B, H, N, d = qd.shape
    o = np.empty_like(vd)
    for b in range(B):
        for h in range(H):
            s = scale * (qd[b, h] @ kd[b, h].T)
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
            m = s.max(axis=1, keepdims=True) - rng.uniform(0, 2.75, (N, 1)) * math.log(2)
            p = np.exp(s - m)
            r = fold_ratios(np.asarray(sv[b, h], dtype=np.float64), N)
            x = round_e4m3(p * 64.0 * r[None, :], drop_bit=(mistake == "bit"))
            if mistake == "tile":
                x[:, 64:128] = 0.0
            num = x @ (vd[b, h] / sv[b, h].max() if mistake == "fold" else vd[b, h] / r[:, None])
            den = (x / r[None, :]).sum(axis=1, keepdims=True)
            o[b, h] = num / den
    return fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_bits(o.astype(np.float32)))


def operands(kind, N=333, d=64, seed=5):
    g = fa_inputs.make_qkv(1, 2, N, d, seed, "outlier_replace")
    v = g.v.copy()
    if kind == "zero_block":
        v[:, :, 256:] = 0.0
    elif kind == "spread":
        for t, f in enumerate((100.0, 1.0, 0.01)):
            v[:, :, 128 * t:128 * (t + 1)] *= f
    elif kind == "tiny":
        v *= 1e-3
        v[:, :, 256:] = 0.0
    qc, sq = fp8.quantize(g.q)
    kc, sk = fp8.quantize(g.k)
    vc, sv = fp8.quantize(v)
    return [fp8.dequantize(c, s) for c, s in ((qc, sq), (kc, sk), (vc, sv))], sv


@pytest.mark.parametrize("kind", ["plain", "zero_block", "spread", "tiny"])
@pytest.mark.parametrize("causal", [False, True])
def test_emulated_kernel_inside_bound(kind, causal):
    (qd, kd, vd), sv = operands(kind)
    scale = 1 / 8
    o, lse, bo, bl, var = fp8_reference_and_bounds(qd, kd, vd, sv, causal, scale)
    got = emulate_kernel(qd, kd, vd, sv, causal, scale, 1)
    ok, st = fp8_gate(got, o, bo, var)
    assert ok, st
    assert 0.2 < st["rms_ratio"] < 0.9, st   # not vacuous: the errors reach the allowance


@pytest.mark.parametrize("mistake", ["fold", "bit", "tile"])
def test_planted_mistakes_leave_the_bound(mistake):
    kind = "spread" if mistake == "fold" else "plain"
    (qd, kd, vd), sv = operands(kind)
    o, lse, bo, bl, var = fp8_reference_and_bounds(qd, kd, vd, sv, False, 1 / 8)
    got = emulate_kernel(qd, kd, vd, sv, False, 1 / 8, 2, mistake=mistake)
    ok, st = fp8_gate(got, o, bo, var)
    assert not ok, st
