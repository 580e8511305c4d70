"""CPU checks of the structured ramp workload (fa_inputs.make_qkv_ramp) that
the GPU tests use to exercise the online softmax's rescaling, and of the
backward's rounding bound (tests/gpu_util.bwd_rounding_bound) that gates the
backward on it.

With iid N(0,1) inputs a row's running maximum settles at the first key tile:
a kernel whose rescale factor were wrong would still pass every iid case. The
ramp workload makes scores grow along the key axis. Here an fp64 emulation of
the kernels' lazy online softmax (per wave of 32 queries, tiles of 64 keys,
the reference maximum moved only when some row of the wave grows by more
than 8 log2 units, then O and l multiplied by exp2(old - new)) shows that:
  * the reference moves several times per wave, with factors strictly
    between 0 and 1;
  * the emulation matches the oracle to rounding;
  * the same emulation with the factor mistaken (exp instead of exp2, not
    applied to O, applied to neither) misses the bf16 output gate by a wide
    margin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import fa_inputs
from oracle import attention, attention_backward
from tests.gpu_util import bf16_gate, bwd_rounding_bound, half_ulp_bf16, ramp_amp

LOG2E = 1.4426950408889634
N, D = 1000, 128
GROWTH = 33.0   # log2 units over the N keys: about 8.5 per 256 keys


def lazy_softmax(q, k, v, causal, mistake=None):
    """Lazy online softmax of one head, float64, in the kernels' order.
    Returns (O, number of reference moves per wave, number of row factors
    strictly between 0 and 1)."""
    n, d = q.shape
    s2 = (q @ k.T) / math.sqrt(d) * LOG2E
    out = np.empty((n, v.shape[1]))
    moves, partial = [], 0
    for w0 in range(0, n, 32):
        rows = np.arange(w0, min(n, w0 + 32))
        ss = s2[rows]
        if causal:
            ss = np.where(np.arange(n)[None, :] > rows[:, None], -np.inf, ss)
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        o = np.zeros((len(rows), v.shape[1]))
        nm = 0
        for j0 in range(0, n, 64):
            st = ss[:, j0:j0 + 64]
            mt = st.max(axis=1)
            with np.errstate(invalid="ignore"):
                grow = np.any(mt - m > 8.0)
            if grow:
                mn = np.maximum(m, mt)
                fin = np.isfinite(m)
                if mistake == "exp":
                    a = np.where(fin, np.exp(np.where(fin, m - mn, 0.0)), 0.0)
                elif mistake == "none":
                    a = np.where(fin, 1.0, 0.0)
                else:
                    a = np.where(fin, np.exp2(np.where(fin, m - mn, 0.0)), 0.0)
                partial += int(np.sum((a > 0) & (a < 1)))
                l = l * a
                if mistake != "l_only":
                    o = o * a[:, None]
                m = mn
                nm += 1
            mc = np.where(np.isfinite(m), m, 0.0)
            p = np.exp2(st - mc[:, None])
            l = l + p.sum(axis=1)
            o = o + p @ v[j0:j0 + 64]
        out[rows] = o / l[:, None]
        moves.append(nm)
    return out, moves, partial


@pytest.mark.parametrize("causal", [False, True])
def test_ramp_moves_the_reference_and_catches_a_wrong_factor(causal):
    g = fa_inputs.make_qkv_ramp(1, 1, N, D, 21128, 4.0, ramp_amp(D, GROWTH))
    q, k, v = g.q[0, 0], g.k[0, 0], g.v[0, 0]
    ref, _ = attention(g.q, g.k, g.v, causal)
    ref = ref[0, 0]
    o, moves, partial = lazy_softmax(q, k, v, causal)
    assert np.abs(o - ref).max() < 1e-12
    # the first move (from -inf) happens in every wave; the ramp adds more
    assert np.mean(moves) >= (2.5 if causal else 4.0)
    assert partial >= N
    for mistake in ("exp", "none", "l_only"):
        bad, _, _ = lazy_softmax(q, k, v, causal, mistake)
        ok, st = bf16_gate(bad, ref)
        assert not ok and st["max_abs"] > 10 * 1e-2, (mistake, st)


def test_iid_inputs_settle_at_the_first_tile():
    """Why the ramp is needed: on iid N(0,1) inputs the reference moves once
    per wave (from -inf), so no factor strictly between 0 and 1 occurs."""
    g = fa_inputs.make_qkv(1, 1, N, D, 21129)
    _, moves, partial = lazy_softmax(g.q[0, 0], g.k[0, 0], g.v[0, 0], False)
    assert max(moves) == 1 and partial == 0


def _bf16(x):
    return fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_bits(np.asarray(x, dtype=np.float32)))


def _backward_bound_ratio(g, do, causal, drop_tile=False):
    """Worst ratio of |G - R| to the rounding bound (plus half an ulp of the
    output) over one head, G from an fp64 emulation of the backward's
    roundings (P and dS to bf16 as operands, each gradient to bf16), R the
    oracle's gradient with D from the bf16 O."""
    n, d = g.q.shape[2], g.q.shape[3]
    scale = 1.0 / math.sqrt(d)
    o, lse = attention(g.q, g.k, g.v, causal)
    ob = _bf16(o)
    lse32 = lse.astype(np.float32).astype(np.float64)
    ref = attention_backward(g.q, g.k, g.v, do, causal, o=ob)
    q, k, v, dO = g.q[0, 0], g.k[0, 0], g.v[0, 0], do[0, 0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - lse32[0, 0][:, None])
    ds = p * (dO @ v.T - (dO * ob[0, 0]).sum(axis=1)[:, None])
    if drop_tile:   # a planted mistake: one key tile's contributions lost
        p[:, 64:128] = 0.0
        ds[:, 64:128] = 0.0
    got = (_bf16(scale * (_bf16(ds) @ k)), _bf16(scale * (_bf16(ds).T @ q)), _bf16(_bf16(p).T @ dO))
    bounds = bwd_rounding_bound(q, k, v, dO, ob[0, 0], lse32[0, 0], causal, scale)
    worst = 0.0
    for x, r, b in zip(got, (ref[0][0, 0], ref[1][0, 0], ref[2][0, 0]), bounds):
        allowed = b + half_ulp_bf16(np.abs(r) + b) + 1e-7
        worst = max(worst, float((np.abs(x - r) / allowed).max()))
    return worst


@pytest.mark.parametrize("ramp", [False, True])
def test_backward_rounding_bound(ramp):
    """The emulated roundings stay inside the bound (causal, the tighter
    mask), and a dropped key tile leaves it by far."""
    n, d = (640, 64) if ramp else (300, 64)
    g = (fa_inputs.make_qkv_ramp(1, 1, n, d, 9765, 4.0, ramp_amp(d, 8.5 * n / 256)) if ramp
         else fa_inputs.make_qkv(1, 1, n, d, 9064))
    _, do = fa_inputs.make_grad(1, 1, n, d, 9766)
    assert _backward_bound_ratio(g, do, True) < 1.0
    assert _backward_bound_ratio(g, do, True, drop_tile=True) > 10.0
