"""Property tests of the float64 oracle on random small inputs (hypothesis):
against a pure-Python brute force built on math.fsum, and the invariants of
exact attention (softmax-weighted averages of V rows).

Shapes, masks, scales and values are drawn; each property is a fact of the
mathematics, not of the oracle's code, so a slip in the oracle (a transposed
product, a wrong mask direction, a dropped max subtraction, a wrong LSE term)
fails one of them.
"""
import math

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle import attention  # noqa: E402
from tests.test_oracle import brute_force  # noqa: E402

SETTINGS = dict(max_examples=40, deadline=None, derandomize=True)


@st.composite
def problems(draw):
    B = draw(st.integers(1, 2))
    H = draw(st.integers(1, 2))
    N = draw(st.integers(1, 24))
    d = draw(st.sampled_from([1, 2, 3, 8, 16]))
    causal = draw(st.booleans())
    scale = draw(st.sampled_from([0.05, 0.25, 1.0, 4.0]))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    amp = draw(st.sampled_from([0.1, 1.0, 8.0]))
    q, k, v = (amp * rng.standard_normal((B, H, N, d)) for _ in range(3))
    return q, k, v, causal, scale


@settings(**SETTINGS)
@given(problems())
def test_matches_brute_force(p):
    q, k, v, causal, scale = p
    o, lse = attention(q, k, v, causal, scale)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            ob, lb = brute_force(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), causal, scale)
            np.testing.assert_allclose(o[b, h], ob, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], lb, rtol=1e-12, atol=1e-10)


@settings(**SETTINGS)
@given(problems())
def test_rows_are_convex_combinations(p):
    q, k, v, causal, scale = p
    o, _ = attention(q, k, v, causal, scale)
    N = q.shape[2]
    for i in range(N):
        keys = slice(0, i + 1) if causal else slice(0, N)
        lo = v[:, :, keys].min(axis=2)
        hi = v[:, :, keys].max(axis=2)
        assert np.all(o[:, :, i] >= lo - 1e-12) and np.all(o[:, :, i] <= hi + 1e-12)


@settings(**SETTINGS)
@given(problems(), st.floats(-3, 3))
def test_key_shift_moves_only_lse(p, c):
    """Adding u to every key row multiplies every weight of row i by the same
    exp(scale q_i.u): O is unchanged, LSE moves by scale q_i.u."""
    q, k, v, causal, scale = p
    d = q.shape[-1]
    u = c * np.linspace(-1.0, 1.0, d)
    o1, l1 = attention(q, k, v, causal, scale)
    o2, l2 = attention(q, k + u, v, causal, scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(l2, l1 + scale * (q @ u), rtol=1e-10, atol=1e-9)


@settings(**SETTINGS)
@given(problems(), st.floats(-2, 2), st.floats(-2, 2))
def test_linear_in_v(p, a, b):
    q, k, v, causal, scale = p
    w = np.flip(v, axis=-1).copy()
    o_v, _ = attention(q, k, v, causal, scale)
    o_w, _ = attention(q, k, w, causal, scale)
    o_ab, _ = attention(q, k, a * v + b * w, causal, scale)
    np.testing.assert_allclose(o_ab, a * o_v + b * o_w, rtol=1e-9, atol=1e-9)


@settings(**SETTINGS)
@given(problems(), st.integers(0, 2 ** 32 - 1))
def test_joint_key_value_permutation(p, seed):
    """Non-causal attention does not depend on the order of the keys."""
    q, k, v, _, scale = p
    perm = np.random.default_rng(seed).permutation(q.shape[2])
    o1, l1 = attention(q, k, v, False, scale)
    o2, l2 = attention(q, k[:, :, perm], v[:, :, perm], False, scale)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-12)
