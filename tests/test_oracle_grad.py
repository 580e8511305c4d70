"""Pins of the float64 attention-gradient oracle against things other than
itself: central finite differences of the forward oracle, a library routine's
automatic differentiation (torch, float64, CPU), closed forms, invariants.

A transposed product, a sign or a missing softmax-Jacobian term in the
oracle fails the finite differences; a wrong scale fails them and the library
check; a mask in the wrong direction fails the causal closed form.
"""
import numpy as np
import pytest

from oracle import attention, attention_backward


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N", [1, 3, 6])
@pytest.mark.parametrize("d", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(N, d, causal):
    """d/dx of L = sum(dO * attention(Q, K, V)) by central differences of the
    forward oracle, entry by entry."""
    seed = 100 * N + 10 * d + causal
    q, k, v, do = (_rand((1, 2, N, d), seed + i) for i in range(4))
    scale = 0.7
    grads = attention_backward(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        o, _ = attention(qq, kk, vv, causal, scale)
        return float((do * o).sum())

    h = 1e-6
    for which, g in zip(range(3), grads):
        args = [q, k, v]
        x = args[which]
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_library_autograd_float64(causal):
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 37, 16
    q, k, v, do = (_rand((B, H, N, d), 200 + i) for i in range(4))
    scale = 0.3
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    dq, dk, dv = attention_backward(q, k, v, do, causal, scale)
    for ours, lib in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(ours, lib.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys(causal):
    """All keys equal: every attended key has the same weight (1/N, or
    1/(i+1) causal), so dQ = 0 exactly and dV_j = sum over attending queries
    i of dO_i / (number of keys query i attends)."""
    B, H, N, d = 1, 2, 20, 8
    q, v, do = (_rand((B, H, N, d), 300 + i) for i in range(3))
    k = np.repeat(_rand((B, H, 1, d), 310), N, axis=2)
    dq, dk, dv = attention_backward(q, k, v, do, causal, 0.5)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    counts = np.arange(1, N + 1) if causal else np.full(N, N)
    expect = np.empty_like(dv)
    for j in range(N):
        rows = np.arange(j, N) if causal else np.arange(N)
        expect[:, :, j] = (do[:, :, rows] / counts[rows][None, None, :, None]).sum(axis=2)
    np.testing.assert_allclose(dv, expect, rtol=1e-12, atol=1e-12)


def test_single_key():
    """N = 1: P = 1, so dV = dO and dQ = dK = 0."""
    q, k, v, do = (_rand((2, 2, 1, 4), 400 + i) for i in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, False, 1.3)
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Rows of dS sum to zero, so the dK rows of a (batch, head) sum to zero;
    rows of P sum to one, so the dV rows sum to the dO rows' sum; a shift of
    every key by the same vector leaves O, hence every gradient, unchanged."""
    B, H, N, d = 2, 2, 33, 6
    q, k, v, do = (_rand((B, H, N, d), 500 + i) for i in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, causal, 0.9)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-11)
    u = _rand((d,), 510)
    dq2, dk2, dv2 = attention_backward(q, k + u, v, do, causal, 0.9)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_allclose(b, a, rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_row_term_from_forward_output(causal):
    """With the exact forward output the row term sum_c dO_ic O_ic equals
    sum_j P_ij dP_ij, so passing o changes nothing. Perturbing o by E shifts
    the row term by e_i = sum_c dO_ic E_ic and dS_ij by -P_ij e_i: dV is
    unchanged, dQ_i moves by -scale e_i (P K)_i with (P K)_i the forward
    output for values K, and the dK rows' sum moves by -scale sum_i e_i Q_i
    (rows of P sum to one)."""
    B, H, N, d = 2, 2, 29, 7
    q, k, v, do = (_rand((B, H, N, d), 600 + i) for i in range(4))
    scale = 0.8
    o, _ = attention(q, k, v, causal, scale)
    base = attention_backward(q, k, v, do, causal, scale)
    same = attention_backward(q, k, v, do, causal, scale, o=o)
    for a, b in zip(base, same):
        np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-12)
    e_mat = 1e-3 * _rand((B, H, N, d), 610)
    dq, dk, dv = attention_backward(q, k, v, do, causal, scale, o=o + e_mat)
    e = (do * e_mat).sum(axis=3)                       # [B, H, N]
    pk, _ = attention(q, k, k, causal, scale)
    np.testing.assert_allclose(dv, base[2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dq - base[0], -scale * e[..., None] * pk, rtol=1e-8, atol=1e-13)
    np.testing.assert_allclose((dk - base[1]).sum(axis=2), -scale * (e[..., None] * q).sum(axis=2),
                               rtol=1e-8, atol=1e-13)
