"""Pins of the float64 attention oracle against things other than itself:
closed forms, a hand-derived fixture, brute force with math.fsum, a library
routine (torch's float64 CPU attention) and invariants of exact attention.

Each pin is chosen so that a plausible slip in the oracle fails at least one:
a transposed product (brute force, fixture), a wrong scale (fixture, brute
force), the causal mask in the wrong direction (causal row 0, fixture), a
missing max subtraction (one-hot with a huge scale overflows), a wrong LSE
term (closed-form LSE checks), a wrong normaliser (ones-V and hull checks).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, attention_sampled
import fa_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_force(q, k, v, causal, scale):
    """Pure-Python double loop with math.fsum, one query at a time."""
    N, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(N)]
    lse = [0.0] * N
    for i in range(N):
        keys = range(i + 1) if causal else range(N)
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        for t in range(d):
            o[i][t] = math.fsum(w[a] * v[j][t] for a, j in enumerate(keys)) / z
        lse[i] = m + math.log(z)
    return np.array(o), np.array(lse)


def test_golden_two_keys():
    g = json.load(open(os.path.join(GOLDEN, "two_keys_closed_form.json")))
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for causal, key in ((False, "noncausal"), (True, "causal")):
        o, lse = attention(q, k, v, causal=causal, scale=g["scale"])
        np.testing.assert_allclose(o[0, 0], np.array(g[key]["o"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], np.array(g[key]["lse"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("N", [1, 2, 3, 17, 65])
@pytest.mark.parametrize("d", [4, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(N, d, causal):
    rng_seed = 1000 + 10 * N + d + causal
    q, k, v = (_rand((N, d), rng_seed + i) for i in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention(q[None, None], k[None, None], v[None, None], causal, scale)
    ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    np.testing.assert_allclose(o[0, 0], ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_library_sdpa_float64(causal):
    torch = pytest.importorskip("torch")
    B, H, N, d = 2, 3, 129, 96
    q, k, v = (_rand((B, H, N, d), 7 + i) for i in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention(q, k, v, causal, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ot.numpy(), rtol=0, atol=1e-12)
    s = scale * torch.matmul(tq, tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    B, H, N, d = 1, 2, 200, 64
    q = _rand((B, H, N, d), 1)
    krow = _rand((d,), 2)
    k = np.broadcast_to(krow, (B, H, N, d)).copy()
    v = _rand((B, H, N, d), 3)
    scale = 0.125
    o, lse = attention(q, k, v, causal, scale)
    if causal:
        counts = np.arange(1, N + 1)[None, None, :, None]
        expect = np.cumsum(v, axis=2) / counts
        expect_lse = scale * (q @ krow) + np.log(np.arange(1, N + 1))[None, None, :]
    else:
        expect = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        expect_lse = scale * (q @ krow) + np.log(N)
    np.testing.assert_allclose(o, expect, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, expect_lse, rtol=0, atol=1e-12)


def test_causal_row0_is_v0():
    B, H, N, d = 2, 2, 300, 128
    q, k, v = (_rand((B, H, N, d), 40 + i) for i in range(3))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention(q, k, v, True, scale)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-12)


def test_single_key():
    q, k, v = (_rand((1, 1, 1, 64), 50 + i) for i in range(3))
    for causal in (False, True):
        o, lse = attention(q, k, v, causal, 0.3)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse[0, 0, 0], 0.3 * float(q[0, 0, 0] @ k[0, 0, 0]), atol=1e-12)


def test_one_hot_query_huge_scale_selects_argmax_row():
    N, d = 257, 64
    rng = np.random.default_rng(60)
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    cols = np.arange(N) % d
    q = np.zeros((N, d))
    q[np.arange(N), cols] = 1.0
    scale = 1e4          # exp(S) overflows unless the row max is subtracted
    for causal in (False, True):
        o, lse = attention(q[None, None], k[None, None], v[None, None], causal, scale)
        for i in range(N):
            keys = np.arange(i + 1) if causal else np.arange(N)
            col = k[keys, cols[i]]
            j = keys[np.argmax(col)]
            gap = np.sort(col)[-1] - (np.sort(col)[-2] if len(col) > 1 else -np.inf)
            if gap * scale < 50:
                continue      # near-tie: the closed form needs a unique maximum
            np.testing.assert_allclose(o[0, 0, i], v[j], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[0, 0, i], scale * k[j, cols[i]], rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, N, d = 1, 2, 150, 32
    q, k, v = (_rand((B, H, N, d), 70 + i) for i in range(3))
    scale = 0.2
    o, lse = attention(q, k, v, causal, scale)
    # rows of P sum to one: V = ones gives O = ones
    o1, _ = attention(q, k, np.ones_like(v), causal, scale)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-12)
    # O lies in the hull of the attended V rows (per coordinate)
    for i in (0, 1, N // 2, N - 1):
        keys = slice(0, i + 1) if causal else slice(0, N)
        assert np.all(o[:, :, i] <= v[:, :, keys].max(axis=2) + 1e-12)
        assert np.all(o[:, :, i] >= v[:, :, keys].min(axis=2) - 1e-12)
    # linear in V
    v2 = _rand((B, H, N, d), 80)
    o2, _ = attention(q, k, v2, causal, scale)
    o3, _ = attention(q, k, 2.0 * v - 3.0 * v2, causal, scale)
    np.testing.assert_allclose(o3, 2.0 * o - 3.0 * o2, rtol=0, atol=1e-11)
    # adding u to every key leaves O unchanged and shifts LSE by scale * q.u
    u = _rand((d,), 81)
    o4, lse4 = attention(q, k + u, v, causal, scale)
    np.testing.assert_allclose(o4, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse4, lse + scale * (q @ u), rtol=0, atol=1e-11)
    # rotating Q and K by an orthogonal matrix leaves O and LSE unchanged
    m, _ = np.linalg.qr(_rand((d, d), 82))
    o5, lse5 = attention(q @ m, k @ m, v, causal, scale)
    np.testing.assert_allclose(o5, o, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse5, lse, rtol=0, atol=1e-11)


def test_key_permutation_invariance_noncausal():
    B, H, N, d = 1, 1, 100, 16
    q, k, v = (_rand((B, H, N, d), 90 + i) for i in range(3))
    perm = np.random.default_rng(93).permutation(N)
    o, lse = attention(q, k, v, False, 0.25)
    op, lsep = attention(q, k[:, :, perm], v[:, :, perm], False, 0.25)
    np.testing.assert_allclose(op, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lsep, lse, rtol=0, atol=1e-12)


def test_sampled_rows_match_full():
    B, H, N, d = 2, 2, 70, 16
    q, k, v = (_rand((B, H, N, d), 100 + i) for i in range(3))
    for causal in (False, True):
        o, lse = attention(q, k, v, causal)
        samples = np.array([[0, 0, 0], [1, 1, 69], [0, 1, 33], [1, 0, 7]])
        os_, ls = attention_sampled(q, k, v, samples, causal)
        for r, (b, h, i) in enumerate(samples):
            np.testing.assert_allclose(os_[r], o[b, h, i], rtol=0, atol=1e-14)
            np.testing.assert_allclose(ls[r], lse[b, h, i], rtol=0, atol=1e-14)


def test_row_chunking_does_not_change_rows(monkeypatch):
    import importlib
    oa = importlib.import_module("oracle.attention")
    q, k, v = (_rand((1, 1, 300, 8), 110 + i) for i in range(3))
    o_full, l_full = attention(q, k, v, True)
    monkeypatch.setattr(oa, "ROW_CHUNK", 7)
    o_chunk, l_chunk = oa.attention(q, k, v, True)
    np.testing.assert_allclose(o_chunk, o_full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l_chunk, l_full, rtol=0, atol=1e-13)


def test_input_generator_rounding_and_seeding():
    x = fa_inputs.make_qkv(1, 2, 33, 64, seed=5)
    y = fa_inputs.make_qkv(1, 2, 33, 64, seed=5)
    np.testing.assert_array_equal(x.q_bits, y.q_bits)
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    q32 = rng.standard_normal((1, 2, 33, 64), dtype=np.float32)
    ref = torch.from_numpy(q32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(x.q, ref)
    # outlier model: a fraction ~1e-3 of entries are large
    z = fa_inputs.make_qkv(2, 16, 1024, 128, seed=5, dist="outlier_replace")
    frac = np.mean(np.abs(z.q) > 6)
    assert 2e-4 < frac < 2e-3


# --- queries and keys of different lengths (decode) ---------------------------

def brute_force_kv(q, k, v, causal, scale):
    """Pure-Python loops; query i stands at position i + Nk - Nq."""
    Nq, Nk, d = len(q), len(k), len(q[0])
    o = np.zeros((Nq, d))
    lse = np.zeros(Nq)
    for i in range(Nq):
        keys = range(i + Nk - Nq + 1) if causal else range(Nk)
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        for t in range(d):
            o[i, t] = math.fsum(w[a] * v[j][t] for a, j in enumerate(keys)) / z
        lse[i] = m + math.log(z)
    return o, lse


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 7), (3, 9), (5, 5), (4, 11)])
@pytest.mark.parametrize("causal", [False, True])
def test_kv_brute_force(Nq, Nk, causal):
    from oracle import attention_kv
    d = 5
    q = _rand((1, 1, Nq, d), 700 + Nq)
    k, v = _rand((1, 1, Nk, d), 710 + Nk), _rand((1, 1, Nk, d), 720 + Nk)
    o, lse = attention_kv(q, k, v, causal, 0.7)
    ob, lb = brute_force_kv(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.7)
    np.testing.assert_allclose(o[0, 0], ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lb, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_equal_lengths_is_attention(causal):
    from oracle import attention_kv
    q, k, v = (_rand((2, 3, 70, 16), 730 + i) for i in range(3))
    o1, l1 = attention(q, k, v, causal, 0.25)
    o2, l2 = attention_kv(q, k, v, causal, 0.25)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_kv_identical_keys_mean_over_visible_prefix():
    """Equal scores: O_i is the mean of V over the keys query i sees, which
    with the end alignment are keys 0 .. i + Nk - Nq."""
    from oracle import attention_kv
    Nq, Nk, d = 6, 40, 8
    q = _rand((1, 1, Nq, d), 740)
    k = np.broadcast_to(_rand((d,), 741), (1, 1, Nk, d)).copy()
    v = _rand((1, 1, Nk, d), 742)
    o, lse = attention_kv(q, k, v, True, 0.5)
    for i in range(Nq):
        n = i + Nk - Nq + 1
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0, i], 0.5 * float(q[0, 0, i] @ k[0, 0, 0]) + math.log(n),
                                   rtol=0, atol=1e-12)
    o, _ = attention_kv(q, k, v, False, 0.5)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (Nq, d)), atol=1e-12)


def test_kv_causal_needs_enough_keys():
    from oracle import attention_kv
    x = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        attention_kv(x, x[:, :, :3], x[:, :, :3], True)
