"""GPU parity of the bf16 backward pass against the float64 oracle.

The chain is the one a caller runs: the library's forward gives O (bf16) and
LSE, then the backward takes Q, K, V, O, LSE and a seeded dO. The oracle
differentiates exact attention of the same bf16 inputs in float64, with its
row term sum_c dO_ic O_ic formed from the O the backward was given (the
backward's definition: the stored output's rounding is an input, not an
error). The mid-size cases are also held to the exact gradient.

Gate per gradient G with oracle value R (derivation in the design notes: the
kernels round P and dS to bf16 as operands and round G to bf16; an emulation
of exactly that rounding gives a relative RMS error of 2.2e-3 to 2.7e-3 and a
worst element below 4.5e-3 max|R| on these workloads):
  |G - R| <= 1e-2 * max|R| + half a bf16 ulp of R + 1e-4, elementwise, and
  ||G - R||_2 <= 5e-3 * ||R||_2 + 1e-4 * sqrt(size).
The 1e-4 floor covers gradients that vanish exactly (a single key: dK = 0).
Every case prints its name, shape and seed before it touches the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import fa_inputs
from oracle import attention_backward
from tests.gpu_util import bwd_gate, run_bwd

pytestmark = pytest.mark.gpu


def announce(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def check_bwd(fa, B, H, N, d, causal, seed, exact_too=False):
    announce("bwd", B, H, N, d, "causal" if causal else "noncausal", "seed", seed)
    g = fa_inputs.make_qkv(B, H, N, d, seed)
    do_bits, do = fa_inputs.make_grad(B, H, N, d, seed + fa_inputs.SEEDS["grad_offset"])
    got, o = run_bwd(fa, g, do_bits, causal)
    refs = [("given-O", attention_backward(g.q, g.k, g.v, do, causal, o=o))]
    if exact_too:
        refs.append(("exact", attention_backward(g.q, g.k, g.v, do, causal)))
    for kind, ref in refs:
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            ok, st = bwd_gate(x, r)
            announce("  ", kind, name, st)
            assert ok, (kind, name, st)


@pytest.mark.parametrize("causal", [False, True])
def test_small_config(lib, causal):
    check_bwd(lib, 1, 2, 256, 64, causal, fa_inputs.SEEDS["small"])


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 65, 127, 129, 300])
def test_ragged_lengths(lib, N, d):
    for causal in (False, True):
        check_bwd(lib, 1, 2, N, d, causal, 9000 + N + d)


@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_several_heads(lib, d):
    # B*H = 24 heads: a multiple of 8 (one run of heads per accelerator die)
    for causal in (False, True):
        check_bwd(lib, 2, 12, 640, d, causal, 9500 + d)


@pytest.mark.parametrize("causal", [False, True])
def test_mid_config(lib, causal):
    check_bwd(lib, 4, 16, 2048, 128, causal, fa_inputs.SEEDS["mid"], exact_too=True)


def test_deterministic(lib):
    import torch
    announce("bwd determinism 2 8 1000 128 causal")
    g = fa_inputs.make_qkv(2, 8, 1000, 128, 77)
    do_bits, _ = fa_inputs.make_grad(2, 8, 1000, 128, 78)
    from tests.gpu_util import to_device
    q, k, v = to_device(g)
    do = fa_inputs.to_torch_bf16(do_bits, "cuda")
    o, lse = lib.fwd(q, k, v, causal=True)
    a = lib.bwd(q, k, v, o, lse, do, causal=True)
    b = lib.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_scale_argument(lib):
    # a scale other than 1/sqrt(d) reaches both the forward and the backward
    announce("bwd scale 1 2 200 64 causal scale 0.3")
    g = fa_inputs.make_qkv(1, 2, 200, 64, 79)
    do_bits, do = fa_inputs.make_grad(1, 2, 200, 64, 80)
    got, o = run_bwd(lib, g, do_bits, True, scale=0.3)
    ref = attention_backward(g.q, g.k, g.v, do, True, scale=0.3, o=o)
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        ok, st = bwd_gate(x, r)
        announce("  ", name, st)
        assert ok, (name, st)


@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_head_dim_sweep_size_sampled_heads(lib, d):
    """The bench's head-dim sweep workload (B=2 H=16 N=8192 causal) in the
    launch configuration the bench times; the oracle checks two whole
    (batch, head) slices, chosen by seed."""
    import torch
    B, H, N = 2, 16, 8192
    seed = fa_inputs.SEEDS["dim_sweep_base"] + (64, 96, 128, 256).index(d)
    announce("bwd sweep size", B, H, N, d, "causal seed", seed)
    g = fa_inputs.make_qkv(B, H, N, d, seed)
    do_bits, do = fa_inputs.make_grad(B, H, N, d, seed + fa_inputs.SEEDS["grad_offset"])
    got, o = run_bwd(lib, g, do_bits, True)
    rng = np.random.default_rng(seed)
    for bh in rng.choice(B * H, size=2, replace=False):
        b, h = divmod(int(bh), H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = attention_backward(g.q[sl], g.k[sl], g.v[sl], do[sl], True, o=o[sl])
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            ok, st = bwd_gate(x[sl], r)
            announce("  ", (b, h), name, st)
            assert ok, (b, h, name, st)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_closed_forms_at_mid_size(lib, causal):
    """Every K row of a head equal: all scores of a query are equal, so
    P_ij = 1/n_i over the n_i keys it attends (N, or i+1 causal). At the full
    mid size, without the oracle (D_i = dO_i . O_i with the O the backward is
    given, as the backward defines it):
      dV_j = sum_{i attends j} dO_i / n_i,
      dK_j = scale sum_{i attends j} ((dO_i . V_j) - D_i) Q_i / n_i
           (non-causal: scale/N (M V_j - sum_i D_i Q_i), M = sum_i Q_i dO_i^T;
            causal: checked on sampled key rows),
      dQ_i = scale k sum_j dS_ij = scale k (dO_i . mean_j V_j - D_i) / ... = 0
           up to D's use of the bf16 O."""
    import torch
    B, H, N, d = 4, 16, 2048, 128
    announce("bwd identical keys", B, H, N, d, "causal" if causal else "noncausal")
    g = fa_inputs.make_qkv(B, H, N, d, 9700)
    rng = np.random.default_rng(9701)
    krow = fa_inputs.bf16_bits(rng.standard_normal((B, H, 1, d), dtype=np.float32))
    k_bits = np.ascontiguousarray(np.broadcast_to(krow, (B, H, N, d)))
    do_bits, do = fa_inputs.make_grad(B, H, N, d, 9702)
    q = fa_inputs.to_torch_bf16(g.q_bits, "cuda")
    k = fa_inputs.to_torch_bf16(k_bits, "cuda")
    v = fa_inputs.to_torch_bf16(g.v_bits, "cuda")
    dot = fa_inputs.to_torch_bf16(do_bits, "cuda")
    o, lse = lib.fwd(q, k, v, causal=causal)
    dq, dk, dv = lib.bwd(q, k, v, o, lse, dot, causal=causal)
    torch.cuda.synchronize()
    f64 = lambda t: fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(t))
    dq, dk, dv, o64 = f64(dq), f64(dk), f64(dv), f64(o)
    qf, vf = g.q, g.v
    scale = 1.0 / np.sqrt(d)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    D = (do * o64).sum(axis=3)                                   # [B, H, N]
    w = do / n[None, None, :, None]
    if causal:
        dv_ref = np.cumsum(w[:, :, ::-1], axis=2)[:, :, ::-1]
    else:
        dv_ref = np.broadcast_to(w.sum(axis=2, keepdims=True), do.shape)
    ok, st = bwd_gate(dv, dv_ref)
    announce("   dv", st)
    assert ok, st
    if not causal:
        M = np.einsum("bhic,bhie->bhce", qf, do)                 # sum_i Q_i dO_i^T
        dk_ref = scale / N * (np.einsum("bhce,bhje->bhjc", M, vf)
                              - np.einsum("bhi,bhic->bhc", D, qf)[:, :, None, :])
        ok, st = bwd_gate(dk, dk_ref)
        announce("   dk", st)
        assert ok, st
    else:
        for (b, h) in ((0, 0), (1, 7), (2, 11), (3, 15)):
            js = np.array([0, 1, 63, 64, 127, 128, 1000, 2046, 2047] +
                          list(rng.integers(0, N, 23)))
            ref = np.empty((len(js), d))
            for a, j in enumerate(js):
                i = np.arange(j, N)
                coef = (do[b, h, i] @ vf[b, h, j] - D[b, h, i]) / n[i]
                ref[a] = scale * coef @ qf[b, h, i]
            ok, st = bwd_gate(dk[b, h, js], ref)
            announce("   dk rows", (b, h), st)
            assert ok, st
    # dQ_i = scale k (sum_j P_ij dP_ij - D_i) = scale k dO_i . (O_exact - O)_i
    bound = scale * np.abs(fa_inputs.bf16_bits_to_f64(krow)).max() * \
        (np.abs(do) * np.abs(o64)).sum(axis=3).max() * 2.0 ** -8
    announce("   max|dQ|", float(np.abs(dq).max()), "bound", bound)
    assert float(np.abs(dq).max()) <= bound + 1e-3
