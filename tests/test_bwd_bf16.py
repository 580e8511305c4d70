"""GPU parity of the bf16 backward pass against the float64 oracle.

The backward takes Q, K, V, the forward's O and LSE, and a seeded dO. Here O
and LSE come from the oracle's exact forward (O rounded to bf16, the
forward's output format; LSE to float32), so no output of the library enters
any reference. Each case is held to two references: the oracle's gradient
with its row term sum_c dO_ic O_ic formed from the bf16 O the backward was
given (the backward's definition: the stored output's rounding is an input,
not an error), and the exact gradient.

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
from tests.gpu_util import (bwd_gate, bwd_rounding_bound, half_ulp_bf16, oracle_backward_full,
                            oracle_fwd_inputs, ramp_amp, run_bwd)

pytestmark = pytest.mark.gpu


def announce(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def check_bwd(fa, B, H, N, d, causal, seed, scale=None, heads=None, g=None):
    announce("bwd", B, H, N, d, "causal" if causal else "noncausal", "seed", seed,
             "scale", scale, g.dist if g is not None else "")
    if g is None:
        g = fa_inputs.make_qkv(B, H, N, d, seed)
    do_bits, do = fa_inputs.make_grad(B, H, N, d, seed + fa_inputs.SEEDS["grad_offset"])
    got, o = run_bwd(fa, g, do_bits, causal, scale=scale)
    q, k, v = g.q, g.k, g.v
    given = oracle_backward_full(q, k, v, do, causal, scale, o=o, heads=heads)
    exact = oracle_backward_full(q, k, v, do, causal, scale, heads=heads)
    sel = (slice(None),) if heads is None else (tuple(b for b, _ in heads), tuple(h for _, h in heads))
    for name, x, r, e in zip(("dq", "dk", "dv"), got, given, exact):
        ok, st = bwd_gate(x[sel], r[sel])
        announce("   given-O", name, st)
        assert ok, ("given-O", name, st)
        # Against the exact gradient the gate also allows the oracle's own
        # distance between the two references: the effect of the bf16
        # rounding of O on D = rowsum(dO * O), which the backward's
        # definition takes from the O it is given (large where few keys
        # leave dP - D small, e.g. N = 2).
        ok, st = bwd_gate(x[sel], e[sel], extra=np.abs(r[sel] - e[sel]))
        announce("   exact", name, st)
        assert ok, ("exact", name, st)


@pytest.mark.parametrize("causal", [False, True])
def test_small_config(lib, causal):
    check_bwd(lib, 1, 2, 256, 64, causal, fa_inputs.SEEDS["small"])


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 65, 127, 129, 300])
def test_ragged_lengths(lib, N, d):
    for causal in (False, True):
        check_bwd(lib, 1, 2, N, d, causal, 9000 + N + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ramp_scores(lib, d, causal):
    """Scores growing along the key axis (fa_inputs.make_qkv_ramp, about 8.5
    log2 units every 256 keys): P = exp(scale * S - LSE) is formed from
    large, nearly cancelling terms, each query attends a narrow band of keys,
    and dQ's column 0 is a small difference of large terms (sum_j dS_ij = 0
    against K's ramp column), where rounding dS to bf16 costs several times
    the relative gate of the iid workloads (an fp64 emulation of that
    rounding reaches 1-4% of max|dQ|). Gated elementwise by the bound that
    the kernels' arithmetic implies on any input (bwd_rounding_bound: P and
    dS rounded to bf16, float32 elsewhere) plus the output's rounding; on
    the CPU that emulation sits at 0.4-0.9 of it and a dropped key tile at
    50x or more."""
    B, H, N = 1, 2, 640
    scale = 1.0 / np.sqrt(d)
    g = fa_inputs.make_qkv_ramp(B, H, N, d, 9700 + d + causal, 4.0,
                                ramp_amp(d, 8.5 * N / 256))
    announce("bwd ramp", B, H, N, d, "causal" if causal else "noncausal", "seed", g.seed)
    do_bits, do = fa_inputs.make_grad(B, H, N, d, g.seed + fa_inputs.SEEDS["grad_offset"])
    o_bits, lse = oracle_fwd_inputs(g, causal)
    got, o = run_bwd(lib, g, do_bits, causal, fwd=(o_bits, lse))
    given = oracle_backward_full(g.q, g.k, g.v, do, causal, o=o)
    exact = oracle_backward_full(g.q, g.k, g.v, do, causal)
    lse64 = lse.astype(np.float64)
    for h in range(H):
        bounds = bwd_rounding_bound(g.q[0, h], g.k[0, h], g.v[0, h], do[0, h], o[0, h],
                                    lse64[0, h], causal, scale)
        for name, x, r, e, b in zip(("dq", "dk", "dv"), got, given, exact, bounds):
            x, r, e = x[0, h], r[0, h], e[0, h]
            allowed = b + half_ulp_bf16(np.abs(r) + b) + 1e-7
            err = np.abs(x - r)
            announce("   head", h, name, "worst ratio to the rounding bound",
                     float((err / allowed).max()), "rel_max", float(err.max() / np.abs(r).max()))
            assert np.all(np.isfinite(x)) and np.all(err <= allowed), (name, h)
            # exact gradient: plus the oracle's own distance between the two
            # references (the bf16 rounding of the O that forms D)
            assert np.all(np.abs(x - e) <= allowed + np.abs(r - e)), (name, h, "exact")


@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_several_heads(lib, d):
    # B*H = 24 heads: a multiple of 8 (one run of heads per accelerator die)
    for causal in (False, True):
        check_bwd(lib, 2, 12, 640, d, causal, 9500 + d)


@pytest.mark.parametrize("causal", [False, True])
def test_mid_config(lib, causal):
    check_bwd(lib, 4, 16, 2048, 128, causal, fa_inputs.SEEDS["mid"])


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


def test_grid_order_bitwise(lib):
    """Both backward kernels with their workgroups in reverse order (and
    without the per-XCD head grouping; FA_DEBUG=1) give the default order's
    gradients bit for bit: every gradient row has one writer and no result
    depends on which workgroups run first."""
    import os
    import torch
    from tests.gpu_util import to_device
    for causal in (False, True):
        announce("bwd grid order 2 8 1000 128", "causal" if causal else "noncausal")
        g = fa_inputs.make_qkv(2, 8, 1000, 128, 80 + causal)
        do_bits, _ = fa_inputs.make_grad(2, 8, 1000, 128, 82 + causal)
        q, k, v = to_device(g)
        do = fa_inputs.to_torch_bf16(do_bits, "cuda")
        o, lse = lib.fwd(q, k, v, causal=causal)
        a = lib.bwd(q, k, v, o, lse, do, causal=causal)
        os.environ["FA_DEBUG"] = "1"
        try:
            b = lib.bwd(q, k, v, o, lse, do, causal=causal)
        finally:
            del os.environ["FA_DEBUG"]
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_scale_argument(lib):
    # a scale other than 1/sqrt(d) reaches the backward
    check_bwd(lib, 1, 2, 200, 64, True, 79, scale=0.3)


@pytest.mark.parametrize("d", [64, 96, 128, 256])
def test_head_dim_sweep_size_sampled_heads(lib, d):
    """The bench's head-dim sweep workload (B=2 H=16 N=8192 causal) in the
    launch configuration the bench times; the oracle's forward covers every
    head, its backward two whole (batch, head) slices chosen by seed."""
    B, H, N = 2, 16, 8192
    seed = fa_inputs.SEEDS["dim_sweep_base"] + (64, 96, 128, 256).index(d)
    rng = np.random.default_rng(seed)
    heads = [divmod(int(bh), H) for bh in rng.choice(B * H, size=2, replace=False)]
    check_bwd(lib, B, H, N, d, True, seed, heads=heads)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_closed_forms_at_mid_size(lib, causal):
    """Every K row of a head equal: all scores of a query are equal, so
    P_ij = 1/n_i over the n_i keys it attends (N, or i+1 causal). At the full
    mid size, without the oracle: the forward's O and LSE are given in closed
    form, and (D_i = dO_i . O_i with the bf16 O the backward is given, as the
    backward defines it):
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
    qf, vf = g.q, g.v
    scale = 1.0 / np.sqrt(d)
    n = np.arange(1, N + 1) if causal else np.full(N, N)
    # the forward's output in closed form: O_i = mean of the attended V rows,
    # LSE_i = scale q_i . k + ln n_i; O rounded to bf16, LSE to float32
    kf = fa_inputs.bf16_bits_to_f64(krow)
    if causal:
        o_exact = np.cumsum(vf, axis=2) / n[None, None, :, None]
    else:
        o_exact = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
    o_bits = fa_inputs.bf16_bits(o_exact.astype(np.float32))
    lse = (scale * (qf * kf).sum(axis=3) + np.log(n)[None, None, :]).astype(np.float32)
    o = fa_inputs.to_torch_bf16(o_bits, "cuda")
    dq, dk, dv = lib.bwd(q, k, v, o, torch.from_numpy(lse).cuda(), dot, causal=causal)
    torch.cuda.synchronize()
    f64 = lambda t: fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(t))
    dq, dk, dv = f64(dq), f64(dk), f64(dv)
    o64 = fa_inputs.bf16_bits_to_f64(o_bits)
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
