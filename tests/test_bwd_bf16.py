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
