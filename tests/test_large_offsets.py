"""GPU parity at the largest tensors the tests allocate: every tensor holds
more than 2^31 elements (B*H = 33*4096 heads of N = 128 rows, d = 128; about
4.4 GB in bf16), so heads from index 2^17 on start past 2^31 elements and past
2^32 bytes. This exercises the 64-bit head offsets of every kernel: the bf16
forward (both masks), the FP8 end-to-end path (its quantisation pass and the
e4m3 kernel), the backward and the split-KV forward. One 128-row tile per
head keeps the work to milliseconds.

The inputs are drawn on the device by a seeded generator (fa_inputs); the
heads checked (the first two, the three around the 2^31-element boundary, the
last one and three at random) are copied back and compared with the oracle
under the gates of the other parity tests. Every case prints its name before
it touches the GPU.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import fa_inputs
from oracle import attention, attention_backward, attention_kv, fp8
from tests.gpu_util import FP8_REL_RMSE, LSE_MAX_ABS, bf16_gate, bwd_gate
from tests.test_fp8 import splitmix64_signs

pytestmark = pytest.mark.gpu

B, H, N, D = 33, 4096, 128, 128
BOUNDARY = (1 << 31) // (N * D)       # first head starting at element 2^31


def announce(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def checked_heads():
    rng = np.random.default_rng(fa_inputs.SEEDS["large"])
    flat = [0, 1, BOUNDARY - 1, BOUNDARY, BOUNDARY + 1, B * H - 1]
    flat += [int(x) for x in rng.integers(0, B * H, 3)]
    return [divmod(f, H) for f in flat]


HEADS = checked_heads()


def heads_f64(t):
    """The checked heads of a bf16 device tensor [B, H, n, d] -> float64
    [len(HEADS), n, d]."""
    return np.stack([fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(t[b, h]))
                     for b, h in HEADS])


@pytest.fixture(scope="module")
def big():
    import torch
    assert B * H * N * D > (1 << 31)
    announce("large tensors: drawing Q, K, V", B, H, N, D)
    seed = fa_inputs.SEEDS["large"]
    q, k, v = (fa_inputs.device_normal_bf16((B, H, N, D), seed + i) for i in range(3))
    torch.cuda.synchronize()
    host = {name: heads_f64(t) for name, t in (("q", q), ("k", k), ("v", v))}
    yield q, k, v, host
    del q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bf16_past_2_31_elements(lib, big, causal):
    import torch
    q, k, v, host = big
    announce("large fwd bf16", B, H, N, D, "causal" if causal else "noncausal")
    o, lse = lib.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    got = heads_f64(o)
    got_lse = np.stack([lse[b, h].cpu().numpy().astype(np.float64) for b, h in HEADS])
    del o, lse
    ref, ref_lse = attention(host["q"][None], host["k"][None], host["v"][None], causal)
    ok, st = bf16_gate(got, ref[0])
    lse_err = float(np.abs(got_lse - ref_lse[0]).max())
    announce("  stats", st, "lse_max_abs", lse_err)
    assert ok, st
    assert lse_err <= LSE_MAX_ABS


def test_fwd_fp8_end_to_end_past_2_31_elements(lib, big):
    import torch
    q, k, v, host = big
    announce("large fwd fp8 end to end", B, H, N, D)
    o, _ = lib.fwd(q, k, v, causal=False, dtype=lib.FA_FP8_E4M3)
    torch.cuda.synchronize()
    got = heads_f64(o)
    del o
    # The end-to-end path rotates Q and K by the library's fixed signs; the
    # oracle's emulator of the method on the checked heads is printed beside
    # the error against exact attention (the gate: a head read from a wrong
    # offset would be far off).
    signs = splitmix64_signs(D)
    qc, sq = fp8.quantize(host["q"][None], signs=signs)
    kc, sk = fp8.quantize(host["k"][None], signs=signs)
    vc, sv = fp8.quantize(host["v"][None])
    emul = fp8.fp8_attention_emulate(qc, kc, vc, sq, sk, sv, False, 1.0 / math.sqrt(D))[0]
    ref, _ = attention(host["q"][None], host["k"][None], host["v"][None], False)

    def rel(a, r):
        return float(np.linalg.norm(a - r) / np.linalg.norm(r))

    e_ref = rel(got, ref[0])
    announce("  rel_rmse vs exact", e_ref, "(emulator's prediction", rel(emul, ref[0]), ")")
    assert np.all(np.isfinite(got))
    assert e_ref <= 1.5 * FP8_REL_RMSE


def test_bwd_past_2_31_elements(lib, big):
    """The backward is handed the oracle's forward output (O in bf16, LSE in
    float32) on the checked heads; the other heads get the library's forward
    output, which only fills them (their gradients are not checked)."""
    import torch
    q, k, v, host = big
    announce("large bwd", B, H, N, D, "causal")
    do = fa_inputs.device_normal_bf16((B, H, N, D), fa_inputs.SEEDS["large"] + 3)
    o, lse = lib.fwd(q, k, v, causal=True)
    ref_o, ref_lse = attention(host["q"][None], host["k"][None], host["v"][None], True)
    o_bits = fa_inputs.bf16_bits(ref_o[0].astype(np.float32))
    for i, (b, h) in enumerate(HEADS):
        o[b, h] = fa_inputs.to_torch_bf16(o_bits[i], "cuda")
        lse[b, h] = torch.from_numpy(ref_lse[0, i].astype(np.float32)).cuda()
    dq, dk, dv = lib.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    got = [heads_f64(t) for t in (dq, dk, dv)]
    do_h = heads_f64(do)
    del do, o, lse, dq, dk, dv
    o_given = fa_inputs.bf16_bits_to_f64(o_bits)
    for kind, oo in (("given-O", o_given[None]), ("exact", None)):
        ref = attention_backward(host["q"][None], host["k"][None], host["v"][None], do_h[None],
                                 True, o=oo)
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            ok, st = bwd_gate(x, r[0])
            announce("  ", kind, name, st)
            assert ok, (kind, name, st)


@pytest.mark.parametrize("Nq,causal,splits", [(1, False, 0), (33, True, 0), (N, True, 2)])
def test_splitkv_past_2_31_elements(lib, big, Nq, causal, splits):
    """Decode, Nq != Nk, and Nq = Nk with two splits (the forward kernel's
    split mode; its float32 partials span 17.8 GB)."""
    import torch
    _, k, v, host = big
    announce("large splitkv", B, H, Nq, N, D, "causal" if causal else "noncausal",
             "splits", splits)
    q = fa_inputs.device_normal_bf16((B, H, Nq, D), fa_inputs.SEEDS["large"] + 4 + Nq)
    o, lse = lib.fwd_splitkv(q, k, v, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    got, q_h = heads_f64(o), heads_f64(q)
    got_lse = np.stack([lse[b, h].cpu().numpy().astype(np.float64) for b, h in HEADS])
    del q, o, lse
    ref, ref_lse = attention_kv(q_h[None], host["k"][None], host["v"][None], causal)
    ok, st = bf16_gate(got, ref[0])
    lse_err = float(np.abs(got_lse - ref_lse[0]).max())
    announce("  stats", st, "lse_max_abs", lse_err)
    assert ok, st
    assert lse_err <= LSE_MAX_ABS


def test_decode_grid_past_2_24_workgroups(lib):
    """Decode over B*H = 2^24 + 1024 heads (one query, two keys each, d = 64):
    the split-KV kernel runs one single-wave workgroup per head, a grid past
    the 2^24 workgroups below which the other kernels carry debug flags in
    their workgroup-count argument; the heads around 2^24, the first and last
    and three at random are checked against the oracle."""
    import torch
    Bd, Hd, Nk, d = 16385, 1024, 2, 64
    nheads = Bd * Hd
    assert nheads > (1 << 24) and lib.splitkv_splits(Bd, Hd, 1, Nk) == 1
    announce("decode grid past 2^24 workgroups", Bd, Hd, 1, Nk, d)
    seed = fa_inputs.SEEDS["large"] + 10
    q = fa_inputs.device_normal_bf16((Bd, Hd, 1, d), seed)
    k = fa_inputs.device_normal_bf16((Bd, Hd, Nk, d), seed + 1)
    v = fa_inputs.device_normal_bf16((Bd, Hd, Nk, d), seed + 2)
    o, lse = lib.fwd_splitkv(q, k, v)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    flat = [0, 1, (1 << 24) - 1, 1 << 24, (1 << 24) + 1, nheads - 1]
    flat += [int(x) for x in rng.integers(0, nheads, 3)]
    picks = [divmod(f, Hd) for f in flat]

    def rows(t):
        return np.stack([fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(t[b, h]))
                         for b, h in picks])

    got, qh, kh, vh = rows(o), rows(q), rows(k), rows(v)
    got_lse = np.stack([lse[b, h].cpu().numpy().astype(np.float64) for b, h in picks])
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    ref, ref_lse = attention_kv(qh[None], kh[None], vh[None], False)
    ok, st = bf16_gate(got, ref[0])
    lse_err = float(np.abs(got_lse - ref_lse[0]).max())
    announce("  stats", st, "lse_max_abs", lse_err)
    assert ok, st
    assert lse_err <= LSE_MAX_ABS
