"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the float64
oracle for queries and keys of different lengths (decode shapes, few heads,
ragged lengths, both masks, several split counts), under the forward's bf16
gate. Every case prints its name, shape and seed before it touches the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import fa_inputs
from oracle import attention_kv
from tests.gpu_util import LSE_MAX_ABS, bf16_gate, ramp_amp

pytestmark = pytest.mark.gpu


def announce(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def make(B, H, Nq, Nk, d, seed, ramp=False):
    if ramp:
        # scores growing along the key axis, about 8.5 log2 units every 256 keys
        amp = ramp_amp(d, 8.5 * Nk / 256)
        g = fa_inputs.make_qkv_ramp(B, H, Nk, d, seed, 4.0, amp)
        gq = fa_inputs.make_qkv_ramp(B, H, Nq, d, seed + 50000, 4.0, amp)
    else:
        g = fa_inputs.make_qkv(B, H, Nk, d, seed)           # K, V (and an unused Q)
        gq = fa_inputs.make_qkv(B, H, Nq, d, seed + 50000)  # Q
    return gq.q_bits, g.k_bits, g.v_bits


def run(fa, qb, kb, vb, causal, splits, scale=None):
    import torch
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (qb, kb, vb))
    o, lse = fa.fwd_splitkv(q, k, v, causal=causal, num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    return (fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o)),
            lse.cpu().numpy().astype(np.float64))


def check(fa, B, H, Nq, Nk, d, causal, splits, seed, scale=None, ramp=False):
    announce("splitkv", B, H, Nq, Nk, d, "causal" if causal else "noncausal", "splits", splits,
             "(used", fa.splitkv_splits(B, H, Nq, Nk, splits, causal), ") seed", seed,
             "ramp" if ramp else "")
    qb, kb, vb = make(B, H, Nq, Nk, d, seed, ramp)
    o, lse = run(fa, qb, kb, vb, causal, splits, scale)
    o_ref, lse_ref = attention_kv(*(fa_inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb)), causal,
                                  scale)
    ok, st = bf16_gate(o, o_ref)
    lse_err = float(np.abs(lse - lse_ref).max())
    announce("  stats", st, "lse_max_abs", lse_err)
    assert ok, st
    assert lse_err <= LSE_MAX_ABS


CASES = [
    # (B, H, Nq, Nk, d, causal, splits)
    (2, 4, 1, 1000, 128, False, 0),     # decode
    (2, 4, 1, 1000, 128, True, 0),
    (1, 3, 1, 4097, 64, True, 5),
    (2, 2, 7, 300, 96, True, 3),
    (1, 2, 32, 2048, 128, True, 0),     # one wave per workgroup, full wave
    (1, 2, 33, 2048, 128, False, 0),    # four waves per workgroup
    (1, 2, 200, 200, 128, True, 3),     # Nq == Nk: fa_fwd's mask
    (1, 2, 257, 1000, 64, True, 4),
    (2, 2, 1, 64, 128, False, 1),       # one tile
    (1, 1, 1, 1, 64, True, 0),          # one key
    (1, 2, 5, 130, 96, False, 64),      # more splits requested than tiles
    (1, 2, 100, 100, 64, False, 0),
    # 8 or more splits (one workgroup per row in the merge): early causal rows
    # have whole splits without a visible key; 13 splits over 8 merge groups
    (1, 2, 1664, 1664, 64, True, 13),
    (2, 2, 3, 2000, 96, False, 9),
    # causal with several query tiles and B*H that neither divides 8 nor is
    # divided by it (longest-first item order over the heads), with empty
    # workgroups past the diagonal
    (1, 3, 300, 300, 64, True, 4),
    (3, 1, 500, 700, 128, True, 6),
    (1, 5, 1100, 1100, 96, True, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_splitkv_parity(lib, case):
    B, H, Nq, Nk, d, causal, splits = case
    check(lib, B, H, Nq, Nk, d, causal, splits, 11000 + Nq + Nk + d)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_mid_size(lib, causal):
    # decode: one new query per (b, h) against a 16k-token cache
    check(lib, 4, 16, 1, 16384, 128, causal, 0, 12001)


def test_scale_and_split_counts_agree(lib):
    qb, kb, vb = make(1, 2, 64, 3000, 128, 12002)
    announce("splitkv split counts 1 2 7 47, scale 0.2")
    outs = [run(lib, qb, kb, vb, True, s, 0.2) for s in (1, 2, 7, 47)]
    o_ref, lse_ref = attention_kv(*(fa_inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb)), True, 0.2)
    for o, lse in outs:
        ok, st = bf16_gate(o, o_ref)
        assert ok, st
        assert float(np.abs(lse - lse_ref).max()) <= LSE_MAX_ABS


def test_matches_fa_fwd_when_lengths_are_equal(lib):
    import torch
    announce("splitkv vs fa_fwd 2 4 640 640 128 causal")
    g = fa_inputs.make_qkv(2, 4, 640, 128, 12003)
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (g.q_bits, g.k_bits, g.v_bits))
    o1, l1 = lib.fwd(q, k, v, causal=True)
    o2, l2 = lib.fwd_splitkv(q, k, v, causal=True, num_splits=4)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 2e-2
    assert float((l1 - l2).abs().max()) <= 1e-3


def test_optional_lse(lib):
    """Without an LSE output the merge skips its store and O is bit for bit
    the same."""
    import torch
    announce("splitkv without lse 2 3 5 700 64 causal")
    qb, kb, vb = make(2, 3, 5, 700, 64, 12004)
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (qb, kb, vb))
    o1, l1 = lib.fwd_splitkv(q, k, v, causal=True, num_splits=3)
    o2, l2 = lib.fwd_splitkv(q, k, v, causal=True, num_splits=3, return_lse=False)
    torch.cuda.synchronize()
    assert l2 is None
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_deterministic(lib):
    """Repeated calls give bitwise identical outputs (fixed split boundaries
    and merge order)."""
    import torch
    announce("splitkv determinism 2 4 16 5000 128 causal")
    qb, kb, vb = make(2, 4, 16, 5000, 128, 12005)
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (qb, kb, vb))
    runs = [lib.fwd_splitkv(q, k, v, causal=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(lse, runs[0][1])


@pytest.mark.parametrize("case", [(2, 4, 1, 4100, 128, True, 0), (1, 3, 257, 1000, 96, True, 4),
                                  (2, 2, 7, 300, 64, False, 3)],
                         ids=lambda c: "-".join(map(str, c)))
def test_grid_order_and_lds_poison_bitwise(lib, case):
    """The split kernel with its workgroups in reverse order and its LDS ring
    filled with NaN bytes before the first copy (FA_DEBUG=3) gives the
    default run's output bit for bit: decode (one wave per workgroup, 32-key
    tiles) and queries of another length than the keys (four waves, 64-key
    tiles)."""
    import os
    import torch
    B, H, Nq, Nk, d, causal, splits = case
    announce("splitkv grid order / lds poison", *case)
    qb, kb, vb = make(B, H, Nq, Nk, d, 12100 + Nq)
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (qb, kb, vb))
    a = lib.fwd_splitkv(q, k, v, causal=causal, num_splits=splits)
    os.environ["FA_DEBUG"] = "3"
    try:
        b = lib.fwd_splitkv(q, k, v, causal=causal, num_splits=splits)
    finally:
        del os.environ["FA_DEBUG"]
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


RAMP_CASES = [
    # (B, H, Nq, Nk, d, causal, splits)
    (2, 2, 1, 4100, 128, False, 0),     # decode
    (1, 2, 16, 4100, 96, True, 0),
    (1, 2, 1500, 1500, 128, True, 4),   # Nq == Nk: the forward kernel's split mode
    (1, 2, 1500, 1500, 64, False, 3),
]


@pytest.mark.parametrize("case", RAMP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_splitkv_running_max_moves(lib, case):
    """Scores growing along the key axis (fa_inputs.make_qkv_ramp): inside a
    split the running maximum moves several times, and the splits'
    log-sum-exps differ by tens of units, so the merge weights span many
    orders of magnitude."""
    B, H, Nq, Nk, d, causal, splits = case
    check(lib, B, H, Nq, Nk, d, causal, splits, 22000 + Nq + d, ramp=True)
