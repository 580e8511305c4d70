"""GPU test of the allocation-free split-KV entry point
(fa_fwd_splitkv_noalloc): through the C ABI, two calls in a row (the second
with a smaller input, so it runs on what the first left in the shared
scratch array) must equal fa_fwd_splitkv on the same inputs bit for bit (the
same kernels and split count; only the scratch differs), and both meet the
forward's bf16 gate against the float64 oracle. Every case prints its shape
before it touches the GPU.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import fa_inputs
from oracle import attention_kv
from tests.gpu_util import LSE_MAX_ABS, bf16_gate

pytestmark = pytest.mark.gpu


def announce(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def inputs(B, H, Nq, Nk, d, seed):
    g = fa_inputs.make_qkv(B, H, Nk, d, seed)
    gq = fa_inputs.make_qkv(B, H, Nq, d, seed + 50000)
    return gq.q_bits, g.k_bits, g.v_bits


def call_c(lib, entry, q, k, v, o, lse, causal, splits):
    """One call of a split-KV C entry point with raw device pointers on the
    current stream."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = getattr(lib.lib, entry)(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), B, H, Nq, Nk, d, int(causal),
        float(1.0 / np.sqrt(d)), splits, stream)
    assert st == lib.FA_OK, (entry, st, lib.status_string(st))


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_pool_entry_two_calls(lib, causal):
    import torch
    # a larger decode call (64 splits), then smaller ones with fewer splits:
    # self-attention (the forward kernel's split mode) and Nq != Nk
    shapes = [(1, 16, 16, 16384, 128, 0), (1, 2, 640, 640, 128, 4), (2, 3, 5, 1000, 64, 3)]
    for i, (B, H, Nq, Nk, d, splits) in enumerate(shapes):
        used = lib.splitkv_splits(B, H, Nq, Nk, splits, causal)
        need = used * B * H * Nq * (d + 1) * 4
        announce("noalloc splitkv call", i, B, H, Nq, Nk, d, "causal" if causal else "noncausal",
                 "splits", used, "scratch bytes", need)
        assert need <= lib.NOALLOC_SCRATCH_BYTES
        qb, kb, vb = inputs(B, H, Nq, Nk, d, 13100 + i)
        q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (qb, kb, vb))
        o1 = torch.empty_like(q)
        l1 = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
        o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
        call_c(lib, "fa_fwd_splitkv_noalloc", q, k, v, o1, l1, causal, splits)
        call_c(lib, "fa_fwd_splitkv", q, k, v, o2, l2, causal, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        o64 = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o1))
        o_ref, lse_ref = attention_kv(*(fa_inputs.bf16_bits_to_f64(x) for x in (qb, kb, vb)),
                                      causal)
        ok, st = bf16_gate(o64, o_ref)
        lse_err = float(np.abs(l1.cpu().numpy() - lse_ref).max())
        announce("  stats", st, "lse_max_abs", lse_err)
        assert ok, st
        assert lse_err <= LSE_MAX_ABS


def test_noalloc_python_binding_and_limit(lib):
    """The binding's wrapper gives the same result; a call needing more than
    the fixed scratch is refused before any launch."""
    import torch
    B, H, Nq, Nk, d = 4, 16, 1, 16384, 128
    announce("noalloc binding", B, H, Nq, Nk, d)
    qb, kb, vb = inputs(B, H, Nq, Nk, d, 13200)
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (qb, kb, vb))
    o1, l1 = lib.fwd_splitkv_noalloc(q, k, v, causal=True)
    o2, l2 = lib.fwd_splitkv(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    big_q = torch.zeros((16, 16, 2048, 128), dtype=torch.bfloat16, device="cuda")
    big_kv = torch.zeros((16, 16, 8192, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.FAError) as err:
        lib.fwd_splitkv_noalloc(big_q, big_kv, big_kv, num_splits=4)
    assert err.value.status == lib.FA_ERR_SCRATCH_LIMIT
