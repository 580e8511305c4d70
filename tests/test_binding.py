"""The Python binding refuses caller-provided outputs and side inputs that do
not match what the kernels read or write (shape, dtype, contiguity, device),
and outputs that share memory with an input or another output, before any
launch. Small tensors; nothing is computed."""
from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu


def test_wrong_buffers_are_refused(lib):
    import torch
    dev = "cuda"
    B, H, N, d = 1, 2, 130, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    bad_o = [torch.zeros(B, H, N - 1, d, dtype=torch.bfloat16, device=dev),      # shape
             torch.zeros(B, H, N, d, dtype=torch.float16, device=dev),           # dtype
             torch.zeros(B, H, d, N, dtype=torch.bfloat16, device=dev).transpose(2, 3),  # layout
             torch.zeros(B, H, N, d, dtype=torch.bfloat16)]                      # host memory
    for o in bad_o:
        with pytest.raises(ValueError):
            lib.fwd(q, k, v, out=o)
        with pytest.raises(ValueError):
            lib.fwd_splitkv(q, k, v, out=o)
    for lse in (torch.zeros(B, H, N - 1, device=dev), torch.zeros(B, H, N, device=dev,
                                                                 dtype=torch.float64)):
        with pytest.raises(ValueError):
            lib.fwd(q, k, v, lse=lse)
        with pytest.raises(ValueError):
            lib.fwd_splitkv(q, k, v, lse=lse)

    o, lse = lib.fwd(q, k, v)
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError):
            lib.bwd(q, k, v, o, lse, o, **{name: bad_o[0]})

    # outputs that share memory with an input or with another output
    for t in (q, k, v):
        with pytest.raises(ValueError, match="overlaps"):
            lib.fwd(q, k, v, out=t)
        with pytest.raises(ValueError, match="overlaps"):
            lib.fwd_splitkv(q, k, v, out=t)
    out = torch.empty_like(q)
    lse_in_out = out.view(torch.float32).view(-1)[: B * H * N].view(B, H, N)
    with pytest.raises(ValueError, match="overlaps"):
        lib.fwd(q, k, v, out=out, lse=lse_in_out)
    buf = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="overlaps"):
        lib.bwd(q, k, v, o, lse, o, dq=o)
    with pytest.raises(ValueError, match="overlaps"):
        lib.bwd(q, k, v, o, lse, o, dk=buf, dv=buf)

    nblk = (N + 127) // 128
    with pytest.raises(ValueError):
        lib.quant_fp8(q, scales=torch.zeros(B, H, nblk - 1, device=dev))
    with pytest.raises(ValueError):
        lib.quant_fp8(q, out=torch.zeros(B, H, N, d, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        lib.quant_fp8(q, signs=torch.ones(d + 1, device=dev))
    q8, sq = lib.quant_fp8(q)
    k8, sk = lib.quant_fp8(k)
    v8, sv = lib.quant_fp8(v)
    with pytest.raises(ValueError):
        lib.fwd_fp8(q8, k8, v8, sq, sk[:, :, :0], sv)
    with pytest.raises(ValueError):
        lib.fwd_fp8(q8, k8, v8, sq, sk, sv.to(torch.float16))
    with pytest.raises(ValueError):
        lib.fwd_fp8(q8, k8, v8, sq, sk, sv, out=bad_o[0])
    torch.cuda.synchronize()


def test_side_streams_and_scratch_pool(lib):
    """Calls enqueue on the caller's current stream: the same inputs run on
    two side streams at once (FP8 end to end, backward and split-KV, which
    take stream-ordered scratch from the library's pool) give the bits of a
    run on the default stream."""
    import torch
    import fa_inputs
    g = fa_inputs.make_qkv(2, 4, 1000, 128, 760)
    q, k, v = (fa_inputs.to_torch_bf16(b, "cuda") for b in (g.q_bits, g.k_bits, g.v_bits))
    do = torch.randn_like(q)

    def run():
        o8, l8 = lib.fwd(q, k, v, causal=True, dtype=lib.FA_FP8_E4M3)
        o, lse = lib.fwd(q, k, v, causal=True)
        grads = lib.bwd(q, k, v, o, lse, do, causal=True)
        os_, ls = lib.fwd_splitkv(q[:, :, -7:].contiguous(), k, v, causal=True)
        return (o8, l8, o, lse, *grads, os_, ls)

    ref = run()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append(run())
    torch.cuda.synchronize()
    for res in outs:
        for a, b in zip(res, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_graph_capture_bf16_forward(lib):
    """The bf16 forward (no scratch, one kernel launch) can be captured in a
    HIP graph through torch's graph API: every replay, with new inputs copied
    in and eager work and synchronisation between replays, equals an eager
    call on the same inputs bit for bit."""
    import torch
    import fa_inputs
    B, H, N, d = 2, 8, 640, 128
    q = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    k, v = torch.empty_like(q), torch.empty_like(q)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")

    def load(seed):
        g = fa_inputs.make_qkv(B, H, N, d, seed)
        for dst, bits in ((q, g.q_bits), (k, g.k_bits), (v, g.v_bits)):
            dst.copy_(fa_inputs.to_torch_bf16(bits, "cuda"))

    load(770)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lib.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.fwd(q, k, v, causal=True, out=o, lse=lse)
    for seed in (771, 772, 773):
        load(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_graph, lse_graph = o.clone(), lse.clone()
        o_eager, lse_eager = lib.fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o_graph.view(torch.int16), o_eager.view(torch.int16))
        assert torch.equal(lse_graph, lse_eager)


@pytest.mark.parametrize("shape", [(4, 16, 1, 4096, 128, True, 0), (1, 2, 1536, 1536, 64, True, 3)],
                         ids=["decode", "self-attention-split"])
def test_graph_capture_splitkv_noalloc(lib, shape):
    """The allocation-free split-KV entry (its scratch a fixed device array:
    nothing is allocated or cleared inside the call) captured in a HIP graph:
    every replay, with new inputs copied in and eager work between replays,
    equals an eager fa_fwd_splitkv call bit for bit. Decode runs the split
    kernel and the merge; Nq = Nk runs the forward kernel's split mode and
    the merge."""
    import torch
    import fa_inputs
    B, H, Nq, Nk, d, causal, splits = shape
    q = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(B, H, Nk, d, dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, dtype=torch.float32, device="cuda")

    def load(seed):
        gk = fa_inputs.make_qkv(B, H, Nk, d, seed)
        gq = fa_inputs.make_qkv(B, H, Nq, d, seed + 50000)
        for dst, bits in ((q, gq.q_bits), (k, gk.k_bits), (v, gk.v_bits)):
            dst.copy_(fa_inputs.to_torch_bf16(bits, "cuda"))

    def call():
        lib.fwd_splitkv_noalloc(q, k, v, causal=causal, num_splits=splits, out=o, lse=lse)

    load(780)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for seed in (781, 782, 783):
        load(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_graph, lse_graph = o.clone(), lse.clone()
        o_eager, lse_eager = lib.fwd_splitkv(q, k, v, causal=causal, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o_graph.view(torch.int16), o_eager.view(torch.int16))
        assert torch.equal(lse_graph, lse_eager)
