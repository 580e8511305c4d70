"""The Python binding refuses caller-provided outputs and side inputs that do
not match what the kernels read or write (shape, dtype, contiguity, device),
before any launch. Small tensors; nothing is computed."""
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
