"""Python binding of libfa.so, the MI355X FlashAttention library (forward and
backward passes).

Argument marshalling only: tensors are checked, outputs are allocated with
torch on the caller's device, and the C entry points of include/fa.h are called
on torch's current stream. Every step of the attention path runs in the
library's HIP kernels; there is no fallback. Importing this package fails
loudly when libfa.so has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_BF16 = 0
FA_FP8_E4M3 = 1
FP8_BLOCK = 128

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_MISALIGNED = -3
FA_ERR_HIP = -4
FA_ERR_TOO_LARGE = -5
FA_ERR_SCRATCH_LIMIT = -6
NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ("fa_fwd", "fa_quant_fp8", "fa_fwd_fp8", "fa_bwd", "fa_fwd_splitkv",
           "fa_fwd_splitkv_noalloc", "fa_splitkv_splits", "fa_status_string", "fa_version")


class FAError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


def _load():
    # torch brings its own HIP runtime (soname libamdhip64.so.7, requested as
    # libamdhip64.so). Importing it first makes libfa.so bind to that same
    # runtime; loaded the other way round the process would hold two HIP
    # runtimes and the library's launches would not see torch's device memory.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with "
            "`python -m exact_attention_14_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fp = ctypes.c_void_p
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_quant_fp8.argtypes = [vp, vp, fp, i, i, i, i, i, fp, vp]
    lib.fa_quant_fp8.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, fp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_bwd.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, fp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_splitkv_splits.argtypes = [i, i, i, i, i, i]
    lib.fa_splitkv_splits.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.fa_status_string(int(status)).decode()


def version() -> int:
    return int(lib.fa_version())


def _check(status: int, fn: str):
    if status != FA_OK:
        raise FAError(status, fn)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _launch(fn, name, device, *args):
    """Calls a C entry point with the tensors' device current (the library
    launches on the calling thread's current device) and that device's
    current torch stream as the last argument; raises FAError on failure."""
    import torch
    with torch.cuda.device(device):
        _check(fn(*args, _stream(device)), name)


def _check_buf(t, name, shape, dtype, device):
    """A caller-provided output or side input must match exactly what the
    kernels read or write: contiguous, this dtype, shape and device."""
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _no_overlap(outputs, inputs):
    """Outputs must not share memory with the inputs (nor with each other):
    the kernels read the inputs while other workgroups write the outputs."""
    def span(t):
        return t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()
    outs = [(n, t) for n, t in outputs if t is not None]
    ins = [(n, t) for n, t in inputs if t is not None]
    for i, (no, to) in enumerate(outs):
        a0, a1 = span(to)
        for ni, ti in ins + outs[i + 1:]:
            b0, b1 = span(ti)
            if a0 < b1 and b0 < a1:
                raise ValueError(f"{no} overlaps {ni} in memory")


def _check_qkv(q, k, v, dtype):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v are on different devices")
    return torch


def fwd(q, k, v, causal: bool = False, scale: float | None = None, dtype: int = FA_BF16,
        out=None, lse=None, return_lse: bool = True):
    """Attention forward on bf16 [B, H, N, d] tensors; returns (o, lse).

    dtype=FA_BF16 runs the bf16 path; dtype=FA_FP8_E4M3 the end-to-end FP8
    path (rotation, block quantisation and the e4m3 kernel inside the call).
    """
    torch = _check_qkv(q, k, v, torch_bf16())
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_buf(out, "out", q.shape, torch.bfloat16, q.device)
    _check_buf(lse, "lse", (B, H, N), torch.float32, q.device)
    _no_overlap((("out", out), ("lse", lse)), (("q", q), ("k", k), ("v", v)))
    o = torch.empty_like(q) if out is None else out
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _launch(lib.fa_fwd, "fa_fwd", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N,
            d, int(bool(causal)), float(scale), int(dtype))
    return o, lse


def quant_fp8(x, per_tensor: bool = False, signs=None, out=None, scales=None):
    """Block-quantise a bf16 [B, H, N, d] tensor to e4m3fn; returns (x8, scales)."""
    import torch
    if x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [B, H, N, d] tensor")
    if x.device.type != "cuda":
        raise ValueError("x must be on a GPU")
    B, H, N, d = x.shape
    nblk = (N + FP8_BLOCK - 1) // FP8_BLOCK
    _check_buf(out, "out", x.shape, torch.float8_e4m3fn, x.device)
    _check_buf(scales, "scales", (B, H, nblk), torch.float32, x.device)
    _check_buf(signs, "signs", (d,), torch.float32, x.device)
    _no_overlap((("out", out), ("scales", scales)), (("x", x), ("signs", signs)))
    x8 = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device) if out is None else out
    sc = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device) if scales is None else scales
    _launch(lib.fa_quant_fp8, "fa_quant_fp8", x.device, _ptr(x), _ptr(x8), _ptr(sc), B, H, N, d,
            int(bool(per_tensor)), _ptr(signs))
    return x8, sc


def fwd_fp8(q8, k8, v8, sq, sk, sv, causal: bool = False, scale: float | None = None,
            out=None, lse=None, return_lse: bool = True):
    """Attention forward on e4m3fn operands with block scales; returns (o bf16, lse)."""
    torch = _check_qkv(q8, k8, v8, _fp8())
    B, H, N, d = q8.shape
    nblk = (N + FP8_BLOCK - 1) // FP8_BLOCK
    for name, t in (("sq", sq), ("sk", sk), ("sv", sv)):
        if t is None:
            raise ValueError(f"{name} is required")
        _check_buf(t, name, (B, H, nblk), torch.float32, q8.device)
    _check_buf(out, "out", q8.shape, torch.bfloat16, q8.device)
    _check_buf(lse, "lse", (B, H, N), torch.float32, q8.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _no_overlap((("out", out), ("lse", lse)),
                (("q8", q8), ("k8", k8), ("v8", v8), ("sq", sq), ("sk", sk), ("sv", sv)))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _launch(lib.fa_fwd_fp8, "fa_fwd_fp8", q8.device, _ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq),
            _ptr(sk), _ptr(sv), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), float(scale))
    return o, lse


def fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0,
                out=None, lse=None, return_lse: bool = True):
    """Split-KV forward: q bf16 [B, H, Nq, d] against k, v bf16 [B, H, Nk, d];
    returns (o, lse). Causal places the queries at the last Nq positions."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [B, H, N, d] tensor")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError(f"{name} must be on q's GPU")
    B, H, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError(f"k, v must be [B, H, Nk, d] matching q: {tuple(k.shape)} {tuple(v.shape)}")
    Nk = k.shape[2]
    _check_buf(out, "out", q.shape, torch.bfloat16, q.device)
    _check_buf(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _no_overlap((("out", out), ("lse", lse)), (("q", q), ("k", k), ("v", v)))
    o = torch.empty_like(q) if out is None else out
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _launch(lib.fa_fwd_splitkv, "fa_fwd_splitkv", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
            _ptr(lse), B, H, Nq, Nk, d, int(bool(causal)), float(scale), int(num_splits))
    return o, lse


def fwd_splitkv_noalloc(q, k, v, causal: bool = False, scale: float | None = None,
                        num_splits: int = 0, out=None, lse=None, return_lse: bool = True):
    """fwd_splitkv through the allocation-free entry point: the library's
    part of the call allocates nothing (its scratch is a fixed array of
    NOALLOC_SCRATCH_BYTES per device, shared by all such calls on it).
    Pass `out` (and `lse`, or return_lse=False) to allocate nothing here
    either, e.g. under graph capture."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 [B, H, N, d] tensor")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError(f"{name} must be on q's GPU")
    B, H, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError(f"k, v must be [B, H, Nk, d] matching q: {tuple(k.shape)} {tuple(v.shape)}")
    Nk = k.shape[2]
    _check_buf(out, "out", q.shape, torch.bfloat16, q.device)
    _check_buf(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _no_overlap((("out", out), ("lse", lse)), (("q", q), ("k", k), ("v", v)))
    o = torch.empty_like(q) if out is None else out
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _launch(lib.fa_fwd_splitkv_noalloc, "fa_fwd_splitkv_noalloc", q.device, _ptr(q), _ptr(k),
            _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, int(bool(causal)), float(scale),
            int(num_splits))
    return o, lse


def splitkv_splits(B: int, H: int, Nq: int, Nk: int, num_splits: int = 0,
                   causal: bool = False) -> int:
    """The number of key splits fa_fwd_splitkv uses for these sizes."""
    st = lib.fa_splitkv_splits(B, H, Nq, Nk, int(bool(causal)), num_splits)
    if st < 0:
        raise FAError(st, "fa_splitkv_splits")
    return st


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None):
    """Attention backward on bf16 [B, H, N, d] tensors; returns (dq, dk, dv).

    o and lse are the forward's outputs for the same q, k, v, causal, scale;
    do is the upstream gradient of o.
    """
    torch = _check_qkv(q, k, v, torch_bf16())
    B, H, N, d = q.shape
    for name, t in (("o", o), ("do", do)):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != tuple(q.shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like q")
        if t.device != q.device:
            raise ValueError(f"{name} is on another device than q")
    if lse is None or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buf(t, name, q.shape, torch.bfloat16, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _no_overlap((("dq", dq), ("dk", dk), ("dv", dv)),
                (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("do", do)))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _launch(lib.fa_bwd, "fa_bwd", q.device, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
            _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)), float(scale))
    return dq, dk, dv


def torch_bf16():
    import torch
    return torch.bfloat16


def _fp8():
    import torch
    return torch.float8_e4m3fn
