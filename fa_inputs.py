"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and rounds them to the storage formats the
attention path consumes. It holds none of the attention arithmetic: no score,
softmax, quantisation or rotation is computed here. Both the GPU path and the
CPU oracle receive exactly the arrays produced here.

Workloads (all synthetic; the pages measure on synthetic data themselves):
  * iid N(0,1) entries for Q, K, V, rounded to bf16 with round-to-nearest-even
    (the attention benchmark of the QbitAI FlashAttention-3 article, section on
    the attention benchmark, sweeps sequence length at 16k total tokens with
    random inputs).
  * the outlier model of that article's FP8 accuracy test: N(0,1) entries of
    which a fraction 0.001 carry a large N(0, 10^2) component. Two readings are
    provided: "replace" (the outlier value replaces the entry) and "add" (the
    outlier value is added to the entry, as that article words it).
  * random signs in {-1, +1} for the random-sign Hadamard rotation used by
    incoherent processing (FlashAttention-3 (HE), section on FP8 with
    incoherent processing).
  * an upstream gradient dO for the backward pass: iid N(0,1) entries of the
    output's shape, rounded to bf16 (the pages give no distribution for it;
    this is the plainest choice, the same as the inputs').
  * a structured workload (not on the pages) whose scores grow along the key
    axis: iid N(0,1) entries, then column 0 of Q set to a constant and column
    0 of K to a ramp over the key positions, rounded to bf16. Every row's
    running maximum then moves several times over the sequence, which iid
    inputs do only at the first key tile: it exercises the rescaling of the
    online softmax.
  * for tensors of more than 2^31 elements (the size-limit tests), iid N(0,1)
    entries drawn on the device by torch's seeded generator and rounded to
    bf16 there; the oracle receives the bf16 patterns of the heads it checks,
    copied back, so both sides still see the same values.
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; return the
    16-bit patterns as uint16 (same layout as torch.bfloat16)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def draw(rng: np.random.Generator, shape, dist: str = "normal",
         outlier_p: float = 0.001, outlier_sd: float = 10.0) -> np.ndarray:
    """Draw one float32 tensor of the given distribution."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if dist == "normal":
        return x
    mask = rng.random(shape) < outlier_p
    big = (rng.standard_normal(shape, dtype=np.float32) * np.float32(outlier_sd))
    if dist == "outlier_replace":
        return np.where(mask, big, x).astype(np.float32)
    if dist == "outlier_add":
        return (x + np.where(mask, big, np.float32(0))).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


class QKV:
    """Q, K, V of shape [B, H, N, d]: bf16 bit patterns plus exact float64."""

    def __init__(self, B, H, N, d, seed, dist="normal"):
        self.shape = (B, H, N, d)
        self.seed = seed
        self.dist = dist
        rng = np.random.default_rng(seed)
        self.q_bits = bf16_bits(draw(rng, self.shape, dist))
        self.k_bits = bf16_bits(draw(rng, self.shape, dist))
        self.v_bits = bf16_bits(draw(rng, self.shape, dist))

    @property
    def q(self):
        return bf16_bits_to_f64(self.q_bits)

    @property
    def k(self):
        return bf16_bits_to_f64(self.k_bits)

    @property
    def v(self):
        return bf16_bits_to_f64(self.v_bits)


def make_qkv(B, H, N, d, seed, dist="normal") -> QKV:
    return QKV(B, H, N, d, seed, dist)


def make_qkv_ramp(B, H, N, d, seed, q0, amp) -> QKV:
    """make_qkv's iid N(0,1) Q, K, V, then Q[..., n, 0] = q0 for every row
    and K[..., j, 0] = amp * j / N at key position j (both rounded to bf16)."""
    g = QKV(B, H, N, d, seed)
    q = g.q.astype(np.float32)
    k = g.k.astype(np.float32)
    q[..., 0] = np.float32(q0)
    k[..., 0] = (float(amp) * np.arange(N, dtype=np.float64) / N).astype(np.float32)
    g.q_bits = bf16_bits(q)
    g.k_bits = bf16_bits(k)
    g.dist = "ramp"
    return g


def make_grad(B, H, N, d, seed):
    """Upstream gradient dO [B, H, N, d]: (bf16 bit patterns, exact float64)."""
    rng = np.random.default_rng(seed)
    bits = bf16_bits(draw(rng, (B, H, N, d), "normal"))
    return bits, bf16_bits_to_f64(bits)


def random_signs(d: int, seed: int) -> np.ndarray:
    """d independent signs in {-1, +1} as float32."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def to_torch_bf16(bits: np.ndarray, device="cpu"):
    """View uint16 bf16 patterns as a torch.bfloat16 tensor (no rounding)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_tensor_to_bits(t) -> np.ndarray:
    """Inverse of to_torch_bf16: torch.bfloat16 tensor -> uint16 patterns."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def device_normal_bf16(shape, seed, device="cuda", chunk=1 << 27):
    """A torch.bfloat16 tensor of iid N(0,1) entries drawn on `device` by
    torch's generator seeded with `seed`, in float32 chunks of `chunk`
    elements rounded to bf16 on the device."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    return out


# Seeds are fixed per workload in advance.
SEEDS = {
    "small": 1,          # B=1 H=2 N=256 d=64
    "mid": 2,            # B=4 H=16 N=2048 d=128
    "seq_sweep_base": 300,   # + log2(N/512)
    "dim_sweep_base": 400,   # + index of d in (64, 96, 128, 256)
    "fp8": 5,
    "fp8_signs": 55,
    "grad_offset": 100000,   # dO seed = the Q/K/V seed + this offset
    "large": 600,        # tensors of more than 2^31 elements (device-drawn)
}
