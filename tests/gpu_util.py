"""Helpers for the GPU parity tests: run the library on seeded inputs and
compare with the float64 oracle under the stated gates."""
from __future__ import annotations

import numpy as np

import fa_inputs

# bf16 gates: |O_gpu - O_ref| <= 1e-2 + half a bf16 ulp of O_ref elementwise,
# and mean |O_gpu - O_ref| <= 1e-3 + mean |rne_bf16(O_ref) - O_ref|. The 1e-2
# and 1e-3 budgets cover the kernel's arithmetic; the added terms are the
# rounding of the mandated bf16 output, which on its own exceeds the literal
# budgets where |O| is near 1 (few keys: early causal rows, tiny N).
# LSE: max-abs <= 1e-3.
BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3
FP8_REL_RMSE = 5e-2


def half_ulp_bf16(x):
    """Half the spacing of bf16 values at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 0.5 * np.exp2(e - 7)


def bf16_gate(o_gpu, o_ref):
    """Returns (ok, stats) for the bf16 output gate."""
    err = np.abs(o_gpu - o_ref)
    allowed = BF16_MAX_ABS + half_ulp_bf16(o_ref)
    floor = np.abs(fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_bits(o_ref.astype(np.float32))) - o_ref)
    mean_floor = float(floor.mean()) if floor.size else 0.0
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "rounding_floor": float(floor.max()) if floor.size else 0.0,
        "mean_rounding_floor": mean_floor,
        "worst_excess": float((err - allowed).max()) if err.size else -1.0,
    }
    ok = bool(np.all(err <= allowed)) and stats["mean_abs"] <= BF16_MEAN_ABS + mean_floor
    return ok, stats


# Backward gates, relative to the gradient's own size (see test_bwd_bf16.py).
BWD_REL_MAX = 1e-2
BWD_REL_RMSE = 5e-3
# Absolute floor for gradients that vanish exactly (one key: dK = 0), where the
# float32 sums of the kernel leave residues near 2^-24 of their terms.
BWD_ABS_FLOOR = 1e-4


def bwd_gate(g_gpu, g_ref):
    """Returns (ok, stats) for one gradient tensor of the backward pass."""
    err = np.abs(g_gpu - g_ref)
    if err.size == 0:
        return True, {}
    scale_max = float(np.abs(g_ref).max())
    norm = float(np.sqrt((g_ref ** 2).sum()))
    allowed = BWD_REL_MAX * scale_max + half_ulp_bf16(g_ref) + BWD_ABS_FLOOR
    stats = {
        "max_abs": float(err.max()),
        "ref_max": scale_max,
        "rel_max": float(err.max()) / scale_max if scale_max > 0 else float(err.max()),
        "rel_rmse": float(np.sqrt((err ** 2).sum())) / norm if norm > 0 else float(err.max()),
        "finite": bool(np.all(np.isfinite(g_gpu))),
    }
    rmse_ok = np.sqrt((err ** 2).sum()) <= BWD_REL_RMSE * norm + BWD_ABS_FLOOR * np.sqrt(err.size)
    ok = stats["finite"] and bool(np.all(err <= allowed)) and bool(rmse_ok)
    return ok, stats


def run_bwd(fa, g, do_bits, causal, scale=None):
    """The library's forward, then its backward; returns float64
    ((dq, dk, dv), o) with o the forward output the backward was given."""
    import torch
    q, k, v = to_device(g)
    do = fa_inputs.to_torch_bf16(do_bits, "cuda")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    grads = tuple(fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(t)) for t in (dq, dk, dv))
    return grads, fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o))


def to_device(g, device="cuda"):
    q = fa_inputs.to_torch_bf16(g.q_bits, device)
    k = fa_inputs.to_torch_bf16(g.k_bits, device)
    v = fa_inputs.to_torch_bf16(g.v_bits, device)
    return q, k, v


def run_bf16(fa, g, causal, scale=None):
    import torch
    q, k, v = to_device(g)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o64 = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o))
    return o64, lse.cpu().numpy().astype(np.float64)


def sample_rows(B, H, N, count, seed):
    """(b, h, i) samples: first/last rows, tile edges and random rows."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 2, N - 1]
    fixed = [i for i in fixed if 0 <= i < N]
    rows = []
    for i in fixed:
        rows.append((int(rng.integers(B)), int(rng.integers(H)), i))
    while len(rows) < count:
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))))
    return np.array(rows, dtype=np.int64)
