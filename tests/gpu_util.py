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


def ramp_amp(d, growth_log2, q0=4.0):
    """Height of the key ramp of fa_inputs.make_qkv_ramp (column 0 of Q set
    to q0) that makes the scores, at scale 1/sqrt(d), grow by about
    growth_log2 log2 units from the first key to the last."""
    import math
    return growth_log2 * math.sqrt(d) / (math.log2(math.e) * q0)


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


def bwd_gate(g_gpu, g_ref, extra=None):
    """Returns (ok, stats) for one gradient tensor of the backward pass.
    extra: an elementwise allowance added to the gate (and its norm to the
    RMS gate), for a reference that differs from the kernel's definition by
    a known amount."""
    err = np.abs(g_gpu - g_ref)
    if err.size == 0:
        return True, {}
    scale_max = float(np.abs(g_ref).max())
    norm = float(np.sqrt((g_ref ** 2).sum()))
    allowed = BWD_REL_MAX * scale_max + half_ulp_bf16(g_ref) + BWD_ABS_FLOOR
    extra_norm = 0.0
    if extra is not None:
        allowed = allowed + extra
        extra_norm = float(np.sqrt((extra ** 2).sum()))
    stats = {
        "max_abs": float(err.max()),
        "ref_max": scale_max,
        "rel_max": float(err.max()) / scale_max if scale_max > 0 else float(err.max()),
        "rel_rmse": float(np.sqrt((err ** 2).sum())) / norm if norm > 0 else float(err.max()),
        "finite": bool(np.all(np.isfinite(g_gpu))),
    }
    rmse_ok = (np.sqrt((err ** 2).sum())
               <= BWD_REL_RMSE * norm + BWD_ABS_FLOOR * np.sqrt(err.size) + extra_norm)
    ok = stats["finite"] and bool(np.all(err <= allowed)) and bool(rmse_ok)
    return ok, stats


def bwd_rounding_bound(q, k, v, do, o, lse, causal, scale):
    """Elementwise bound on |G - R| for the backward of one head (float64
    [N, d] arrays; o and lse as the backward was given them), R the gradient
    with D formed from that o, derived from the kernels' arithmetic rather
    than from a workload: S = Q K^T, dP = dO V^T and D = rowsum(dO * O) are
    float32 sums of exact products, P = exp2(scale*log2e*S - LSE*log2e) and
    dS = P (dP - D) are formed in float32, then P and dS are rounded to bf16
    (8 significant bits: relative error <= 2^-8) as operands of
    dV = P^T dO, dK = scale dS^T Q and dQ = scale dS K, which accumulate in
    float32. The rounding of G to bf16 is not included (the caller adds half
    an ulp). Where dQ comes from cancellation (sum_j dS_ij = 0 against large
    K rows) this allows more than the relative gate of the iid workloads.
    Returns (bound_dq, bound_dk, bound_dv)."""
    n, d = q.shape
    u = 2.0 ** -24
    log2e = 1.4426950408889634
    s = scale * (q @ k.T)
    mask = np.arange(n)[None, :] > np.arange(n)[:, None] if causal else None
    if mask is not None:
        s = np.where(mask, -np.inf, s)
    p = np.exp(s - lse[:, None])
    dp = do @ v.T
    dr = (do * o).sum(axis=1)
    ds = p * (dp - dr[:, None])
    # float32 error of P: its exp2 argument is a difference of terms of size
    # scale*log2e*sum|q||k| and |LSE|*log2e, each formed with at most d + 2
    # roundings; exp2 itself adds about one ulp
    arg = (d + 2) * u * (scale * log2e * (np.abs(q) @ np.abs(k).T) + log2e * np.abs(lse)[:, None])
    eps_p = np.log(2.0) * arg + 4 * u
    err_dp = d * u * (np.abs(do) @ np.abs(v).T)
    err_dr = d * u * (np.abs(do) * np.abs(o)).sum(axis=1)
    ds32 = np.abs(ds) * (eps_p + 2 * u) + p * (1 + eps_p) * (err_dp + err_dr[:, None])
    e_ds = 2.0 ** -8 * (np.abs(ds) + ds32) + ds32
    e_p = 2.0 ** -8 * p * (1 + eps_p) + p * eps_p
    if mask is not None:
        e_ds = np.where(mask, 0.0, e_ds)
        e_p = np.where(mask, 0.0, e_p)
    acc = n * u   # float32 accumulation over at most n terms
    bq = scale * (e_ds @ np.abs(k) + acc * (np.abs(ds) @ np.abs(k)))
    bk = scale * (e_ds.T @ np.abs(q) + acc * (np.abs(ds).T @ np.abs(q)))
    bv = e_p.T @ np.abs(do) + acc * (p.T @ np.abs(do))
    return bq, bk, bv


def oracle_fwd_inputs(g, causal, scale=None):
    """The forward output the backward is handed, from the oracle: O rounded
    to bf16 (the forward's output format) and LSE rounded to float32.
    Returns (o_bits uint16, lse float32), both over every (batch, head)."""
    o, lse = oracle_full(g.q, g.k, g.v, causal, scale)
    return fa_inputs.bf16_bits(o.astype(np.float32)), lse.astype(np.float32)


def run_bwd(fa, g, do_bits, causal, scale=None, fwd=None):
    """The library's backward on the oracle's forward output; returns float64
    ((dq, dk, dv), o) with o the bf16 O the backward was given. No output of
    the library enters the reference. fwd: (o_bits, lse) to use instead of
    the oracle's (a closed form)."""
    import torch
    q, k, v = to_device(g)
    do = fa_inputs.to_torch_bf16(do_bits, "cuda")
    o_bits, lse = fwd if fwd is not None else oracle_fwd_inputs(g, causal, scale)
    o = fa_inputs.to_torch_bf16(o_bits, "cuda")
    lse_t = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda()
    dq, dk, dv = fa.bwd(q, k, v, o, lse_t, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    grads = tuple(fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(t)) for t in (dq, dk, dv))
    return grads, fa_inputs.bf16_bits_to_f64(o_bits)


def oracle_backward_full(q, k, v, do, causal, scale=None, o=None, heads=None, workers=None):
    """oracle.attention_backward over the (batch, head) pairs `heads` (all by
    default) of float64 [B, H, N, d] inputs, spread over a thread pool as in
    oracle_full. Returns (dq, dk, dv) of the full shape (heads not asked for
    are left at zero)."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention_backward

    B, H, N, d = q.shape
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        got = attention_backward(q[sl], k[sl], v[sl], do[sl], causal, scale,
                                 o=None if o is None else o[sl])
        for x, y in zip(out, got):
            x[b, h] = y[0, 0]

    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(heads)))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, heads))
    return tuple(out)


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


def oracle_full(q, k, v, causal, scale=None, workers=None):
    """oracle.attention over every (batch, head) of float64 [B, H, N, d]
    inputs, the heads spread over a thread pool: NumPy releases the GIL in
    its matrix products and elementwise loops, and BLAS is held to one thread
    per worker. Each head is the oracle's own computation, unchanged.
    Returns (o, lse) as oracle.attention does."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention

    B, H, N, d = q.shape
    o = np.empty((B, H, N, v.shape[-1]))
    lse = np.empty((B, H, N))

    def one(bh):
        b, h = divmod(bh, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ob, lb = attention(q[sl], k[sl], v[sl], causal, scale)
        o[b, h], lse[b, h] = ob[0, 0], lb[0, 0]

    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0)), B * H))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(B * H)))
    return o, lse
