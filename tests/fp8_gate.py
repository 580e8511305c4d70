"""Tolerance of the e4m3 forward kernel against exact attention on its own
dequantised operands, derived from the rounding of P to e4m3.

The kernel forms the scores of the dequantised (rotated) operands exactly up
to float32 rounding, so apart from float32 effects (relative 1e-6) its output
differs from exact attention on those operands only by the rounding of the
probabilities it feeds to the e4m3 P V product: it rounds x = P * 2^6 * r to
e4m3, with P = exp(score - m) for a reference maximum m at or below the row's
true maximum (so P >= the oracle's P, relative to the true maximum, and the
largest P of a row is >= 1) and r the V fold ratio of the key's block, which
lies in [max(2^-4, s_V / max s_V), 1] (the reference V scale of a wave never
exceeds the head's largest V block scale, and the fold keeps r >= 2^-4). Its
row sum adds the same rounded values. Rounding to nearest e4m3 (3 mantissa
bits; subnormal spacing 2^-9) moves x by at most max(2^-4 x, 2^-10), so each
P moves by at most  e_j = max(2^-4 P_j, 2^-16 / r_j).

With w_j = P_j / sum P and O = sum_j w_j V_j, the kernel returns
O~ = sum_j P~_j V_j / sum P~, and because sum_j P_j (V_j - O) = 0,
    O~ - O = sum_j (P~_j - P_j) (V_j - O) / sum P~,
    |O~_c - O_c| <= sum_j e_j |V_jc - O_c| / (sum_j P_j - sum_j e_j)
                 <= (sum_j e_j |V_jc| + |O_c| sum_j e_j) / (sum_j P_j - sum_j e_j),
which is largest when the kernel's reference maximum equals the true one
(P relative to the true maximum, as the oracle forms it). The second form
(two matrix products, at any size) is the elementwise bound, plus the bf16
rounding of the output (half an ulp) and a float32 allowance. The log-sum-exp moves by at most -ln(1 - sum e / sum P).

A statistical check beside it: with the rounding error of each x spread
uniformly over +-(its bound), E|O~ - O|^2 <= sum_j e_j^2 / 3 |V_j - O|^2 /
(sum P)^2 per element (an upper bound: the real error of rounding to nearest
is smaller for most x); the whole tensor's squared error must stay below the
sum of these plus the output rounding.
"""
from __future__ import annotations

import numpy as np

P_REL = 2.0 ** -4        # half an e4m3 ulp, relative to the value (3 mantissa bits)
X_SUB_ABS = 2.0 ** -10   # half the e4m3 subnormal spacing
HEADROOM = 2.0 ** 6      # the kernel rounds P * 2^6 * r
R_MIN = 2.0 ** -4        # the V fold ratio never falls below this
BLOCK = 128


def half_ulp_bf16(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 0.5 * np.exp2(e - 7)


def fp8_reference_and_bounds(qd, kd, vd, sv, causal, scale):
    """Exact attention of dequantised operands [B, H, N, d] (float64) with
    the elementwise error bound of the e4m3 kernel. sv: the V block scales
    [B, H, ceil(N/128)] the kernel was given (positive).

    Returns (o, lse, bound_o, bound_lse, var_o): o, bound_o, var_o
    [B, H, N, d]; lse, bound_lse [B, H, N]."""
    B, H, N, d = qd.shape
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    bound_o = np.empty_like(o)
    bound_lse = np.empty_like(lse)
    var_o = np.empty_like(o)
    sv = np.asarray(sv, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scale * (qd[b, h] @ kd[b, h].T)
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)                                   # row maximum 1
            z = p.sum(axis=1, keepdims=True)
            oh = (p @ vd[b, h]) / z
            o[b, h] = oh
            lse[b, h] = m[:, 0] + np.log(z[:, 0])
            r = np.maximum(R_MIN, np.repeat(sv[b, h] / sv[b, h].max(), BLOCK)[:N])
            e = np.maximum(P_REL * p, X_SUB_ABS / (HEADROOM * r)[None, :])
            e = np.where(p > 0, e, 0.0)                         # masked keys carry no P
            esum = e.sum(axis=1, keepdims=True)
            denom = z - esum
            if np.any(denom <= 0):
                raise ValueError("rounding bound not informative (sum of P below its error)")
            vh = vd[b, h]
            # sum_j e_j |V_jc - O_ic| <= sum_j e_j |V_jc| + |O_ic| sum_j e_j
            bound = (e @ np.abs(vh) + esum * np.abs(oh)) / denom
            bound_o[b, h] = bound + half_ulp_bf16(np.abs(oh) + bound) + 1e-6 * np.abs(vh).max()
            # sum_j e_j^2 (V_jc - O_ic)^2, the square expanded
            e2 = e ** 2
            var = (e2 @ vh ** 2 - 2.0 * oh * (e2 @ vh) + oh ** 2 * e2.sum(axis=1, keepdims=True))
            var_o[b, h] = np.maximum(var, 0.0) / 3.0 / z ** 2
            bound_lse[b, h] = -np.log1p(-esum[:, 0] / z[:, 0]) + 1e-5
    return o, lse, bound_o, bound_lse, var_o


def fp8_gate(o_gpu, o, bound_o, var_o, rms=True):
    """Returns (ok, stats): elementwise |o_gpu - o| <= bound_o, and (rms)
    the squared error summed over the tensor within the statistical
    allowance (a statistical check: it needs a few thousand (query, key)
    pairs to be steady, so tiny shapes skip it)."""
    err = np.abs(o_gpu - o)
    rounding = half_ulp_bf16(o) ** 2 / 3.0 * 4.0   # output rounding, uniform within +-1 ulp/2 (x4 margin)
    allowed_sq = float(var_o.sum() + rounding.sum())
    stats = {
        "max_abs": float(err.max()),
        "worst_ratio": float((err / bound_o).max()),
        "rel_rmse": float(np.linalg.norm(o_gpu - o) / np.linalg.norm(o)),
        "rms_ratio": float(np.sqrt((err ** 2).sum() / allowed_sq)) if allowed_sq > 0 else 0.0,
        "finite": bool(np.all(np.isfinite(o_gpu))),
    }
    ok = stats["finite"] and bool(np.all(err <= bound_o)) and (not rms or stats["rms_ratio"] <= 1.0)
    return ok, stats
