"""GPU parity of the FP8 path, every gate against the float64 oracle only.

  * The block quantiser against the oracle's quantiser (code = e4m3 of y / s,
    round to nearest even): the kernel applies the scale through its
    correctly rounded float32 reciprocal, so a code may differ only where
    the kernel's scaled value and the exact quotient lie on two sides of a
    rounding midpoint of adjacent e4m3 values; such codes are counted and
    bounded.
  * The e4m3 forward kernel against exact attention on its own dequantised
    operands, within the bound that the rounding of P to e4m3 allows
    (tests/fp8_gate.py), and its log-sum-exp likewise. The oracle's FP8
    emulator only prints a prediction beside it.
  * The full FP8 workload (B=2 H=16 N=8192 d=128, outliers) against exact
    attention on the original bf16 inputs over the whole tensor: relative
    RMSE <= 5e-2 with block scales and the Hadamard rotation, reported
    beside the block-only and per-tensor variants.
  * The end-to-end path (fa_fwd in FP8 mode) against the explicit pipeline,
    bit for bit, and against the exact oracle.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest

import fa_inputs
from oracle import attention, fp8
from tests.fp8_gate import fp8_gate, fp8_reference_and_bounds
from tests.gpu_util import FP8_REL_RMSE, oracle_full, ramp_amp

pytestmark = pytest.mark.gpu


def announce(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


def rel_rmse(a, ref):
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def gpu_quant(lib, bits, per_tensor, signs):
    import torch
    x = fa_inputs.to_torch_bf16(bits, "cuda")
    s = torch.from_numpy(signs).cuda() if signs is not None else None
    x8, sc = lib.quant_fp8(x, per_tensor=per_tensor, signs=s)
    torch.cuda.synchronize()
    return x8.view(torch.uint8).cpu().numpy(), sc.cpu().numpy()


def gpu_fwd_fp8(lib, codes, scales, causal, scale=None):
    import torch
    dev = [torch.from_numpy(c).cuda().view(torch.float8_e4m3fn) for c in codes]
    sc = [torch.from_numpy(np.ascontiguousarray(s)).cuda() for s in scales]
    o, lse = lib.fwd_fp8(*dev, *sc, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o64 = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o))
    return o64, lse.cpu().numpy().astype(np.float64)


def near_midpoint(t, t_err):
    """Whether t lies within t_err of a midpoint between adjacent e4m3
    values (where a scaled value off by t_err may round either way)."""
    code = fp8.e4m3_encode(t).astype(np.int64)
    mag = np.abs(fp8.e4m3_decode(code & 0x7F))
    up = fp8.e4m3_decode(np.minimum((code & 0x7F) + 1, 0x7E))
    down = fp8.e4m3_decode(np.maximum((code & 0x7F) - 1, 0))
    a = np.abs(t)
    return (np.abs(a - 0.5 * (mag + up)) <= t_err) | (np.abs(a - 0.5 * (mag + down)) <= t_err)


def check_codes(codes_gpu, codes_ref, t_exact, t_err):
    """Codes equal in value, except where the exact quotient t lies within
    t_err of the midpoint between the two codes' values (the kernel's own
    scaled value may then round to the other side). bf16 inputs have 8
    significant bits, so such near-ties are far more frequent than for
    continuous values (up to a few per thousand of the outlier workload's
    codes): their number is printed beside the number of codes that differ,
    which may not exceed it (nor 1% of the codes)."""
    a = fp8.e4m3_decode(codes_gpu)
    b = fp8.e4m3_decode(codes_ref)
    diff = a != b
    n = int(diff.sum())
    eligible = int(near_midpoint(t_exact, t_err).sum())
    announce("  codes differing:", n, "near a rounding midpoint:", eligible, "of", codes_gpu.size)
    if n:
        mid = 0.5 * (a[diff] + b[diff])
        assert np.all(np.abs(t_exact[diff] - mid) <= t_err[diff]), \
            float((np.abs(t_exact[diff] - mid) / t_err[diff]).max())
        lo = np.minimum(np.abs(a[diff]), np.abs(b[diff]))
        hi = np.maximum(np.abs(a[diff]), np.abs(b[diff]))
        # adjacent values: the larger magnitude is the next code after the smaller
        nxt = fp8.e4m3_decode(fp8.e4m3_encode(lo).astype(np.int64) + 1)
        assert np.all(hi == nxt)
    assert n <= eligible and n <= 1e-2 * codes_gpu.size


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_quant_unrotated(lib, d, per_tensor):
    announce("quant unrotated", d, per_tensor)
    g = fa_inputs.make_qkv(2, 3, 300, d, 500 + d, "outlier_replace")
    codes, sc = gpu_quant(lib, g.q_bits, per_tensor, None)
    rc, rs = fp8.quantize(g.q, per_tensor=per_tensor)
    np.testing.assert_array_equal(sc, rs)      # s = amax / 448, correctly rounded, both sides
    s_rows = np.repeat(rs.astype(np.float64), 128, axis=2)[:, :, :300, None]
    t = np.clip(g.q / s_rows, -448.0, 448.0)
    # kernel: float32(y * float32(1/s)), two roundings of 2^-24 relative
    check_codes(codes, rc, t, np.abs(t) * 2.0 ** -22)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_quant_rotated(lib, d, per_tensor):
    announce("quant rotated", d, per_tensor)
    g = fa_inputs.make_qkv(2, 3, 300, d, 600 + d, "outlier_replace")
    signs = fa_inputs.random_signs(d, 601)
    codes, sc = gpu_quant(lib, g.q_bits, per_tensor, signs)
    rc, rs = fp8.quantize(g.q, per_tensor=per_tensor, signs=signs)
    # the kernel's float32 butterflies may move amax, hence s, by an ulp
    np.testing.assert_allclose(sc, rs, rtol=2.0 ** -22)
    y = fp8.rotate_unnormalised(g.q, signs)
    s_rows = np.repeat(rs.astype(np.float64) * math.sqrt(d), 128, axis=2)[:, :, :300, None]
    t = np.clip(y / s_rows, -448.0, 448.0)
    # float32 butterfly sums: log2(d) stages, each within 2^-24 of the row's
    # absolute sum; then the scale's reciprocal and the product
    rowabs = np.abs(g.q).sum(axis=3, keepdims=True)
    t_err = (math.log2(d) + 1) * 2.0 ** -24 * rowabs / s_rows + np.abs(t) * 2.0 ** -21
    check_codes(codes, rc, t, t_err)


def check_fwd_fp8(lib, codes, scales, causal, scale, exact=None, rms=True):
    """Runs the e4m3 kernel on the codes; gates O and LSE against exact
    attention on the dequantised operands; prints the emulator's prediction
    and (if given) the error against exact attention on the bf16 inputs."""
    qc, kc, vc = codes
    sq, sk, sv = scales
    o_gpu, lse_gpu = gpu_fwd_fp8(lib, codes, scales, causal, scale)
    qd, kd, vd = (fp8.dequantize(c, s) for c, s in zip(codes, scales))
    o_ref, lse_ref, bo, bl, var = fp8_reference_and_bounds(qd, kd, vd, sv, causal, scale)
    ok, st = fp8_gate(o_gpu, o_ref, bo, var, rms=rms)
    lse_ok = bool(np.all(np.isfinite(lse_gpu)) and np.all(np.abs(lse_gpu - lse_ref) <= bl))
    o_emul = fp8.fp8_attention_emulate(qc, kc, vc, sq, sk, sv, causal, scale)
    extra = {"emulator_rel_rmse_vs_dequantised": rel_rmse(o_emul, o_ref)}
    if exact is not None:
        extra["rel_rmse_vs_exact_bf16_inputs"] = rel_rmse(o_gpu, exact)
    announce("  vs dequantised oracle", st, "lse max", float(np.abs(lse_gpu - lse_ref).max()),
             "lse bound min", float(bl.min()), extra)
    assert ok, st
    assert lse_ok
    return o_gpu, st


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_small(lib, d, causal):
    announce("fwd fp8 small", d, causal)
    B, H, N = 1, 2, 333
    g = fa_inputs.make_qkv(B, H, N, d, 700 + d, "outlier_replace")
    signs = fa_inputs.random_signs(d, 701)
    qc, sq = fp8.quantize(g.q, signs=signs)
    kc, sk = fp8.quantize(g.k, signs=signs)
    vc, sv = fp8.quantize(g.v)
    o_ref, _ = attention(g.q, g.k, g.v, causal)
    o_gpu, _ = check_fwd_fp8(lib, (qc, kc, vc), (sq, sk, sv), causal, 1.0 / math.sqrt(d),
                             exact=o_ref)
    # the 5e-2 target is stated for the full FP8 workload (below); at this
    # small shape the method's own error (Q, K, V quantisation) sits near it
    assert rel_rmse(o_gpu, o_ref) <= 1.5 * FP8_REL_RMSE


@pytest.mark.parametrize("N", [1, 17, 65, 129, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_ragged(lib, N, causal):
    """Ragged sequence lengths: key-tile counts from 1 to 5 (both parities of
    the last step's stage), partial last tiles, queries past N in the last
    query tile."""
    announce("fwd fp8 ragged", N, causal)
    B, H, d = 1, 2, 64
    g = fa_inputs.make_qkv(B, H, N, d, 730 + N, "outlier_replace")
    codes, scales = zip(*(fp8.quantize(x) for x in (g.q, g.k, g.v)))
    check_fwd_fp8(lib, codes, scales, causal, 1.0 / math.sqrt(d), rms=N >= 64)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_scale_argument_and_optional_lse(lib, causal):
    """A scale other than 1/sqrt(d) reaches the e4m3 kernel's scores, and
    skipping the LSE store leaves O bit for bit unchanged."""
    import torch
    announce("fwd fp8 scale 0.05 / no lse", causal)
    B, H, N, d = 1, 2, 300, 128
    g = fa_inputs.make_qkv(B, H, N, d, 740, "outlier_replace")
    signs = fa_inputs.random_signs(d, 741)
    qc, sq = fp8.quantize(g.q, signs=signs)
    kc, sk = fp8.quantize(g.k, signs=signs)
    vc, sv = fp8.quantize(g.v)
    check_fwd_fp8(lib, (qc, kc, vc), (sq, sk, sv), causal, 0.05)
    dev = [torch.from_numpy(c).cuda().view(torch.float8_e4m3fn) for c in (qc, kc, vc)]
    sc = [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (sq, sk, sv)]
    o1, l1 = lib.fwd_fp8(*dev, *sc, causal=causal, scale=0.05)
    o2, l2 = lib.fwd_fp8(*dev, *sc, causal=causal, scale=0.05, return_lse=False)
    torch.cuda.synchronize()
    assert l2 is None
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def structured_v(kind, v):
    """V with structure the plain workload lacks: a zero-padded last block
    (its scale is 1, far above the others), blocks whose magnitudes differ
    by 100x, or tiny values (amax ~1e-3) beside a zero block."""
    v = v.copy()
    if kind == "zero_block":
        v[:, :, 256:] = 0.0
    elif kind == "spread":
        for t, f in enumerate((100.0, 1.0, 0.01)):
            v[:, :, 128 * t:128 * (t + 1)] *= f
    elif kind == "spread_rising":
        for t, f in enumerate((0.01, 1.0, 100.0)):
            v[:, :, 128 * t:128 * (t + 1)] *= f
    elif kind == "tiny":
        v *= 1e-3
        v[:, :, 256:] = 0.0
    return v


@pytest.mark.parametrize("kind", ["zero_block", "spread", "spread_rising", "tiny"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_structured_v_scales(lib, kind, d, causal):
    """V block scales far apart within one head: the V fold keeps every
    tile's P * 2^6 * r at or above 2^2 * P (the reference V scale moves when
    the ratio leaves [2^-4, 1]), so these cases meet the same rounding bound
    as the plain workload, and rows that never reach the zero block stay
    finite."""
    announce("fwd fp8 structured V", kind, d, causal)
    B, H, N = 1, 2, 384
    g = fa_inputs.make_qkv(B, H, N, d, 760 + d, "outlier_replace")
    v = structured_v(kind, g.v)
    signs = fa_inputs.random_signs(d, 761)
    qc, sq = fp8.quantize(g.q, signs=signs)
    kc, sk = fp8.quantize(g.k, signs=signs)
    vc, sv = fp8.quantize(v)
    announce("  V block scales", sv[0, 0].tolist())
    o_ref, _ = attention(g.q, g.k, v, causal)
    check_fwd_fp8(lib, (qc, kc, vc), (sq, sk, sv), causal, 1.0 / math.sqrt(d), exact=o_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_running_max_moves(lib, causal):
    """Scores growing along the key axis (fa_inputs.make_qkv_ramp, about 8.5
    log2 units every 256 keys; Q and K rotated): the e4m3 kernel's reference
    maximum, with its 2.75 log2-unit window, moves at most key tiles, each
    move rescaling the accumulator and the row sum; K's block scales grow
    along the sequence. Gated against exact attention on the dequantised
    operands like the other cases."""
    announce("fwd fp8 ramp", causal)
    B, H, N, d = 1, 2, 1000, 128
    g = fa_inputs.make_qkv_ramp(B, H, N, d, 780 + causal, 4.0, ramp_amp(d, 8.5 * N / 256))
    signs = fa_inputs.random_signs(d, 781)
    qc, sq = fp8.quantize(g.q, signs=signs)
    kc, sk = fp8.quantize(g.k, signs=signs)
    vc, sv = fp8.quantize(g.v)
    o_ref, _ = attention(g.q, g.k, g.v, causal)
    check_fwd_fp8(lib, (qc, kc, vc), (sq, sk, sv), causal, 1.0 / math.sqrt(d), exact=o_ref)


def test_fwd_fp8_long_sequence_table_reload(lib):
    """N = 8320 (65 quantisation blocks): the kernel's per-block factor table
    holds 64 blocks and is reloaded for block 64; V's last block is far
    smaller than the rest."""
    announce("fwd fp8 N=8320 d=128 noncausal (table reload)")
    B, H, N, d = 1, 2, 8320, 128
    g = fa_inputs.make_qkv(B, H, N, d, 770, "outlier_replace")
    v = g.v.copy()
    v[:, :, 8192:] *= 0.001
    signs = fa_inputs.random_signs(d, 771)
    qc, sq = fp8.quantize(g.q, signs=signs)
    kc, sk = fp8.quantize(g.k, signs=signs)
    vc, sv = fp8.quantize(v)
    check_fwd_fp8(lib, (qc, kc, vc), (sq, sk, sv), False, 1.0 / math.sqrt(d))


def test_fwd_fp8_causal_row0_closed_form(lib):
    announce("fwd fp8 causal row 0")
    g = fa_inputs.make_qkv(1, 2, 200, 128, 710)
    qc, sq = fp8.quantize(g.q)
    kc, sk = fp8.quantize(g.k)
    vc, sv = fp8.quantize(g.v)
    o_gpu, _ = gpu_fwd_fp8(lib, (qc, kc, vc), (sq, sk, sv), True)
    v0 = fp8.dequantize(vc, sv)[:, :, 0]
    # row 0 attends key 0 only: P = 1, O = dequantised V[0], then bf16-rounded
    expect = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_bits(v0.astype(np.float32)))
    np.testing.assert_allclose(o_gpu[:, :, 0], expect, rtol=2 ** -8, atol=0)


@pytest.mark.parametrize("dist", ["outlier_replace", "outlier_add"])
def test_fp8_config_full_tensor(lib, dist):
    """B=2 H=16 N=8192 d=128, outliers replacing 0.1% of entries (and the
    QbitAI article's additive wording of the same model), block scales with
    Hadamard rotation; beside it the variants without rotation and with one
    scale per tensor. Relative RMSE over the whole tensor against exact
    attention on the bf16 inputs."""
    import torch
    announce("fp8 full config, whole tensor", dist)
    B, H, N, d = 2, 16, 8192, 128
    g = fa_inputs.make_qkv(B, H, N, d, fa_inputs.SEEDS["fp8"], dist)
    signs = fa_inputs.random_signs(d, fa_inputs.SEEDS["fp8_signs"])
    q, k, v = (fa_inputs.to_torch_bf16(b, "cuda") for b in (g.q_bits, g.k_bits, g.v_bits))
    st = torch.from_numpy(signs).cuda()
    outs = {}
    for name, per_tensor, rot in (("block+hadamard", False, True), ("block", False, False),
                                  ("per-tensor", True, False)):
        s_ = st if rot else None
        q8, sq = lib.quant_fp8(q, per_tensor=per_tensor, signs=s_)
        k8, sk = lib.quant_fp8(k, per_tensor=per_tensor, signs=s_)
        v8, sv = lib.quant_fp8(v, per_tensor=per_tensor)
        o, _ = lib.fwd_fp8(q8, k8, v8, sq, sk, sv)
        torch.cuda.synchronize()
        outs[name] = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o))
        del q8, k8, v8, o
    announce("  oracle over", B * H, "heads")
    o_ref, _ = oracle_full(g.q, g.k, g.v, False)
    errs = {name: rel_rmse(o, o_ref) for name, o in outs.items()}
    announce("  rel_rmse", errs,
             "per-tensor / block+hadamard", errs["per-tensor"] / errs["block+hadamard"])
    assert all(np.all(np.isfinite(o)) for o in outs.values())
    assert errs["block+hadamard"] <= FP8_REL_RMSE
    assert errs["block+hadamard"] < errs["per-tensor"]


def test_fp8_end_to_end_path(lib):
    import torch
    announce("fp8 end-to-end fa_fwd")
    B, H, N, d = 1, 4, 2048, 128
    g = fa_inputs.make_qkv(B, H, N, d, 720, "outlier_replace")
    q, k, v = (fa_inputs.to_torch_bf16(b, "cuda") for b in (g.q_bits, g.k_bits, g.v_bits))
    for causal in (False, True):
        o, lse = lib.fwd(q, k, v, causal=causal, dtype=lib.FA_FP8_E4M3)
        torch.cuda.synchronize()
        o64 = fa_inputs.bf16_bits_to_f64(fa_inputs.bf16_tensor_to_bits(o))
        o_ref, lse_ref = attention(g.q, g.k, g.v, causal)
        e = rel_rmse(o64, o_ref)
        announce("  causal", causal, "rel_rmse", e,
                 "lse max abs", float(np.abs(lse.cpu().numpy() - lse_ref).max()))
        assert e <= FP8_REL_RMSE


def splitmix64_signs(d, key=0x5A17C0DE):
    """The end-to-end path's fixed signs, from the published SplitMix64
    definition (Steele, Lea, Flood 2014): sign i is -1 where the top bit of
    SplitMix64(key + i) is set."""
    mask = (1 << 64) - 1
    out = np.empty(d, dtype=np.float32)
    for i in range(d):
        x = (key + i + 0x9E3779B97F4A7C15) & mask
        x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & mask
        x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & mask
        x ^= x >> 31
        out[i] = -1.0 if x >> 63 else 1.0
    return out


@pytest.mark.parametrize("d", [64, 128, 256])
def test_end_to_end_equals_explicit_pipeline(lib, d):
    """fa_fwd(FP8) quantises Q inside the forward kernel; its output must be
    bit for bit that of fa_quant_fp8 (Q and K rotated by the fixed signs, V
    plain) followed by fa_fwd_fp8."""
    import torch
    for causal in (False, True):
        B, H, N = 1, 3, 300
        announce("fp8 end-to-end vs explicit pipeline", B, H, N, d, "causal" if causal else "")
        g = fa_inputs.make_qkv(B, H, N, d, 730 + d, "outlier_replace")
        q, k, v = (fa_inputs.to_torch_bf16(b, "cuda") for b in (g.q_bits, g.k_bits, g.v_bits))
        o1, l1 = lib.fwd(q, k, v, causal=causal, dtype=lib.FA_FP8_E4M3)
        s = torch.from_numpy(splitmix64_signs(d)).cuda()
        q8, sq = lib.quant_fp8(q, signs=s)
        k8, sk = lib.quant_fp8(k, signs=s)
        v8, sv = lib.quant_fp8(v)
        o2, l2 = lib.fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        o3, l3 = lib.fwd(q, k, v, causal=causal, dtype=lib.FA_FP8_E4M3, return_lse=False)
        torch.cuda.synchronize()
        assert l3 is None and torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def test_fp8_deterministic_and_grid_order(lib):
    """Repeated end-to-end FP8 calls (quantisation passes, in-kernel Q
    quantisation, e4m3 forward) give bitwise identical outputs, also with
    the workgroups run in reverse order and the LDS filled with NaN bytes
    before the first copy (FA_DEBUG=3): a tile read before its copy landed,
    or a workgroup depending on another, would change the result."""
    import torch
    announce("fp8 determinism and reversed grid 2 4 1000 128 causal")
    g = fa_inputs.make_qkv(2, 4, 1000, 128, 750, "outlier_replace")
    q, k, v = (fa_inputs.to_torch_bf16(b, "cuda") for b in (g.q_bits, g.k_bits, g.v_bits))
    runs = [lib.fwd(q, k, v, causal=True, dtype=lib.FA_FP8_E4M3) for _ in range(3)]
    os.environ["FA_DEBUG"] = "3"
    try:
        runs.append(lib.fwd(q, k, v, causal=True, dtype=lib.FA_FP8_E4M3))
    finally:
        del os.environ["FA_DEBUG"]
    torch.cuda.synchronize()
    for o, lse in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(lse, runs[0][1])
