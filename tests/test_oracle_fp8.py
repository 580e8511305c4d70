"""Pins of the oracle's FP8 pieces: the e4m3fn encoder/decoder against torch's
CPU float8_e4m3fn cast (a library routine) and the format's closed forms; the
Sylvester Hadamard matrix against its closed form; the block quantiser against
the error bound of a 3-bit mantissa and its defining identities; rotation
invariance of exact attention; a hand-built block's codes and scales; the
emulator's reduction to exact attention.
"""
import math

import numpy as np
import pytest

from oracle import attention
from oracle import fp8
import fa_inputs

torch = pytest.importorskip("torch")


def torch_e4m3_codes(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_matches_library_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(ours[ok], lib[ok])
    assert np.nanmax(ours) == 448.0
    assert fp8.e4m3_decode(np.array([1]))[0] == 2.0 ** -9
    assert fp8.e4m3_decode(np.array([8]))[0] == 2.0 ** -6


def test_encode_matches_library():
    vals = fp8.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2                  # exact ties
    rng = np.random.default_rng(3)
    rand = rng.uniform(-448, 448, 20000)
    small = rng.uniform(-2 ** -5, 2 ** -5, 20000)
    x = np.concatenate([vals, -vals, mids, -mids, rand, small,
                        np.nextafter(mids, 0), np.nextafter(mids, 1000), [0.0, -0.0, 448.0, -448.0]])
    x = x.astype(np.float32).astype(np.float64)         # values a float32 kernel can hold
    np.testing.assert_array_equal(fp8.e4m3_encode(x), torch_e4m3_codes(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([449.0]))


def test_hadamard_closed_form():
    for d in (1, 2, 8, 64, 128, 256):
        h = fp8.hadamard(d)
        i = np.arange(d)
        pop = np.vectorize(lambda a: bin(a).count("1"))(i[:, None] & i[None, :])
        np.testing.assert_array_equal(h, (-1.0) ** pop)
        np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


@pytest.mark.parametrize("per_tensor", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_bounds_and_identities(per_tensor, rotate):
    B, H, N, d = 2, 2, 300, 64
    x = fa_inputs.make_qkv(B, H, N, d, seed=11, dist="outlier_replace").q
    signs = fa_inputs.random_signs(d, 12) if rotate else None
    codes, scales = fp8.quantize(x, per_tensor=per_tensor, signs=signs)
    assert codes.dtype == np.uint8 and scales.shape == (B, H, 3)
    y = fp8.rotate_unnormalised(x, signs) if rotate else x
    norm = 1.0 / math.sqrt(d) if rotate else 1.0
    nblk = 3
    s_unnorm = np.zeros((B, H, nblk))
    for b in range(B):
        for h in range(H):
            for t in range(nblk):
                blk = y[b, h, t * 128:(t + 1) * 128]
                s_unnorm[b, h, t] = np.float32(np.abs(blk).max() / 448.0)
    if per_tensor:
        s_unnorm[...] = np.float32(np.abs(y).max() / 448.0)
        assert np.all(scales == scales.flat[0])
    np.testing.assert_allclose(scales, s_unnorm * norm, rtol=2 ** -24)
    vals = fp8.e4m3_decode(codes)
    # every block reaches the top code 448 (per tensor: the block with the amax)
    top = np.abs(vals).reshape(B, H, -1).max(axis=2)
    if not per_tensor:
        assert np.all(top == 448.0)
    # dequantisation error: half an e4m3 ulp of the scaled value
    srows = np.repeat(s_unnorm, 128, axis=2)[:, :, :N, None]
    t = np.clip(y / srows, -448.0, 448.0)
    err = np.abs(vals - t)
    bound = np.where(np.abs(t) >= 2 ** -6, 2.0 ** -4 * np.abs(t), 2.0 ** -10)
    assert np.all(err <= bound)
    # dequantize reproduces value * stored scale
    np.testing.assert_allclose(fp8.dequantize(codes, scales), vals * np.repeat(scales, 128, axis=2)[:, :, :N, None])


def test_rotation_leaves_attention_unchanged():
    B, H, N, d = 1, 2, 130, 128
    g = fa_inputs.make_qkv(B, H, N, d, seed=13)
    signs = fa_inputs.random_signs(d, 14).astype(np.float64)
    m = np.diag(signs) @ fp8.hadamard(d) / math.sqrt(d)
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-15)
    np.testing.assert_allclose(fp8.rotate_unnormalised(g.q, signs) / math.sqrt(d), g.q @ m, atol=1e-13)
    for causal in (False, True):
        o, lse = attention(g.q, g.k, g.v, causal)
        o2, lse2 = attention(g.q @ m, g.k @ m, g.v, causal)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


def test_emulator_reduces_to_exact_attention():
    B, H, N, d = 1, 1, 140, 64
    rng = np.random.default_rng(15)
    codes = [rng.integers(0, 0x7F, (B, H, N, d)).astype(np.uint8) | (rng.integers(0, 2, (B, H, N, d)) << 7).astype(np.uint8)
             for _ in range(3)]
    codes = [np.where((c & 0x7F) == 0x7F, c & 0x80, c).astype(np.uint8) for c in codes]  # no NaN codes
    ones = np.full((B, H, 2), 2.0 ** -7, dtype=np.float32)
    vals = [fp8.e4m3_decode(c) * 2.0 ** -7 for c in codes]
    for causal in (False, True):
        o_emul = fp8.fp8_attention_emulate(*codes, ones, ones, ones, causal, 0.5, round_p=False)
        o_ref, _ = attention(*vals, causal, 0.5)
        np.testing.assert_allclose(o_emul, o_ref, rtol=0, atol=1e-12)
        o_round = fp8.fp8_attention_emulate(*codes, ones, ones, ones, causal, 0.5)
        rel = np.linalg.norm(o_round - o_ref) / np.linalg.norm(o_ref)
        assert 0 < rel < 0.05


def test_quantize_closed_form_block():
    """A hand-built block whose largest magnitude is 7/4: s = 7/4 / 448 =
    2^-8 exactly, so every code is e4m3(y * 256) (division by s, not
    multiplication), ties going to the even code. A second block of zeros
    gets s = 1 and zero codes. Values:
      y = 7/4            -> 448 (0x7E)     y = -1              -> -256 (0xF8)
      y = 17/256         -> 17 lies midway between 16 and 18: even code 16 (0x58)
      y = 19/256         -> 19 lies midway between 18 and 20: even code 20 (0x5A)
      y = 3 * 2^-17      -> 3 * 2^-9 is a subnormal code (0x03)
      y = 2^-18          -> 2^-10 lies midway between 0 and 2^-9: even code 0."""
    ys = [7 / 4, -1.0, 17 / 256, 19 / 256, 3 * 2.0 ** -17, 2.0 ** -18]
    expect = [0x7E, 0xF8, 0x58, 0x5A, 0x03, 0x00]
    x = np.zeros((1, 1, 256, 8))
    x[0, 0, 0, :len(ys)] = ys
    codes, scales = fp8.quantize(x)
    assert scales.dtype == np.float32
    np.testing.assert_array_equal(scales, np.array([[[2.0 ** -8, 1.0]]], dtype=np.float32))
    np.testing.assert_array_equal(codes[0, 0, 0, :len(ys)], np.array(expect, dtype=np.uint8))
    assert not codes[0, 0, 0, len(ys):].any() and not codes[0, 0, 1:].any()
    # rotation: the stored scale carries 1/sqrt(d); d = 4, signs +1, one row
    # x = (1, 0, 0, 0) rotates to y = (1, 1, 1, 1), amax 1, s = 1/448
    x4 = np.zeros((1, 1, 1, 4))
    x4[0, 0, 0, 0] = 1.0
    c4, s4 = fp8.quantize(x4, signs=np.ones(4))
    np.testing.assert_array_equal(c4[0, 0, 0], [0x7E] * 4)
    assert s4[0, 0, 0] == np.float32(1 / 448 / 2)
