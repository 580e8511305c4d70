"""The C-ABI library loads, exports every symbol include/fa.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(fa_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted(
        ["fa_bwd", "fa_fwd", "fa_fwd_fp8", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
         "fa_quant_fp8", "fa_splitkv_splits", "fa_status_string", "fa_version"])


def test_library_exports_all_declared(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(lib.EXPORTS) == set(declared_functions())


def test_version_and_status_strings(lib):
    assert lib.version() >= 100
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.status_string(st) and lib.status_string(st) != "unknown status"
    assert lib.status_string(12345) == "unknown status"


P = 4096  # a 16-byte-aligned fake address; never dereferenced (validation fails first)


def fwd(lib, q=P, k=P, v=P, o=P, lse=None, B=1, H=1, N=8, d=64, causal=0, scale=0.125,
        dtype=0):
    return lib.lib.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


def test_fwd_validation_order(lib):
    assert fwd(lib, q=None) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, o=None) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, B=0) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, N=-3) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, d=80) == lib.FA_ERR_UNSUPPORTED
    assert fwd(lib, dtype=7) == lib.FA_ERR_UNSUPPORTED
    assert fwd(lib, d=96, dtype=lib.FA_FP8_E4M3) == lib.FA_ERR_UNSUPPORTED
    assert fwd(lib, scale=0.0) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, scale=float("nan")) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, scale=float("inf")) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, N=1 << 25, d=64) == lib.FA_ERR_TOO_LARGE
    # a launch of 2^24 workgroups of 256 threads exceeds the 32-bit grid size
    assert fwd(lib, B=1 << 12, H=1 << 12, N=1) == lib.FA_ERR_TOO_LARGE
    assert fwd(lib, B=1 << 12, H=1 << 12, N=1, dtype=lib.FA_FP8_E4M3) == lib.FA_ERR_TOO_LARGE
    assert fwd(lib, B=1 << 11, H=1 << 12, N=129) == lib.FA_ERR_TOO_LARGE
    # just below the limit the size check passes and the next check decides
    assert fwd(lib, B=1 << 12, H=(1 << 12) - 1, N=128, q=P + 2) == lib.FA_ERR_MISALIGNED
    assert fwd(lib, q=P + 2) == lib.FA_ERR_MISALIGNED
    assert fwd(lib, lse=P + 4) == lib.FA_ERR_MISALIGNED
    # earlier checks win over later ones
    assert fwd(lib, q=None, d=80) == lib.FA_ERR_INVALID_ARG
    assert fwd(lib, d=80, scale=-1.0) == lib.FA_ERR_UNSUPPORTED
    assert fwd(lib, scale=-1.0, q=P + 2) == lib.FA_ERR_INVALID_ARG


def test_quant_validation(lib):
    q = lib.lib.fa_quant_fp8
    assert q(None, P, P, 1, 1, 8, 64, 0, None, None) == lib.FA_ERR_INVALID_ARG
    assert q(P, P, None, 1, 1, 8, 64, 0, None, None) == lib.FA_ERR_INVALID_ARG
    assert q(P, P, P, 1, 0, 8, 64, 0, None, None) == lib.FA_ERR_INVALID_ARG
    assert q(P, P, P, 1, 1, 8, 72, 0, None, None) == lib.FA_ERR_UNSUPPORTED
    assert q(P, P, P, 1, 1, 8, 96, 0, P, None) == lib.FA_ERR_UNSUPPORTED   # rotation needs 2^k
    assert q(P, P + 8, P, 1, 1, 8, 64, 0, None, None) == lib.FA_ERR_MISALIGNED
    assert q(P, P, P, 1 << 12, 1 << 12, 8, 64, 0, None, None) == lib.FA_ERR_TOO_LARGE


def test_fwd_fp8_validation(lib):
    f = lib.lib.fa_fwd_fp8
    args = dict(q8=P, k8=P, v8=P, sq=P, sk=P, sv=P, o=P, lse=None, B=1, H=1, N=8, d=128,
                causal=0, scale=0.1)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q8"], a["k8"], a["v8"], a["sq"], a["sk"], a["sv"], a["o"], a["lse"], a["B"],
                 a["H"], a["N"], a["d"], a["causal"], a["scale"], None)

    assert call(v8=None) == lib.FA_ERR_INVALID_ARG
    assert call(sk=None) == lib.FA_ERR_INVALID_ARG
    assert call(H=0) == lib.FA_ERR_INVALID_ARG
    assert call(d=96) == lib.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == lib.FA_ERR_INVALID_ARG
    assert call(sv=P + 4) == lib.FA_ERR_MISALIGNED
    assert call(B=1 << 12, H=1 << 12) == lib.FA_ERR_TOO_LARGE


def test_bwd_validation_order(lib):
    f = lib.lib.fa_bwd
    args = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=1, N=8, d=128,
                causal=0, scale=0.1)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                 a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], None)

    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert call(**{name: None}) == lib.FA_ERR_INVALID_ARG, name
    assert call(B=0) == lib.FA_ERR_INVALID_ARG
    assert call(N=0) == lib.FA_ERR_INVALID_ARG
    assert call(d=80) == lib.FA_ERR_UNSUPPORTED
    assert call(d=512) == lib.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == lib.FA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == lib.FA_ERR_INVALID_ARG
    assert call(N=1 << 24, d=128) == lib.FA_ERR_TOO_LARGE
    assert call(B=1 << 12, H=1 << 12, N=1) == lib.FA_ERR_TOO_LARGE
    # just below the tile-grid limit the size check passes and the next check decides
    assert call(B=1 << 12, H=(1 << 12) - 1, N=128, d=64, dq=P + 2) == lib.FA_ERR_MISALIGNED
    for name in ("q", "o", "lse", "do", "dv"):
        assert call(**{name: P + 4}) == lib.FA_ERR_MISALIGNED, name
    # earlier checks win over later ones
    assert call(lse=None, d=80) == lib.FA_ERR_INVALID_ARG
    assert call(d=80, scale=-1.0) == lib.FA_ERR_UNSUPPORTED
    assert call(scale=-1.0, dq=P + 2) == lib.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("entry", ["fa_fwd_splitkv", "fa_fwd_splitkv_noalloc"])
def test_splitkv_validation_order(lib, entry):
    f = getattr(lib.lib, entry)
    args = dict(q=P, k=P, v=P, o=P, lse=None, B=1, H=1, Nq=1, Nk=100, d=128, causal=0, scale=0.1,
                splits=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                 a["causal"], a["scale"], a["splits"], None)

    for name in ("q", "k", "v", "o"):
        assert call(**{name: None}) == lib.FA_ERR_INVALID_ARG, name
    assert call(Nq=0) == lib.FA_ERR_INVALID_ARG
    assert call(Nk=0) == lib.FA_ERR_INVALID_ARG
    assert call(splits=-1) == lib.FA_ERR_INVALID_ARG
    assert call(causal=1, Nq=101) == lib.FA_ERR_INVALID_ARG
    assert call(d=256) == lib.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == lib.FA_ERR_INVALID_ARG
    assert call(Nk=1 << 24) == lib.FA_ERR_TOO_LARGE
    assert call(Nq=1 << 23, Nk=1 << 23) == lib.FA_ERR_TOO_LARGE
    # decode, one split: 2^26 one-wave workgroups = 2^32 work-items
    assert call(B=1 << 13, H=1 << 13, Nk=64) == lib.FA_ERR_TOO_LARGE
    # just below the limit the size check passes and the next check decides
    # (the allocation-free entry's scratch cannot hold those 2^26 partial rows)
    assert call(B=1 << 13, H=(1 << 13) - 1, Nk=64, o=P + 8) == (
        lib.FA_ERR_MISALIGNED if entry == "fa_fwd_splitkv" else lib.FA_ERR_SCRATCH_LIMIT)
    assert call(o=P + 8) == lib.FA_ERR_MISALIGNED
    assert call(lse=P + 4) == lib.FA_ERR_MISALIGNED
    assert call(q=None, d=256) == lib.FA_ERR_INVALID_ARG
    assert call(causal=1, Nq=101, d=256) == lib.FA_ERR_INVALID_ARG
    assert call(d=256, scale=-1.0) == lib.FA_ERR_UNSUPPORTED


def test_splitkv_noalloc_scratch_limit(lib):
    """The allocation-free entry point refuses calls whose partial results
    (splits * B*H*Nq * (d+1) floats) exceed its fixed scratch array, after
    the size checks and before the alignment check; fa_fwd_splitkv takes
    the same sizes (its scratch comes from the pool)."""
    f = lib.lib.fa_fwd_splitkv_noalloc
    g = lib.lib.fa_fwd_splitkv
    limit = lib.NOALLOC_SCRATCH_BYTES

    def need(B, H, Nq, Nk, d, splits):
        return lib.splitkv_splits(B, H, Nq, Nk, splits) * B * H * Nq * (d + 1) * 4

    # decode B=4 H=16 Nq=1 Nk=16384 d=128 (automatic splits) fits
    assert need(4, 16, 1, 16384, 128, 0) <= limit
    assert f(P, P, P, P + 8, None, 4, 16, 1, 16384, 128, 0, 0.1, 0, None) == lib.FA_ERR_MISALIGNED
    # 2048 queries x 256 heads x 4 splits x 129 floats: 1 GiB > 32 MiB
    assert need(16, 16, 2048, 8192, 128, 4) > limit
    assert f(P, P, P, P, None, 16, 16, 2048, 8192, 128, 0, 0.1, 4, None) == lib.FA_ERR_SCRATCH_LIMIT
    assert f(P, P, P, P + 8, None, 16, 16, 2048, 8192, 128, 0, 0.1, 4, None) == \
        lib.FA_ERR_SCRATCH_LIMIT
    assert g(P, P, P, P + 8, None, 16, 16, 2048, 8192, 128, 0, 0.1, 4, None) == lib.FA_ERR_MISALIGNED
    # the exact boundary: need == limit passes, one more query row does not
    B, H, d, Nk, sp = 1, 1, 127, 1 << 14, 1
    rows = limit // (4 * (d + 1))                 # 65536 rows of 128 floats
    assert need(B, H, rows, Nk, 96, sp) <= limit  # d = 96: (96+1) floats per row
    assert f(P, P, P, P + 8, None, 1, 1, rows, Nk, 96, 0, 0.1, 1, None) == lib.FA_ERR_MISALIGNED
    rows97 = limit // (4 * 97) + 1
    assert f(P, P, P, P, None, 1, 1, rows97, Nk, 96, 0, 0.1, 1, None) == lib.FA_ERR_SCRATCH_LIMIT
    assert f(P, P, P, P + 8, None, 1, 1, rows97 - 1, Nk, 96, 0, 0.1, 1, None) == \
        lib.FA_ERR_MISALIGNED


def test_splitkv_split_count(lib):
    """Host logic: decode (Nq <= 32) splits into two rounds of workgroups with
    at least two 64-key tiles each; longer queries split only below a round
    of 256 query-tile workgroups: about 512 items with at least eight tiles
    per split, or, causal, about 768 items, at most 8 splits, at least four
    tiles each; never more splits than tiles, and no empty split."""
    s = lib.splitkv_splits
    assert s(1, 1, 1, 1) == 1
    assert s(1, 1, 1, 64 * 10) == 5              # tiles / 2
    assert s(4, 16, 1, 16384) == 16              # 1024 / 64 workgroups per split
    assert s(64, 64, 1, 16384) == 1              # enough heads already
    assert s(1, 1, 1, 64 * 10, 64) == 10         # capped at the tile count
    assert s(1, 1, 1, 64 * 10, 3) == 3
    assert s(1, 1, 1, 64 * 10, 4) == 4           # 3 tiles per split, 4 splits
    assert s(1, 1, 1, 64 * 10, 6) == 5           # 2 tiles per split: 5 non-empty
    assert s(1, 2, 200, 200, 0) == 1             # 4 tiles: too few to split
    assert s(1, 4, 4096, 4096) == 4              # 128 workgroups -> 4 splits of 16 tiles
    assert s(4, 16, 2048, 2048) == 1             # 1024 workgroups: no split
    assert s(1, 4, 4096, 4096, 0, True) == 6     # causal, 128 query tiles: ~768 items
    assert s(1, 3, 8192, 8192, 0, True) == 4     # 192 query tiles
    assert s(1, 7, 4096, 4096, 0, True) == 3     # 224 query tiles
    assert s(1, 1, 2048, 2048, 0, True) == 8     # 16 query tiles: at most 8 splits
    assert s(1, 1, 512, 512, 0, True) == 2       # 8 key tiles, >= 4 per split
    assert s(4, 16, 2048, 2048, 0, True) == 1    # a round already
    assert s(1, 4, 4096, 4096, 5, True) == 5     # requested counts ignore the mask
    with pytest.raises(lib.FAError):
        s(0, 1, 1, 1)
    for B, H, Nq, Nk, req in ((1, 1, 1, 777, 0), (2, 3, 40, 5000, 0), (1, 1, 1, 6400, 33)):
        n = s(B, H, Nq, Nk, req)
        tiles = -(-Nk // 64)
        tps = -(-tiles // n)
        assert 1 <= n <= tiles and (n - 1) * tps < tiles


def test_python_wrapper_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lib.fwd(x, x, x)
    with pytest.raises(TypeError):
        lib.fwd(x.float(), x, x)
    lse = torch.zeros(1, 1, 4)
    with pytest.raises(ValueError):
        lib.bwd(x, x, x, x, lse, x)
