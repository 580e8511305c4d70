"""Checks on the compiler's gfx950 output for the attention kernels (CPU only:
hipcc cross-compiles to assembly text, nothing runs).

No matrix-core instruction may be issued inside an exec-masked region. The
32x32 products combine operands from all 64 lanes; run under a partial exec
mask (after the compiler moved the last tile's products into a branch that
only some lanes take) they gave wrong outputs. The kernels' epilogues are
branch-free for this reason, and this test keeps it so.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from exact_attention_14_amd import build as fa_build

KERNELS = ("fa_fwd_bf16.hip", "fa_fp8.hip", "fa_bwd_bf16.hip", "fa_fwd_split.hip")


def _hipcc():
    try:
        return fa_build.hipcc()
    except RuntimeError:
        return None


def device_asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [_hipcc(), *fa_build.COMMON, *fa_build.DEVICE_FLAGS, "--cuda-device-only", "-S",
           os.path.join(fa_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read().split("\n")


def mfma_under_exec_mask(lines):
    """{kernel: count} of MFMAs between an exec save (s_and_saveexec /
    s_andn2_saveexec) and the restore of exec, per kernel."""
    bad, kernels, kern, masked = {}, [], None, False
    for line in lines:
        m = re.match(r"^(_Z\w*(?:fwd|bwd)_\w*kernel\w*):", line)
        if m:
            kern, masked = m.group(1), False
            kernels.append(kern)
            continue
        if kern is None:
            continue
        s = line.strip()
        if s.startswith(".Lfunc_end"):
            kern = None
        elif s.startswith(("s_and_saveexec", "s_andn2_saveexec")):
            masked = True
        elif re.match(r"s_(or|mov)_b64 exec", s):
            masked = False
        elif s.startswith("v_mfma") and masked:
            bad[kern] = bad.get(kern, 0) + 1
    return kernels, bad


def test_detector_flags_a_masked_mfma():
    text = ["_ZN2fa3fwd_x_kernelE:", "\ts_and_saveexec_b64 s[0:1], vcc",
            "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
            "\ts_or_b64 exec, exec, s[0:1]", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
            ".Lfunc_end0:"]
    kernels, bad = mfma_under_exec_mask(text)
    assert kernels == ["_ZN2fa3fwd_x_kernelE"] and bad == {"_ZN2fa3fwd_x_kernelE": 1}


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_no_mfma_under_partial_exec(src, tmp_path):
    kernels, bad = mfma_under_exec_mask(device_asm(src, str(tmp_path)))
    assert len(kernels) >= 6, kernels
    assert bad == {}, f"MFMAs inside exec-masked regions: {bad}"


def kernel_resources(lines):
    """{kernel: (registers incl. accumulation registers, scratch bytes)} from
    the code-object descriptors in the assembly."""
    out, name, regs, scratch = {}, None, None, None
    for line in lines:
        s = line.strip()
        if s.startswith(".amdhsa_kernel "):
            name, regs, scratch = s.split()[1], None, None
        elif name and s.startswith(".amdhsa_next_free_vgpr "):
            regs = int(s.split()[1])
        elif name and s.startswith(".amdhsa_private_segment_fixed_size "):
            scratch = int(s.split()[1])
        elif name and s.startswith(".end_amdhsa_kernel"):
            out[name] = (regs, scratch)
            name = None
    return out


def intended_waves(name):
    """Waves per SIMD the attention kernels are compiled for: one at d = 256,
    three at d = 64 (not the split-KV kernel), two otherwise."""
    d = int(re.search(r"kernelILi(\d+)E", name).group(1))
    if d == 256:
        return 1
    if d == 64 and "fwd_split_kernel" not in name:
        return 3
    return 2


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_register_budget_and_no_spills(src, tmp_path):
    """Every attention kernel fits the register budget of its occupancy (512
    registers per lane shared by the waves of a SIMD, allocated in blocks of
    8) and spills nothing to scratch."""
    res = kernel_resources(device_asm(src, str(tmp_path)))
    main = {k: v for k, v in res.items()
            if re.search(r"(fwd_bf16|fwd_fp8|bwd_dkdv|bwd_dq|fwd_split)_kernel", k)}
    assert len(main) >= 6, sorted(res)
    for name, (regs, scratch) in main.items():
        waves = intended_waves(name)
        budget = (512 // waves) // 8 * 8
        assert scratch == 0, (name, scratch)
        assert (regs + 7) // 8 * 8 <= budget, (name, regs, waves)
