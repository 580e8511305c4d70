#!/usr/bin/env python3
"""Attention forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
                    [--extras-only TEXT]

One step is one fa_fwd call (bf16, non-causal) over the workload
B=1, H=16, N=16384, d=128 (the longest row of the sequence sweep at 16k
tokens, hidden 2048) with inputs resident in HBM. The metric is attention
TFLOP/s = 4*B*H*N^2*d / time (halved for causal masks). Rank 0 prints one JSON
line. The extra measurements (B=4 H=16 N=2048, causal, the sequence and
head-dimension sweeps, the FP8 path, the backward pass) ride along in "extra";
"roofline_fp8" is the e4m3 kernel on the FP8 workload; the CPU baseline times
the float64 oracle on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6   # TFLOP/s, dense MFMA, MI355X published
PEAK_FP8 = 5033.2    # TFLOP/s, dense MFMA, MI355X published
WORKLOAD = dict(B=1, H=16, N=16384, d=128, causal=False)
KERNEL_SOURCE = os.path.join(ROOT, "exact_attention_14_amd", "csrc", "fa_fwd_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_B1H16N16384d128.json")
FP8_WORKLOAD = dict(B=2, H=16, N=8192, d=128, causal=False)
FP8_KERNEL_SOURCE = os.path.join(ROOT, "exact_attention_14_amd", "csrc", "fa_fp8.hip")
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_fp8_B2H16N8192d128.json")


PEAK_HBM = 8e12      # B/s, MI355X published
RIDGE_BF16 = PEAK_BF16 * 1e12 / PEAK_HBM  # flop per byte where the two rooflines meet


def algorithmic_bytes(B, H, N, d, e_in):
    """Q, K, V read once (e_in bytes per element), O written in bf16, LSE in fp32."""
    return B * H * N * (3 * d * e_in + 2 * d + 4)


def flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def settle(fn, warmup, min_warm_s=0.3):
    """Runs fn() at least `warmup` times and for at least `min_warm_s`
    seconds (synchronising every 16 calls); returns the seconds spent. After
    the idle spell of generating inputs on the host the GPU clock needs some
    tens of milliseconds of load to ramp back up."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_warm_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_calls(fn, steps, warmup, min_warm_s=0.3):
    """Average duration (ms) of fn() over `steps` calls, HIP events on the
    current stream (the stream the library launches on). The untimed warm-up
    runs at least `warmup` calls and at least `min_warm_s` seconds: after the
    idle spell of generating inputs on the host the GPU clock needs some tens
    of milliseconds to ramp back up."""
    import torch
    settle(fn, warmup, min_warm_s)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def device_qkv(B, H, N, d, seed, dist="normal"):
    import fa_inputs
    g = fa_inputs.make_qkv(B, H, N, d, seed, dist)
    return tuple(fa_inputs.to_torch_bf16(x, "cuda") for x in (g.q_bits, g.k_bits, g.v_bits))


def extras(fa, only=None):
    """The extra measurements; `only` keeps those whose name contains it."""
    import torch
    import fa_inputs
    out = []
    want = lambda name: only is None or only in name

    def run(name, B, H, N, d, causal, seed, dtype=fa.FA_BF16, steps=100):
        if not want(name):
            return
        q, k, v = device_qkv(B, H, N, d, seed)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        ms = time_calls(lambda: fa.fwd(q, k, v, causal=causal, dtype=dtype, out=o, lse=lse),
                        steps, 3)
        tf = flops(B, H, N, d, causal) / (ms * 1e-3) / 1e12
        peak = PEAK_BF16 if dtype == fa.FA_BF16 else PEAK_FP8
        gbps = algorithmic_bytes(B, H, N, d, 2) / (ms * 1e-3) / 1e9
        out.append({"name": name, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                    "dtype": "bf16" if dtype == fa.FA_BF16 else "fp8_e4m3",
                    "ms": round(ms, 4), "tflops": round(tf, 1),
                    "pct_peak": round(100 * tf / peak, 1),
                    "gbps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / (PEAK_HBM / 1e9), 1),
                    "bound": "hbm" if flops(B, H, N, d, causal) / algorithmic_bytes(B, H, N, d, 2)
                             < RIDGE_BF16 else "mfma"})
        del q, k, v, o, lse

    def run_bwd(name, B, H, N, d, causal, seed, steps=50):
        if not want(name):
            return
        q, k, v = device_qkv(B, H, N, d, seed)
        do_bits, _ = fa_inputs.make_grad(B, H, N, d, seed + fa_inputs.SEEDS["grad_offset"])
        do = fa_inputs.to_torch_bf16(do_bits, "cuda")
        o, lse = fa.fwd(q, k, v, causal=causal)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ms = time_calls(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, dq=dq, dk=dk, dv=dv),
                        steps, 3)
        # five N x N x d products (S, dP, dV, dK, dQ) = 2.5 times the forward's two
        tf = 2.5 * flops(B, H, N, d, causal) / (ms * 1e-3) / 1e12
        out.append({"name": name, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                    "dtype": "bf16", "ms": round(ms, 4), "tflops": round(tf, 1),
                    "pct_peak": round(100 * tf / PEAK_BF16, 1)})
        del q, k, v, do, o, lse, dq, dk, dv

    def run_split(name, B, H, Nq, Nk, d, causal, seed, steps=100):
        if not want(name):
            return
        gk = fa_inputs.make_qkv(B, H, Nk, d, seed)
        gq = fa_inputs.make_qkv(B, H, Nq, d, seed + 50000)
        q = fa_inputs.to_torch_bf16(gq.q_bits, "cuda")
        k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (gk.k_bits, gk.v_bits))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
        ms = time_calls(lambda: fa.fwd_splitkv(q, k, v, causal=causal, out=o, lse=lse), steps, 3)
        if causal:  # query i sees i + Nk - Nq + 1 keys
            pairs = Nq * (Nk - Nq) + Nq * (Nq + 1) / 2
        else:
            pairs = Nq * Nk
        fl = 4.0 * B * H * pairs * d
        nbytes = B * H * (2 * Nk * d * 2 + 2 * Nq * d * 2 + 4 * Nq)
        rec = {"name": name, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d, "causal": causal,
               "dtype": "bf16", "splits": fa.splitkv_splits(B, H, Nq, Nk, causal=causal), "ms": round(ms, 4),
               "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
               "pct_peak": round(100 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16, 1),
               "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / PEAK_HBM, 1),
               "bound": "hbm" if fl / nbytes < RIDGE_BF16 else "mfma"}
        out.append(rec)
        del q, k, v, o, lse

    def run_cold(name, B, H, N, d, causal, seed, trials=21):
        """Secondary, cold-cache timing: a 1 GiB device write before each
        call evicts L2 and the MALL, so Q, K and V come from HBM; the median
        of `trials` single calls, each bracketed by HIP events after the
        write."""
        if not want(name):
            return
        q, k, v = device_qkv(B, H, N, d, seed)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        call = lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
        settle(call, 3)
        times = []
        for i in range(trials):
            scrub.fill_(i & 0xFF)
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            call()
            end.record()
            torch.cuda.synchronize()
            times.append(start.elapsed_time(end))
        ms = sorted(times)[len(times) // 2]
        tf = flops(B, H, N, d, causal) / (ms * 1e-3) / 1e12
        out.append({"name": name, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                    "dtype": "bf16", "cache": "cold: 1 GiB write before each call, median of "
                    f"{trials}", "ms": round(ms, 4), "tflops": round(tf, 1),
                    "pct_peak": round(100 * tf / PEAK_BF16, 1)})
        del q, k, v, o, lse, scrub

    for causal in (False, True):
        run_cold("cold-cache mid", 4, 16, 2048, 128, causal, fa_inputs.SEEDS["mid"])
    run_cold("cold-cache headline", 1, 16, 16384, 128, False, fa_inputs.SEEDS["seq_sweep_base"] + 5)

    # decode against a 16k-token cache, one and sixteen new queries per (b, h)
    for causal in (False, True):
        run_split("decode split-KV (fa_fwd_splitkv)", 4, 16, 1, 16384, 128, causal, 13000)
    run_split("decode split-KV (fa_fwd_splitkv)", 1, 16, 16, 65536, 128, True, 13001)
    # few heads: the key axis fills the compute units that B*H*N/128 cannot
    run_split("few heads split-KV (fa_fwd_splitkv)", 1, 4, 4096, 4096, 128, True, 13002)
    run_split("few heads split-KV (fa_fwd_splitkv)", 1, 2, 8192, 8192, 128, False, 13003)

    for causal in (False, True):
        run_bwd("backward (fa_bwd)", 4, 16, 2048, 128, causal, fa_inputs.SEEDS["mid"])
    for i, d in enumerate((64, 96, 128, 256)):
        run_bwd("backward head-dim sweep (fa_bwd)", 2, 16, 8192, d, True,
                fa_inputs.SEEDS["dim_sweep_base"] + i, steps=20)

    # The practical matrix-core ceiling of this part: a plain library GEMM
    # (hipBLASLt through torch) under the same power limit, bf16 and e4m3.
    if want("gemm ceiling"):
        n = 8192
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        ms = time_calls(lambda: torch.matmul(a, b), 20, 3)
        out.append({"name": "gemm ceiling bf16 (torch.matmul 8192^3)", "ms": round(ms, 4),
                    "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1),
                    "pct_peak": round(100 * 2.0 * n ** 3 / (ms * 1e-3) / 1e12 / PEAK_BF16, 1)})
        try:
            a8 = a.to(torch.float8_e4m3fn)
            b8 = b.t().contiguous().to(torch.float8_e4m3fn).t()
            one = torch.ones((), device="cuda")
            ms = time_calls(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                     out_dtype=torch.bfloat16), 20, 3)
            out.append({"name": "gemm ceiling e4m3 (torch._scaled_mm 8192^3)", "ms": round(ms, 4),
                        "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1),
                        "pct_peak": round(100 * 2.0 * n ** 3 / (ms * 1e-3) / 1e12 / PEAK_FP8, 1)})
        except Exception as e:  # the fp8 GEMM may be missing from this build of torch
            out.append({"name": "gemm ceiling e4m3 (torch._scaled_mm 8192^3)",
                        "error": str(e)[:200]})
        del a, b

    run("mid non-causal", 4, 16, 2048, 128, False, fa_inputs.SEEDS["mid"])
    run("mid causal", 4, 16, 2048, 128, True, fa_inputs.SEEDS["mid"])
    for N in (512, 1024, 2048, 4096, 8192, 16384):
        seed = fa_inputs.SEEDS["seq_sweep_base"] + int(math.log2(N // 512))
        for causal in (False, True):
            run("seq sweep", 16384 // N, 16, N, 128, causal, seed)
    for i, d in enumerate((64, 96, 128, 256)):
        run("head-dim sweep", 2, 16, 8192, d, True, fa_inputs.SEEDS["dim_sweep_base"] + i)

    return out


def fp8_measurements(fa, only=None, steps=200):
    """The FP8 workload (B=2 H=16 N=8192 d=128 non-causal, outliers replacing
    0.1% of entries, 128-row block scales with the random-sign Hadamard
    rotation of Q and K): the e4m3 kernel alone (its roofline object against
    the fp8 peak), the end-to-end path, the quantiser. Returns
    (roofline_fp8, extra entries)."""
    import torch
    import fa_inputs
    out = []
    B, H, N, d = (FP8_WORKLOAD[x] for x in ("B", "H", "N", "d"))
    g = fa_inputs.make_qkv(B, H, N, d, fa_inputs.SEEDS["fp8"], "outlier_replace")
    q, k, v = (fa_inputs.to_torch_bf16(x, "cuda") for x in (g.q_bits, g.k_bits, g.v_bits))
    signs = torch.from_numpy(fa_inputs.random_signs(d, fa_inputs.SEEDS["fp8_signs"])).cuda()
    q8, sq = fa.quant_fp8(q, signs=signs)
    k8, sk = fa.quant_fp8(k, signs=signs)
    v8, sv = fa.quant_fp8(v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    f = flops(B, H, N, d, False)
    ms = time_calls(lambda: fa.fwd_fp8(q8, k8, v8, sq, sk, sv, out=o, lse=lse), steps, 3)
    achieved = f / (ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8, 4),
            "traffic": traffic_record(FP8_TRAFFIC_FILE, FP8_KERNEL_SOURCE),
            "kernel": "fwd_fp8_kernel<128,false,4,false>", "kernel_ms": round(ms, 5),
            "workload": f"fa_fwd_fp8 B={B} H={H} N={N} d={d} e4m3 non-causal, block scales + "
                        "Hadamard, outliers replacing 0.1% of entries",
            "x_bf16_same_shape": None}
    out.append({"name": "fp8 kernel (fa_fwd_fp8)", "B": B, "H": H, "N": N, "d": d,
                "causal": False, "dtype": "fp8_e4m3", "ms": round(ms, 4),
                "tflops": round(achieved, 1), "pct_peak": round(100 * achieved / PEAK_FP8, 1)})
    # the bf16 kernel on the same shape, for the FP8/bf16 ratio
    ms_bf = time_calls(lambda: fa.fwd(q, k, v, out=o, lse=lse), steps, 3)
    roof["x_bf16_same_shape"] = round(ms_bf / ms, 3)
    if only is None or "fp8" in only:
        ms = time_calls(lambda: fa.fwd(q, k, v, dtype=fa.FA_FP8_E4M3, out=o, lse=lse), 100, 3)
        out.append({"name": "fp8 end to end (fa_fwd, quantisation included)", "B": B, "H": H,
                    "N": N, "d": d, "causal": False, "dtype": "fp8_e4m3", "ms": round(ms, 4),
                    "tflops": round(f / (ms * 1e-3) / 1e12, 1),
                    "pct_peak": round(100 * f / (ms * 1e-3) / 1e12 / PEAK_FP8, 1)})
        ms = time_calls(lambda: fa.quant_fp8(q, signs=signs, out=q8, scales=sq), 100, 3)
        nbytes = B * H * N * d * 3 + B * H * ((N + 127) // 128) * 4
        out.append({"name": "fp8 quantiser with rotation (fa_quant_fp8, one tensor)", "B": B,
                    "H": H, "N": N, "d": d, "ms": round(ms, 4),
                    "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "pct_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 8e12, 1)})
    del q, k, v, q8, k8, v8, o, lse
    return roof, out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(budget_s=12.0):
    """Times the float64 oracle on whole heads of the headline workload until
    about `budget_s` seconds of CPU work have run."""
    import fa_inputs
    from oracle import attention
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    B, H, N, d = WORKLOAD["B"], WORKLOAD["H"], WORKLOAD["N"], WORKLOAD["d"]
    g = fa_inputs.make_qkv(1, 2, N, d, fa_inputs.SEEDS["seq_sweep_base"] + 5)
    q, k, v = g.q, g.k, g.v
    heads = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        h = heads % 2
        attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], WORKLOAD["causal"])
        heads += 1
    dt = time.perf_counter() - t0
    tf = heads * flops(1, 1, N, d, WORKLOAD["causal"]) / dt / 1e12
    return {"value": round(tf, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{heads} (batch, head) slices of N={N} d={d} non-causal (the headline "
                      f"workload has {B * H}), float64 NumPy with S and P materialised, "
                      f"{dt:.1f} s"}


def traffic_record(path=TRAFFIC_FILE, source=KERNEL_SOURCE):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(source):
        return None
    return rec.get("traffic_bytes")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The default run times about 0.4 s of the headline (1.8 ms per step);
    # the warm-up runs at least this many steps and at least 0.3 s.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 roofline object")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only the FP8 roofline object (e4m3 kernel on the FP8 workload, "
                         "--steps timed calls), printed as one JSON line")
    ap.add_argument("--extras-only", default=None, metavar="TEXT",
                    help="run only the extra measurements whose name contains TEXT")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); every (batch, head) "
              "is independent, so several GPUs would each run this kernel on their share.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_14_amd as fa
    import fa_inputs

    if args.copy_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.fp8_only:
        roof, _ = fp8_measurements(fa, "", steps=args.steps)
        print(json.dumps({"roofline_fp8": roof}), flush=True)
        return

    B, H, N, d, causal = (WORKLOAD[x] for x in ("B", "H", "N", "d", "causal"))
    q, k, v = device_qkv(B, H, N, d, fa_inputs.SEEDS["seq_sweep_base"] + 5)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    step = lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
    # untimed: at least --warmup steps and at least 0.3 s (clock settling)
    warm_s = settle(step, args.warmup)
    # timed: exactly --steps steps, bracketed by synchronisations; the events
    # sit on torch's current stream, which is the stream the library launches on
    # Events also split the timed steps into (up to) five equal trials, whose
    # per-step means give the spread; they add no synchronisation.
    n_tr = min(5, args.steps)
    bounds = [round(i * args.steps / n_tr) for i in range(n_tr + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_tr + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for tr in range(n_tr):
        for _ in range(bounds[tr + 1] - bounds[tr]):
            step()
        evs[tr + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    trial_ms = [evs[i].elapsed_time(evs[i + 1]) / (bounds[i + 1] - bounds[i])
                for i in range(n_tr) if bounds[i + 1] > bounds[i]]
    ms_per_step = wall * 1e3 / args.steps
    f = flops(B, H, N, d, causal)
    value = f / (ms_per_step * 1e-3) / 1e12
    achieved = f / (kernel_ms * 1e-3) / 1e12
    rec = {
        "metric": "attention fwd TFLOP/s (4BHN\u00b2d, causal halved) + % of MFMA peak, bf16 & fp8",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"attention fwd B={B} H={H} N={N} d={d} bf16 non-causal "
                               "(sequence sweep at 16k tokens, hidden 2048)",
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": d,
                   "causal": causal, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4),
                     "traffic": traffic_record(), "kernel": "fwd_bf16_kernel<128,false,4>",
                     "kernel_ms": round(kernel_ms, 5),
                     "kernel_ms_trials": [round(x, 5) for x in trial_ms],
                     "kernel_ms_median": round(sorted(trial_ms)[len(trial_ms) // 2], 5)},
    }
    del q, k, v, o, lse
    fp8_extra = []
    if not args.no_fp8:
        rec["roofline_fp8"], fp8_extra = fp8_measurements(
            fa, "" if args.no_extras else args.extras_only)
    if not args.no_extras:
        rec["extra"] = extras(fa, args.extras_only) + fp8_extra
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
