"""Benchmark of the exact attention forward on one MI355X.

A step is one attention forward over one batch of synthetic inputs already
resident in HBM, at the headline configuration: bf16, d=128, N=8192, B=2,
H=16 (16k tokens, hidden 2048), non-causal. Throughput is reported in
TFLOP/s with the pages' FLOP convention, 4*B*H*N^2*d (halved for causal).

Prints ONE JSON line (metric, value, roofline, cpu_baseline, ...). Extra
measurements (the sequence-length sweep, FP8) go to stderr, and to a JSON
file when --out is given.

The line also carries the parity of the timed output (the cpu_baseline leg
runs the oracle on whole heads of the same inputs and compares them), the
build provenance, and the headline kernel's MFMA utilisation, clock and HBM
traffic from the rocprofv3 counters recorded in profiles/ for the current
kernel source (null once the source changes).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--fp8] [--bwd] [--decode]
       python bench.py --copy-calibration   (plain copy kernel for PMC scaling)
       python bench.py --gemm-ceiling       (dense bf16 GEMM reference, torch.matmul)
       python bench.py --fwd-only D N B H CAUSAL  (one 16-bit forward shape, for profiling)
       python bench.py --ingest-pmc DIR...  (rocprofv3 counter CSVs -> profiles/ summaries)
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

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
METRIC = "attention fwd TFLOPS + % of MFMA peak, bf16 d=128 N=8k (and fp8)"
HEADLINE = dict(B=2, N=8192, H=16, d=128, causal=False)
DECODE = dict(B=8, Hq=64, Hkv=8, Nk=8192, d=128)  # one new token, GQA 8:1, 8192-key cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_fwd_bf16_d128_n8192.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_attn_fwd_bf16_d128_n8192.json")
KERNEL_SRC = os.path.join(ROOT, "exact_attention_forward_attn_amd", "csrc", "attn_fwd.hip")
# the headline kernel (d=128, 32-key tiles, four waves, non-causal, bf16) as
# rocprofv3 names it: mangled in counter CSVs, demangled in kernel traces
HEADLINE_KERNEL = "fwd_kernel<128, 1, 4, false, __bf16>"
HEADLINE_KERNEL_MANGLED = "10fwd_kernelILi128ELi1ELi4ELb0EDF16bE"
# bf16 parity bounds of the forward (max |O - O_ref|, RMSE(O), max |LSE - LSE_ref|)
PARITY_BOUNDS = {"max_abs": 1e-2, "rmse": 3e-3, "lse_abs": 1e-3}


def compulsory_bytes(B, N, H, d):
    """Q, K, V read and O written once (16-bit), plus the fp32 LSE."""
    return 8.0 * B * N * H * d + 4.0 * B * H * N


def flops(B, N, H, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def device_inputs(B, N, H, d, seed=0, outliers=None):
    import numpy as np
    import torch
    from synth_inputs import make_qkv_f32
    # Draws in float32 then rounds on the device (same RNE rounding as the
    # synth_inputs bf16 cast; timing only needs realistic N(0,1) values).
    q, k, v = make_qkv_f32(B, N, H, d, seed=seed, outliers=outliers)
    return [torch.from_numpy(t).cuda().to(torch.bfloat16) for t in (q, k, v)]


def time_launches(fn, steps, warmup, flush=None):
    """Runs fn warmup + steps times; returns (total_ms, per-launch ms list).
    flush, when given, runs before each timed launch outside its events (it
    evicts the inputs from the on-package cache for the short, HBM-bound
    configurations)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), [a.elapsed_time(b) for a, b in ev]


_FLUSH_BUF = None


def mall_flush():
    """Reads 512 MiB (twice the 256 MB MALL) so the next launch reads HBM.
    (A read, not a write: written lines would still be draining to HBM while
    the timed kernel runs.)"""
    global _FLUSH_BUF
    import torch
    if _FLUSH_BUF is None:
        _FLUSH_BUF = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    _FLUSH_BUF.max()


def headline_inputs(B, N, H, d):
    """The headline's Q, K, V from the shared seeded generator: the device
    tensors (the exact bf16 bits) and the same numbers widened to float64
    on the host, which the cpu_baseline leg feeds to the oracle."""
    import numpy as np
    import torch
    from synth_inputs import make_qkv
    bits, vals = make_qkv(B, N, H, d, seed=0)
    dev = [torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16) for b in bits]
    return dev, vals


def bench_bf16(ea, B, N, H, d, causal, steps, warmup, inputs=None):
    import torch
    q, k, v = inputs if inputs is not None else device_inputs(B, N, H, d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fn = lambda: ea.attn_fwd(q, k, v, o, lse, causal=causal)
    total, per = time_launches(fn, steps, warmup)
    per_ms = sum(per) / len(per)
    tf = flops(B, N, H, d, causal) / (per_ms * 1e-3) / 1e12
    r = {"B": B, "N": N, "H": H, "d": d, "causal": causal, "ms": per_ms, "ms_total": total,
         "ms_median": sorted(per)[len(per) // 2], "ms_min": min(per), "ms_max": max(per),
         "TFLOPS": tf, "frac_peak": tf / PEAK_TFLOPS["bf16"],
         "hbm_GBs": compulsory_bytes(B, N, H, d) / (per_ms * 1e-3) / 1e9}
    if causal:
        r["TFLOPS_exact_causal_count"] = tf * (1 + 1 / N)
    if N <= 1024:
        # HBM-bound range: also time with the inputs evicted from the MALL
        _, perc = time_launches(fn, steps, 1, flush=mall_flush)
        msc = sum(perc) / len(perc)
        r["ms_cold"] = msc
        r["hbm_GBs_cold"] = compulsory_bytes(B, N, H, d) / (msc * 1e-3) / 1e9
        r["hbm_frac_cold"] = r["hbm_GBs_cold"] / PEAK_HBM_GBS
    if inputs is not None:
        # the timed launches' output (every launch writes the same bits)
        r["_out"] = (o, lse)
    return r


def bench_bwd(ea, B, N, H, d, causal, steps, warmup):
    """attn_bwd (pre-pass + dK/dV + dQ kernels) on the forward's own O and LSE.
    FLOPs: the pages' five products per tile pair, 2.5x the forward's count
    (10*B*H*N^2*d, halved for causal); this implementation runs seven (it
    recomputes S and dP in the dQ kernel)."""
    import torch
    q, k, v = device_inputs(B, N, H, d)
    g = torch.Generator(device="cuda").manual_seed(1)
    do = torch.randn(q.shape, device="cuda", generator=g).to(q.dtype)
    o, lse = ea.attention(q, k, v, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fn = lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, causal=causal)
    total, per = time_launches(fn, steps, warmup)
    per_ms = sum(per) / len(per)
    tf = 2.5 * flops(B, N, H, d, causal) / (per_ms * 1e-3) / 1e12
    return {"B": B, "N": N, "H": H, "d": d, "causal": causal, "ms": per_ms, "TFLOPS": tf,
            "frac_peak": tf / PEAK_TFLOPS["bf16"]}


def decode_bytes(B, Hq, Hkv, Nk, d):
    """Compulsory bytes of one decode step: the K/V cache read once, one
    query row per head read and one output row written (16-bit), LSE."""
    return 4.0 * B * Nk * Hkv * d + 4.0 * B * Hq * d + 4.0 * B * Hq


def bench_decode(ea, B, Hq, Hkv, Nk, d, splits, steps, warmup):
    """attn_fwd_ex with one query per sequence against an Nk-key cache
    (grouped heads packed into one tile, split-KV + combine). HBM-bound: the
    cache is evicted from the MALL before each timed launch."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn((B, 1, Hq, d), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((B, Nk, Hkv, d), device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn((B, Nk, Hkv, d), device="cuda", generator=g).to(torch.bfloat16)
    if splits is None:
        splits = ea.attn_num_splits_heuristic(B, Hq, Hkv, 1, Nk, d)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    nb = ea.attn_splitkv_workspace_bytes(splits, B, Hq, d)
    ws = torch.empty(max(nb // 4, 4), dtype=torch.float32, device="cuda")
    fn = lambda: ea.attn_fwd_ex(q, k, v, o, lse, causal=True, num_splits=splits, workspace=ws)
    _, per = time_launches(fn, steps, warmup, flush=mall_flush)
    ms = sum(per) / len(per)
    gbs = decode_bytes(B, Hq, Hkv, Nk, d) / (ms * 1e-3) / 1e9
    return {"B": B, "Hq": Hq, "Hkv": Hkv, "Nk": Nk, "d": d, "splits": splits, "ms": ms, "hbm_GBs": gbs,
            "hbm_frac": gbs / PEAK_HBM_GBS}


def hbm_read_ceiling():
    """Plain streaming reads on this part: torch's float32 sum over 1 GiB
    (read-only) and a 1 GiB device copy (read + write), with the MALL
    flushed first. (A max over bytes is bound by its per-byte compares, not
    by HBM.)"""
    import torch
    x = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    xf = x.view(torch.float32)
    _, per = time_launches(lambda: xf.sum(), 10, 2, flush=mall_flush)
    ms_r = sum(per) / len(per)
    _, per = time_launches(lambda: y.copy_(x), 10, 2, flush=mall_flush)
    ms_c = sum(per) / len(per)
    return {"read_GBs": (1 << 30) / (ms_r * 1e-3) / 1e9, "copy_GBs": 2 * (1 << 30) / (ms_c * 1e-3) / 1e9}


def bench_fp8(ea, B, N, H, d, causal, steps, warmup):
    import torch
    q, k, v = device_inputs(B, N, H, d, outliers={"rate": 1e-3, "factor": 10.0, "kind": "scale"})
    q8, sq = ea.fp8_prepare(q, 128, True, 0)
    k8, sk = ea.fp8_prepare(k, 128, True, 0)
    v8, sv = ea.fp8_prepare(v, 128, False, 0)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fn = lambda: ea.attn_fwd_fp8(q8, k8, v8, o, lse, sq, sk, sv, causal=causal)
    total, per = time_launches(fn, steps, warmup)
    per_ms = sum(per) / len(per)
    tf = flops(B, N, H, d, causal) / (per_ms * 1e-3) / 1e12
    prep = lambda: ea.attn_fp8_prepare(q, q8, sq, 128, True, 0)
    _, pper = time_launches(prep, max(3, steps // 2), 2)
    return {"B": B, "N": N, "H": H, "d": d, "causal": causal, "ms": per_ms, "TFLOPS": tf,
            "frac_peak": tf / PEAK_TFLOPS["fp8"], "prepare_ms_per_tensor": sum(pper) / len(pper)}


def cpu_baseline(vals, out=None, target_s=15.0):
    """Times the float64 oracle on the host on a bounded sample of the
    headline workload: whole (b, h) heads of the headline's own inputs (all
    N query rows, all keys), in order, until ~target_s seconds are spent;
    reports TFLOP/s with the same FLOP count. When `out` holds the timed
    launches' (O, LSE), each oracle head is also compared with the GPU's
    (outside the timed regions of both)."""
    import numpy as np
    from oracle.attention import attention_head
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = HEADLINE
    B, N, H, d = cfg["B"], cfg["N"], cfg["H"], cfg["d"]
    q, k, v = vals
    o_gpu = lse_gpu = None
    if out is not None:
        o_gpu = out[0].float().cpu().numpy()
        lse_gpu = out[1].cpu().numpy()
    heads, el = 0, 0.0
    sq = mx = lmx = 0.0
    n_el = 0
    while heads < B * H and el < target_s:
        b, h = divmod(heads, H)
        t0 = time.perf_counter()
        o_ref, l_ref = attention_head(q[b, :, h], k[b, :, h], v[b, :, h], 1 / math.sqrt(d), cfg["causal"])
        el += time.perf_counter() - t0
        heads += 1
        if o_gpu is not None:
            diff = o_gpu[b, :, h].astype(np.float64) - o_ref
            sq += float(np.sum(diff ** 2))
            n_el += diff.size
            mx = max(mx, float(np.abs(diff).max()))
            lmx = max(lmx, float(np.abs(lse_gpu[b, h].astype(np.float64) - l_ref).max()))
    per_head_flops = flops(1, N, 1, d, cfg["causal"])
    tf = heads * per_head_flops / el / 1e12
    res = {"value": tf, "unit": "TFLOP/s", "cores": int(threads), "cpu_count": os.cpu_count(), "kind": "oracle",
           "sample": f"{heads} of {B * H} (b,h) heads of the headline inputs at N={N}, d={d}, full rows, numpy "
                     f"float64 ({el:.1f} s); rate extrapolates linearly over heads"}
    if o_gpu is not None:
        par = {"heads": heads, "elements": n_el, "max_abs": mx, "rmse": math.sqrt(sq / n_el), "lse_abs": lmx,
               "bounds": PARITY_BOUNDS}
        par["ok"] = all(par[k] <= PARITY_BOUNDS[k] for k in PARITY_BOUNDS)
        res["parity"] = par
    return res


def traffic_entry():
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


def counters_entry():
    """MFMA utilisation and the measured shader clock of the headline kernel,
    from the rocprofv3 counters recorded for the current kernel source (None
    once the source has changed since they were taken)."""
    try:
        c = json.load(open(COUNTERS_FILE))
    except Exception:
        return None
    if c.get("kernel_sha") != kernel_sha():
        return None
    return {k: c[k] for k in ("mfma_busy", "clock_GHz", "mfma_per_tile", "valu_per_tile", "lds_per_tile",
                              "kernel_us", "kernel_sha", "source") if k in c}


def is_headline(kernel_name):
    return HEADLINE_KERNEL in kernel_name or HEADLINE_KERNEL_MANGLED in kernel_name


def ingest_pmc(dirs, out_counters=COUNTERS_FILE, out_traffic=TRAFFIC_FILE, commands=None):
    """Reads rocprofv3 counter CSVs (one directory per --pmc run) and writes
    the headline kernel's counter summary (MFMA busy, clock, instructions per
    tile) and, when FETCH_SIZE / WRITE_SIZE and a copy calibration are among
    them, its HBM traffic, each keyed to the kernel source hash.

    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per XCD);
    clock = GRBM_GUI_ACTIVE per XCD / kernel time (from the same CSV's
    start/end timestamps)."""
    import csv
    import glob
    h = HEADLINE
    simds, xcds = 1024, 8
    tiles = (h["N"] // 32) * (h["N"] // 32) * h["B"] * h["H"]  # 32-key tiles x 32-row waves
    per = {}      # counter -> list of per-dispatch values (headline kernel)
    copy = {}
    dur = []
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows = list(csv.DictReader(open(f)))
            seen = {}
            for r in rows:
                name = r.get("Kernel_Name", "")
                key = (r["Dispatch_Id"], r["Counter_Name"])
                seen[key] = seen.get(key, 0.0) + float(r["Counter_Value"])
                if is_headline(name) and "Start_Timestamp" in r and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    dur.append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3)
            names = {r["Dispatch_Id"]: r.get("Kernel_Name", "") for r in rows}
            for (disp, cname), val in seen.items():
                kname = names[disp]
                if is_headline(kname):
                    per.setdefault(cname, []).append((int(disp), val))
                elif "copyBuffer" in kname:
                    copy.setdefault(cname, []).append(val)
    mean = {}
    for cname, lst in per.items():
        lst.sort()
        vals = [v for _, v in lst[1:]] or [v for _, v in lst]  # the dispatches after the first
        mean[cname] = sum(vals) / len(vals)
    sha = kernel_sha()
    if "GRBM_GUI_ACTIVE" in mean and "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
        cyc = mean["GRBM_GUI_ACTIVE"] / xcds
        out = {"kernel": f"{HEADLINE_KERNEL} (bf16, d=128, N=8192, B=2, H=16, non-causal)", "kernel_sha": sha,
               "source": os.path.relpath(out_counters, ROOT), "counters_per_dispatch": mean,
               "mfma_busy": mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc)}
        if dur:
            us = sorted(dur)[len(dur) // 2]
            out["kernel_us"] = us
            out["clock_GHz"] = cyc / (us * 1e3)
        for cname, key in (("SQ_INSTS_MFMA", "mfma_per_tile"), ("SQ_INSTS_LDS", "lds_per_tile")):
            if cname in mean:
                out[key] = mean[cname] / tiles
        if "SQ_INSTS_VALU" in mean and "SQ_INSTS_MFMA" in mean:
            out["valu_per_tile"] = (mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]) / tiles
        out["tiles_per_dispatch"] = tiles
        out["commands"] = commands or []
        with open(out_counters, "w") as f:
            json.dump(out, f, indent=1)
        print("wrote", out_counters)
    if "FETCH_SIZE" in mean and "WRITE_SIZE" in mean and "FETCH_SIZE" in copy and "WRITE_SIZE" in copy:
        n = 1 << 30
        fs = n / (sum(copy["FETCH_SIZE"]) / len(copy["FETCH_SIZE"]) * 1024)
        ws = n / (sum(copy["WRITE_SIZE"]) / len(copy["WRITE_SIZE"]) * 1024)
        t = {"kernel": f"{HEADLINE_KERNEL} (bf16, d=128, N=8192, B=2, H=16, non-causal)", "kernel_sha": sha,
             "fetch_kib_per_dispatch": mean["FETCH_SIZE"], "write_kib_per_dispatch": mean["WRITE_SIZE"],
             "copy_calibration": {"copy_bytes": n, "fetch_scale": fs, "write_scale": ws},
             "bytes_per_launch": int(mean["FETCH_SIZE"] * 1024 * fs + mean["WRITE_SIZE"] * 1024 * ws),
             "algorithmic_bytes_per_launch": int(compulsory_bytes(h["B"], h["N"], h["H"], h["d"])),
             "commands": commands or []}
        with open(out_traffic, "w") as f:
            json.dump(t, f, indent=1)
        print("wrote", out_traffic)


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def gemm_tflops(M, N, K, zeros=False, reps=20):
    """Dense bf16 GEMM throughput (hipBLASLt via torch.matmul) on N(0,1) (or
    all-zero) operands."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
    if zeros:
        a.zero_()
        b.zero_()
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return 2 * M * N * K / ms / 1e9


def gemm_ceiling():
    """Dense bf16 GEMM (hipBLASLt via torch.matmul) on random N(0,1) and on
    all-zero operands: the practical MFMA ceiling on this part, whose clock
    under load depends on how much the data toggles."""
    import torch
    torch.manual_seed(0)
    for (M, N, K) in [(8192, 8192, 8192), (16384, 16384, 8192)]:
        a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        b = torch.randn(K, N, device="cuda").to(torch.bfloat16)
        for kind, (x, y) in (("random", (a, b)), ("zeros", (torch.zeros_like(a), torch.zeros_like(b)))):
            for _ in range(3):
                x @ y
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            reps = 20
            e0.record()
            for _ in range(reps):
                x @ y
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            print(json.dumps({"gemm": f"{M}x{N}x{K}", "data": kind, "ms": round(ms, 4),
                              "TFLOPS": round(2 * M * N * K / ms / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sweep", action="store_true", help="also time the 16k-token sweep (stderr)")
    ap.add_argument("--fp8", action="store_true", help="also time the FP8 forward (stderr)")
    ap.add_argument("--bwd", action="store_true", help="also time the backward (stderr)")
    ap.add_argument("--decode", action="store_true", help="also time split-KV decode (stderr)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode workload (8 x 64/8 heads, 8192-key cache) and exit")
    ap.add_argument("--bwd-only", action="store_true",
                    help="time only the backward at the headline shape (causal) and exit")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the FP8 forward at the headline shape (128-row blocks + Hadamard) and exit")
    ap.add_argument("--fwd-only", nargs=5, type=int, metavar=("D", "N", "B", "H", "CAUSAL"),
                    help="time only the 16-bit forward at one shape (for profiling) and exit")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--out", default=None, help="write all measurements to this JSON file")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--gemm-ceiling", action="store_true", help="time dense bf16 GEMMs (torch.matmul) and exit")
    ap.add_argument("--ingest-pmc", nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc output directories of the headline kernel (and of "
                         "--copy-calibration) into the kernel-keyed counter / traffic files under profiles/, "
                         "then exit (no GPU needed)")
    ap.add_argument("--ingest-command", action="append", default=[],
                    help="with --ingest-pmc: a command that produced the counters (recorded in the file)")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc, commands=args.ingest_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (attention heads and "
              "batch entries are independent, so they would shard across GPUs with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_ceiling:
        gemm_ceiling()
        return

    import torch
    import exact_attention_forward_attn_amd as ea
    ea.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.fp8_only:
        h = HEADLINE
        r = bench_fp8(ea, h["B"], h["N"], h["H"], h["d"], False, args.steps, args.warmup)
        print(json.dumps({"fp8": r}), flush=True)
        return
    if args.bwd_only:
        h = HEADLINE
        r = bench_bwd(ea, h["B"], h["N"], h["H"], h["d"], True, args.steps, args.warmup)
        print(json.dumps({"bwd": r}), flush=True)
        return

    if args.fwd_only:
        d, N, B, H, causal = args.fwd_only
        r = bench_bf16(ea, B, N, H, d, bool(causal), args.steps, args.warmup)
        r.pop("_out", None)
        print(json.dumps({"fwd": r}), flush=True)
        return

    if args.decode_only:
        r = bench_decode(ea, **DECODE, splits=None, steps=args.steps, warmup=args.warmup)
        print(json.dumps({"decode": r}), flush=True)
        return

    h = HEADLINE
    dev, host_vals = headline_inputs(h["B"], h["N"], h["H"], h["d"])
    head = bench_bf16(ea, h["B"], h["N"], h["H"], h["d"], h["causal"], args.steps, args.warmup, inputs=dev)
    head_out = head.pop("_out")
    # the metric's "(and fp8)": the FP8 forward at the same shape, timed like
    # the headline right after it (prepare excluded, its time per tensor
    # reported beside)
    f8 = bench_fp8(ea, h["B"], h["N"], h["H"], h["d"], h["causal"], args.steps, 2)
    log("headline", json.dumps(head))
    extra = {"headline": head}

    if args.sweep:
        rows = []
        for d, H in ((64, 32), (128, 16), (256, 8)):
            for N in (512, 1024, 2048, 4096, 8192, 16384):
                for causal in (False, True):
                    r = bench_bf16(ea, 16384 // N, N, H, d, causal, max(5, args.steps // 2), 2)
                    log("sweep", json.dumps(r))
                    rows.append(r)
        r = bench_bf16(ea, 1, 32768, 16, 128, True, 5, 2)
        log("long", json.dumps(r))
        rows.append(r)
        extra["sweep"] = rows
    if args.bwd:
        rows = []
        for d, H in ((64, 32), (128, 16), (256, 8)):
            for N in (1024, 4096, 8192):
                for causal in (False, True):
                    r = bench_bwd(ea, 16384 // N, N, H, d, causal, max(5, args.steps // 4), 2)
                    log("bwd", json.dumps(r))
                    rows.append(r)
        extra["bwd"] = rows
    if args.decode:
        rows = []
        for Nk in (1024, 4096, 8192, 32768):
            for splits in (1, None):
                r = bench_decode(ea, 8, 64, 8, Nk, 128, splits, max(10, args.steps), 3)
                log("decode", json.dumps(r))
                rows.append(r)
        for B, Hq, Hkv in ((1, 32, 8), (32, 32, 8), (16, 16, 16), (64, 8, 8)):
            r = bench_decode(ea, B, Hq, Hkv, 8192, 128, None, max(10, args.steps), 3)
            log("decode", json.dumps(r))
            rows.append(r)
        ceil = hbm_read_ceiling()
        log("hbm_read_ceiling", json.dumps(ceil))
        extra["decode"] = rows
        extra["hbm_read_ceiling"] = ceil
    fp8_res = None
    if args.fp8:
        try:
            fp8_res = []
            for N in (1024, 2048, 4096, 8192, 16384):
                r = bench_fp8(ea, 16384 // N, N, 16, 128, False, max(5, args.steps // 2), 2)
                log("fp8", json.dumps(r))
                fp8_res.append(r)
            extra["fp8"] = fp8_res
        except ea.AttnError as e:
            log("fp8 unavailable:", e)
            fp8_res = None

    # the practical dense bf16 ceiling on this machine, same kind of data
    gemm = gemm_tflops(16384, 16384, 8192)
    log("gemm_ceiling", json.dumps({"gemm": "16384x16384x8192 bf16, N(0,1)", "TFLOPS": gemm}))

    # the oracle on the host cores, on whole heads of the same inputs; it also
    # checks the timed launches' output head by head
    cpu = None if args.no_cpu else cpu_baseline(host_vals, head_out)
    parity = cpu.pop("parity", None) if cpu else None
    if cpu:
        log("cpu_baseline", json.dumps(cpu))
        log("parity", json.dumps(parity))
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = None
    build = {"library": ea.load().attn_version().decode(), "rocm": rocm, "torch": torch.__version__,
             "hip_runtime": getattr(torch.version, "hip", None)}

    fl = flops(h["B"], h["N"], h["H"], h["d"], h["causal"])
    achieved = fl / (head["ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(head["TFLOPS"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_total"] / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q, K, V i.i.d. N(0,1) rounded to bf16, seed 0",
        "config": {"workload": "exact attention forward, bf16, d=128, N=8192, B=2, H=16 "
                               "(16k tokens, hidden 2048), non-causal",
                   "global_batch": h["B"], "seq_len": h["N"], "heads": h["H"], "head_dim": h["d"],
                   "causal": h["causal"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic_entry(),
                     "practical_ceiling": {"what": "hipBLASLt dense bf16 GEMM 16384x16384x8192 on N(0,1) "
                                                    "data, same run (the part is power-limited below its "
                                                    "nominal clock)",
                                           "TFLOPS": round(gemm, 1), "frac": round(achieved / gemm, 4)}},
        "cpu_baseline": cpu,
        "parity": parity,
        "build": build,
    }
    line["roofline"]["counters"] = counters_entry()
    line["ms_median"] = round(head["ms_median"], 5)
    # spread of the K timed launches (each bracketed by its own HIP events)
    line["ms_min"] = round(head["ms_min"], 5)
    line["ms_max"] = round(head["ms_max"], 5)
    line["fp8"] = {"value": round(f8["TFLOPS"], 2), "unit": "TFLOP/s", "peak": PEAK_TFLOPS["fp8"],
                   "frac": round(f8["TFLOPS"] / PEAK_TFLOPS["fp8"], 4), "ms": round(f8["ms"], 5),
                   "prepare_ms_per_tensor": round(f8["prepare_ms_per_tensor"], 5),
                   # the three prepare passes (Q, K, V) plus the forward
                   "end_to_end_TFLOPS": round(flops(h["B"], h["N"], h["H"], h["d"], h["causal"])
                                              / ((f8["ms"] + 3 * f8["prepare_ms_per_tensor"]) * 1e-3) / 1e12, 2),
                   "config": "e4m3, power-of-two 128-row block scales + Hadamard on Q and K, inputs N(0,1) with 0.1% of "
                             "entries x10, d=128, N=8192, B=2, H=16, non-causal"}
    if args.out:
        with open(args.out, "w") as f:
            json.dump({"line": line, **extra}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
