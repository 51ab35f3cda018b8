"""Benchmark of the exact-attention hot path on one MI355X.

One step = one fused causal prefill (B=1, H=32, N=8192, d=128, bf16, K
doubled) followed by one split-KV decode (B=16, H=32, one query row, a
32768-key bf16 cache, d=128, 64 splits), both on the same HIP stream, with
inputs already resident in HBM. After W warm-up steps, exactly K steps are
timed between two device synchronisations; HIP events recorded on the launch
stream around each call give the per-call kernel time.

Prints one JSON line: `value` is the prefill's attention-forward throughput
(algorithmic FLOPs / average prefill time), with a `roofline` entry for the
fused kernel, the decode's HBM rate in `decode`, and the CPU oracle's
throughput on a bounded sample of the prefill workload in `cpu_baseline`.
After the timed steps, the same decode over a paged cache (`paged_decode`),
the backward pass on the prefill workload (`backward`), the other configurations
of the plan (`reported_configs`: fp32 N=256, bf16 N=1024 d=64, 16K, and the
three-kernel ablation), the FP8 forward on the prefill workload (`fp8_prefill`)
and a 128K-token prefill (`long_prefill`) are timed on their own and reported
apart from `value`.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (% bf16 MFMA peak) at N=8K d=128; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2516.6    # 256 CU x 4096 bf16 FLOP/clk/CU x 2.4 GHz (the published 2.5 PFLOP/s dense)
PEAK_HBM_GBPS = 8000.0       # published HBM3E bandwidth
PEAK_FP8_TFLOPS = 5033.2     # dense FP8 MFMA: twice the bf16 rate (the published 5.0 PFLOP/s)
PEAK_FP32_TFLOPS = 157.3     # published fp32 rate (the fp32 forward is a VALU kernel; reported for information)
PREFILL = "bf16_h32_n8192_d128_causal_k2"
DECODE = "decode_b16h32_l32768_d128"
LONG = "bf16_b4h32_n131072_d128_causal"
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_fwd_bf16_n8192.json")
FWD_SOURCES = [os.path.join(ROOT, "exact_io_aware_74_amd", "csrc", f) for f in ("fa_fwd_bf16.hip", "fa_device.h")]


def fwd_source_digest() -> str:
    h = hashlib.sha256()
    for p in FWD_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(launches_per_record: int = 1):
    """HBM bytes per fused-kernel launch from the committed counter record, if it
    was taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    rec = json.load(open(TRAFFIC_RECORD))
    if rec.get("kernel_source_digest") != fwd_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def warm_up(torch, fn, min_ms: float = 30.0, min_calls: int = 2):
    """Untimed calls of fn until about min_ms of GPU time has passed: after a change
    of load the clock takes a few tens of milliseconds to settle."""
    import time
    t0, n = time.perf_counter(), 0
    while n < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        torch.cuda.synchronize()
        n += 1


def cpu_baseline(w, target_s: float):
    """The oracle, untuned, on whole heads of the prefill workload until about target_s seconds."""
    import numpy as np

    import oracle
    import seeded_inputs as si
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        cores = len(os.sched_getaffinity(0))
    heads, elapsed, flops = 0, 0.0, 0
    while elapsed < target_s and heads < w.H:
        h = heads
        q, k, v = (si.as_float64(si.tensor_slice(w, t, 0, h), w.dtype)[None, None] for t in ("q", "k", "v"))
        t0 = time.perf_counter()
        O, _ = oracle.attention(q, k, v, w.causal, w.scale)
        elapsed += time.perf_counter() - t0
        assert np.isfinite(O).all()
        flops += oracle.attention_flops(1, 1, w.N, w.d, w.causal)
        heads += 1
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"{heads} of {w.H} heads of the N=8192 d=128 causal prefill (all rows), fp64 numpy, "
                      f"{elapsed:.1f} s"}


def backward_leg(fa, torch, si, w, q, k, v, o, lse, steps):
    """Backward pass (recompute method) at the prefill workload, timed with HIP
    events on the launch stream; reported apart from the step's value."""
    dout = torch.from_numpy(si.upstream_grad(w.wid, w.B, w.H, w.N, w.d, "bf16").view("int16")).view(
        torch.bfloat16).to(q.device)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N) // 4, dtype=torch.float32, device=q.device)
    fa.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    stream = torch.cuda.current_stream(q.device)
    warm_up(torch, lambda: fa.bwd(q, k, v, o, dout, lse, causal=True, scale=w.scale, out=grads, workspace=ws))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fa.bwd(q, k, v, o, dout, lse, causal=True, scale=w.scale, out=grads, workspace=ws)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    avg = sum(ms) / len(ms)
    flops = 10 * w.d * w.B * w.H * (w.N * (w.N + 1) // 2)   # S recomputed, dP, dV, dQ, dK: 2 d each per pair
    assert all(torch.isfinite(g.float()).all().item() for g in grads)
    return {"value": round(flops / (avg * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms": round(avg, 4),
            "ms_min": round(min(ms), 4), "flop_per_call": flops, "frac_of_bf16_peak": round(
                flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": "bwd_prep_kernel<128> + bwd_dkdv_kernel<128, causal> + bwd_dq_kernel<128, causal>",
            "workload": "prefill workload, dO ~ N(0,1) seeded"}


def paged_decode_leg(fa, torch, si, wd, dq, dk, dv, steps, page_size=16):
    """Decode workload with the caches in 16-key pages of a shuffled pool (the
    seeded block table of the paged-cache generator, pool built on the device),
    timed with HIP events like the contiguous decode; reported apart."""
    import numpy as np
    B, H, L, d = wd.B, wd.H, wd.Lkv, wd.d
    P = L // page_size
    table, num_pages = si.page_table(wd.wid, B, H, L, d, np.full(B, L), page_size)
    idx = torch.from_numpy(table.reshape(-1).astype(np.int64)).to(dq.device)
    pools = []
    for c in (dk, dv):
        pool = torch.full((num_pages, H, page_size, d), float("nan"), dtype=torch.bfloat16, device=dq.device)
        pool[idx] = c.view(B, H, P, page_size, d).permute(0, 2, 1, 3, 4).reshape(B * P, H, page_size, d)
        pools.append(pool)
    tab = torch.from_numpy(table).to(dq.device)
    lens = torch.full((B,), L, dtype=torch.int32, device=dq.device)
    out = torch.empty_like(dq)
    stream = torch.cuda.current_stream(dq.device)
    warm_up(torch, lambda: fa.decode_paged(dq, pools[0], pools[1], tab, lens, nsplit=wd.nsplit, out=out))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fa.decode_paged(dq, pools[0], pools[1], tab, lens, nsplit=wd.nsplit, out=out)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    avg = sum(ms) / len(ms)
    nbytes = 2 * B * H * L * d * 2 + 2 * B * H * d * 2 + B * P * 4 + B * 4   # K, V pages + q, o + table + lengths
    assert torch.isfinite(out.float()).all().item()
    gbps = nbytes / (avg * 1e-3) / 1e9
    del pools
    return {"value": round(gbps, 1), "unit": "GB/s", "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "ms": round(avg, 4), "ms_min": round(min(ms), 4), "algorithmic_bytes_per_call": nbytes,
            "page_size": page_size, "num_pages": num_pages,
            "kernels": "decode_split_paged_kernel<128> + decode_combine_kernel<128>",
            "workload": "decode workload, pages of a shuffled pool (seeded block table), every sequence full"}


def fp8_prefill_leg(fa, torch, si, w, steps):
    """The prefill workload's draws quantised per tensor to FP8 e4m3, through the FP8
    forward; timed with HIP events, reported apart (peak: the dense FP8 MFMA rate)."""
    import numpy as np
    q8, k8, v8, ds = si.fp8_workload(w)
    q, k, v = (torch.from_numpy(x).cuda() for x in (q8, k8, v8))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    warm_up(torch, lambda: fa.fwd_fp8(q, k, v, ds, causal=True, scale=w.scale, out=o, lse=lse))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fa.fwd_fp8(q, k, v, ds, causal=True, scale=w.scale, out=o, lse=lse)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    avg = sum(ms) / len(ms)
    flops = 4 * w.d * w.B * w.H * (w.N * (w.N + 1) // 2)
    assert torch.isfinite(o.float()).all().item()
    del q, k, v, o, lse
    tf = flops / (avg * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "ms": round(avg, 4), "ms_min": round(min(ms), 4), "flop_per_call": flops,
            "kernel": "fwd_fp8_kernel<causal>",
            "workload": "prefill workload (B=1 H=32 N=8192 d=128 causal, K x2) quantised per tensor to e4m3"}


def long_prefill_leg(fa, torch, si, steps):
    """The 128K-token causal prefill (B=4, H=32, N=131072, d=128, bf16), inputs
    N(0,1) from a seeded device generator, timed with HIP events; reported apart."""
    w = si.WORKLOADS[LONG]
    gen = torch.Generator(device="cuda").manual_seed(w.wid)
    shape = (w.B, w.H, w.N, w.d)
    q, k, v = (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fa.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fa.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    avg = sum(ms) / len(ms)
    flops = 4 * w.d * w.B * w.H * (w.N * (w.N + 1) // 2)
    assert torch.isfinite(lse).all().item()
    del q, k, v, o, lse
    tf = flops / (avg * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "ms": round(avg, 3), "ms_min": round(min(ms), 3), "flop_per_call": flops,
            "kernel": "fwd_bf16_kernel<128, causal>",
            "workload": "prefill B=4 H=32 N=131072 d=128 bf16 causal, N(0,1) inputs from a seeded device generator"}


def reported_configs_leg(fa, torch, si, wp, q, k, v, steps):
    """The configurations reported beside the gated ones, each timed on its own with
    HIP events on the launch stream: the fp32 forward at N=256 d=64, the bf16 forward
    at B=4 H=16 N=1024 d=64 causal, the bf16 forward at the 16K causal workload
    (inputs N(0,1) from a seeded device generator), and the three-kernel ablation
    (S and P through HBM) at N=1024 and at the prefill workload next to the fused kernel."""
    import numpy as np
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        warm_up(torch, fn)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(n):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        return sum(ms) / len(ms), min(ms)

    def pairs(w):
        return w.B * w.H * (w.N * (w.N + 1) // 2 if w.causal else w.N * w.N)

    def entry(w, flops, avg, mn, peak, kernel):
        tf = flops / (avg * 1e-3) / 1e12
        return {"value": round(tf, 3), "unit": "TFLOP/s", "frac_of_peak": round(tf / peak, 4), "peak": peak,
                "ms": round(avg, 4), "ms_min": round(mn, 4), "flop_per_call": flops, "kernel": kernel,
                "workload": f"B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}{' causal' if w.causal else ''}"}

    def to_bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()

    res = {}
    w1 = si.WORKLOADS["f32_n256_d64"]
    q1, k1, v1 = (torch.from_numpy(si.tensor_full(w1, t)).cuda() for t in ("q", "k", "v"))
    avg, mn = timed(lambda: fa.fwd(q1, k1, v1, causal=w1.causal, scale=w1.scale), 5 * steps)
    res["f32_n256_d64"] = entry(w1, 4 * w1.d * pairs(w1), avg, mn, PEAK_FP32_TFLOPS, "fwd_f32_kernel")

    w2 = si.WORKLOADS["bf16_b4h16_n1024_d64_causal"]
    q2, k2, v2 = (to_bf16(si.tensor_full(w2, t)) for t in ("q", "k", "v"))
    avg, mn = timed(lambda: fa.fwd(q2, k2, v2, causal=True, scale=w2.scale), 5 * steps)
    res["bf16_b4h16_n1024_d64_causal"] = entry(w2, 4 * w2.d * pairs(w2), avg, mn, PEAK_BF16_TFLOPS,
                                               "fwd_bf16_kernel<64, causal>")
    ws2 = torch.empty(fa.naive_workspace_bytes(w2.B, w2.H, w2.N) // 4, dtype=torch.float32, device="cuda")
    avg_n, mn_n = timed(lambda: fa.naive_fwd(q2, k2, v2, causal=True, scale=w2.scale, workspace=ws2), steps)
    e = entry(w2, 4 * w2.d * pairs(w2), avg_n, mn_n, PEAK_BF16_TFLOPS, "naive_* (ablation)")
    e["fused_speedup"] = round(avg_n / avg, 2)
    e["score_bytes_per_call"] = 4 * w2.B * w2.H * w2.N * w2.N * 4   # S written, read, P written, read (fp32)
    res["ablation_bf16_b4h16_n1024_d64_causal"] = e
    del q2, k2, v2, ws2

    w4 = si.WORKLOADS["bf16_h32_n16384_d128_causal"]
    gen = torch.Generator(device="cuda").manual_seed(w4.wid)
    shape = (w4.B, w4.H, w4.N, w4.d)
    q4, k4, v4 = (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                  for _ in range(3))
    o4 = torch.empty_like(q4)
    lse4 = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    avg, mn = timed(lambda: fa.fwd(q4, k4, v4, causal=True, scale=w4.scale, out=o4, lse=lse4), steps)
    assert torch.isfinite(lse4).all().item()
    res["bf16_h32_n16384_d128_causal"] = entry(w4, 4 * w4.d * pairs(w4), avg, mn, PEAK_BF16_TFLOPS,
                                               "fwd_bf16_kernel<128, causal>")
    del q4, k4, v4, o4, lse4

    avg_f, _ = timed(lambda: fa.fwd(q, k, v, causal=True, scale=wp.scale), steps)
    ws3 = torch.empty(fa.naive_workspace_bytes(wp.B, wp.H, wp.N) // 4, dtype=torch.float32, device="cuda")
    avg_n, mn_n = timed(lambda: fa.naive_fwd(q, k, v, causal=True, scale=wp.scale, workspace=ws3), max(2, steps // 2))
    e = entry(wp, 4 * wp.d * pairs(wp), avg_n, mn_n, PEAK_BF16_TFLOPS, "naive_* (ablation)")
    e["fused_speedup"] = round(avg_n / avg_f, 2)
    e["score_bytes_per_call"] = 4 * wp.B * wp.H * wp.N * wp.N * 4
    e["workload"] += " (K x2: the prefill workload)"
    res["ablation_bf16_h32_n8192_d128_causal_k2"] = e
    del ws3
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first; the clock takes about a dozen prefill+decode steps to settle")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="CPU work of the oracle baseline (0 disables it)")
    ap.add_argument("--bwd-steps", type=int, default=10,
                    help="timed calls of the backward pass (reported apart from the step; 0 disables it)")
    ap.add_argument("--paged-steps", type=int, default=20,
                    help="timed calls of the paged-KV decode (reported apart from the step; 0 disables it)")
    ap.add_argument("--fp8-steps", type=int, default=20,
                    help="timed calls of the FP8 forward on the prefill workload (reported apart; 0 disables it)")
    ap.add_argument("--long-steps", type=int, default=3,
                    help="timed calls of the 128K-token prefill (reported apart from the step; 0 disables it)")
    ap.add_argument("--report-steps", type=int, default=10,
                    help="timed calls per reported configuration (N=256 fp32, N=1024 d=64, 16K, the ablation; "
                         "reported apart; 0 disables them)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before warm-up, run one plain 1 GiB device copy (a reference for byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: launch it without torch.distributed", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import seeded_inputs as si
    from exact_io_aware_74_amd import binding as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    wp, wd = si.WORKLOADS[PREFILL], si.WORKLOADS[DECODE]
    t_gen = time.perf_counter()
    q, k, v = (to_dev(si.tensor_full(wp, t)) for t in ("q", "k", "v"))
    dq = to_dev(si.tensor_full(wd, "q")[:, :, 0, :])
    dk = to_dev(si.tensor_full(wd, "k"))
    dv = to_dev(si.tensor_full(wd, "v"))
    gen_s = time.perf_counter() - t_gen
    o = torch.empty_like(q)
    lse = torch.empty((wp.B, wp.H, wp.N), dtype=torch.float32, device=dev)
    do = torch.empty_like(dq)

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)    # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(q, k, v, causal=True, scale=wp.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        fa.decode(dq, dk, dv, nsplit=wd.nsplit, out=do)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert torch.isfinite(o).all().item() and torch.isfinite(do.float()).all().item()

    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)

    flops = 4 * wp.d * wp.B * wp.H * (wp.N * (wp.N + 1) // 2)            # 4 d per visible (query, key) pair
    fwd_bytes = 4 * wp.B * wp.H * wp.N * wp.d * 2 + wp.B * wp.H * wp.N * 4  # Q, K, V, O + LSE
    tflops = flops / (fwd_avg * 1e-3) / 1e12
    dec_bytes = 2 * wd.B * wd.H * wd.Lkv * wd.d * 2 + 2 * wd.B * wd.H * wd.d * 2  # K, V caches + q, o
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill B=1 H=32 N=8192 d=128 bf16 causal, K x2 (value); "
                               "decode B=16 H=32 Lkv=32768 d=128 bf16 nsplit=64 (decode)",
                   "prefill": {"B": wp.B, "H": wp.H, "N": wp.N, "d": wp.d, "causal": True, "scale": wp.scale},
                   "decode": {"B": wd.B, "H": wd.H, "Lkv": wd.Lkv, "d": wd.d, "nsplit": wd.nsplit}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": "fwd_bf16_kernel<128, causal>", "algorithmic_flop_per_launch": flops,
                     "kernel_ms": round(fwd_avg, 4)},
        "decode": {"value": round(dec_gbps, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                                "algorithmic_bytes_per_call": dec_bytes,
                                "kernels": "decode_split_kernel<128> + decode_combine_kernel<128>",
                                "ms": round(dec_avg, 4)}},
        "prefill": {"ms": round(fwd_avg, 4), "ms_min": round(min(fwd_ms), 4), "ms_max": round(max(fwd_ms), 4),
                    "compulsory_bytes": fwd_bytes},
        "input_generation_s": round(gen_s, 1),
    }
    if args.paged_steps > 0:
        rec["paged_decode"] = paged_decode_leg(fa, torch, si, wd, dq, dk, dv, args.paged_steps)
    if args.bwd_steps > 0:
        rec["backward"] = backward_leg(fa, torch, si, wp, q, k, v, o, lse, args.bwd_steps)
    if args.report_steps > 0:
        rec["reported_configs"] = reported_configs_leg(fa, torch, si, wp, q, k, v, args.report_steps)
    del q, k, v, dq, dk, dv, o, do
    if args.fp8_steps > 0:
        rec["fp8_prefill"] = fp8_prefill_leg(fa, torch, si, wp, args.fp8_steps)
    if args.long_steps > 0:
        rec["long_prefill"] = long_prefill_leg(fa, torch, si, args.long_steps)
    if args.cpu_baseline_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(wp, args.cpu_baseline_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
