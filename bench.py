"""Benchmark of the fused attention forward on one MI355X.

One step = one attn_fwd call over the whole workload (all of B x H x Nq x Nk),
with inputs already resident in device memory. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The default workload is B=2, H=32, N=4096, d=128, bf16, non-causal. A
decoding workload (one query row per head, names starting "decode_") runs
the split-key forward instead: one step = one attn_fwd_splitkv call (split
forward + merge), and its roofline is the HBM one: the bytes of Q, K and V
read once and of O and LSE written once, over the step time.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 matrix
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
# the sources a kernel's HBM traffic depends on (kernel body and its launch)
KERNEL_SRC = {"bf16": ["exact_io_aware_06_amd/csrc/fwd_bf16_kernel.h",
                       "exact_io_aware_06_amd/csrc/fwd_bf16.hip",
                       "exact_io_aware_06_amd/csrc/fwd_bf16_stream.hip"],
              "f32": ["exact_io_aware_06_amd/csrc/fwd_f32.hip"]}


def _src_hash(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic(workload, dtype):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    the kernel source has not changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_sha256") != _src_hash(KERNEL_SRC[dtype]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def window_flops(w):
    """4 d FLOPs per (query, key) pair inside the sliding window (the band
    around the bottom-right-aligned diagonal, clipped to the key range)."""
    import numpy as np
    left, right = w.window
    if w.causal:
        right = 0
    i = np.arange(w.Nq, dtype=np.int64)
    diag = i + (w.Nk - w.Nq)
    lo = np.zeros_like(i) if left is None or left < 0 else np.maximum(diag - left, 0)
    hi = (np.full_like(i, w.Nk - 1) if right is None or right < 0
          else np.minimum(diag + right, w.Nk - 1))
    pairs = int(np.maximum(hi - lo + 1, 0).sum())
    return 4.0 * w.B * w.H * w.d * pairs


def _threadpools():
    """The host thread pools the oracle runs on (BLAS, OpenMP), as numpy and
    torch loaded them."""
    try:
        from threadpoolctl import threadpool_info
        return [(d.get("user_api"), d.get("internal_api"), d.get("num_threads", 1))
                for d in threadpool_info()]
    except Exception:
        return []


def _blas_threads():
    n = [t for api, _, t in _threadpools() if api == "blas"]
    return max(n) if n else 1


def _host():
    """What the CPU baseline ran on: model, the cores this process may use
    (sched_getaffinity), and the thread pools."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count(),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
            "threadpools": [{"api": a, "impl": i, "threads": t} for a, i, t in _threadpools()]}


def _oracle_single_thread():
    """Single-thread oracle times on the two small configured shapes: the
    whole fp32 single-head workload and one (b, h) head of the d = 64
    workload, each the best of three runs with every thread pool held to
    one thread."""
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits
    out = {}
    for name, one_head in (("c1_f32_single_head", False), ("c2_bf16_d64", True)):
        w = workloads.CONFIGS[name]
        inp = workloads.make_inputs(w)
        sl = (lambda t: t[0:1, 0:1]) if one_head else (lambda t: t)
        q, k, v = (sl(inp[x]).double().numpy() for x in ("q", "k", "v"))
        best = math.inf
        with threadpool_limits(limits=1):
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.attention_forward(q, k, v, scale=inp["scale"], causal=w.causal)
                best = min(best, time.perf_counter() - t0)
        flops = w.flops() / (w.B * w.H if one_head else 1)
        out[name + (" (one head)" if one_head else "")] = {
            "seconds": round(best, 4), "gflops": round(flops / best / 1e9, 3)}
    return out


def cpu_baseline(inp, w, budget_s=15.0):
    """Time the fp64 oracle, as it stands, on whole (b, h) heads of the same
    inputs until the time budget is spent; report the rate in TFLOP/s, the
    host it ran on, and single-thread times on the two small shapes."""
    import oracle
    q, k, v = inp["q"], inp["k"], inp["v"]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    rep = w.H // w.kv_heads   # query head h reads key/value head h // rep
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        hk = h // rep
        oracle.attention_forward(q[b:b + 1, h:h + 1].double().numpy(),
                                 k[b:b + 1, hk:hk + 1].double().numpy(),
                                 v[b:b + 1, hk:hk + 1].double().numpy(),
                                 scale=inp["scale"], causal=w.causal, window=w.window)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = (w.flops() if w.window is None else window_flops(w)) * done / len(heads)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(),
        "kind": "oracle",
        "sample": (f"{done} of {len(heads)} (b,h) heads of {w.name} at full "
                   f"Nq={w.Nq}, Nk={w.Nk}, fp64 materialising S and P, {dt:.1f} s; "
                   "the matrix products run on the BLAS pool (cores = its threads), "
                   "the exponentials and masks on one thread"),
        "host": _host(),
        "single_thread": _oracle_single_thread(),
    }


def varlen_flops(w, lens):
    """4 d FLOPs per (query, key) pair of every packed sequence (halved when
    causal, like the other causal workloads)."""
    pairs = sum(int(n) * int(n) for n in lens)
    return 4.0 * w.H * w.d * pairs * (0.5 if w.causal else 1.0)


def bench_varlen(args, w):
    """Packed variable-length batch: one step = one attn_fwd_varlen call.
    The same sequences padded to the length cap and masked with kv_len (the
    padded rectangle of the pages' Lab 5) are timed too, for the speedup."""
    import torch
    import workloads
    import exact_io_aware_06_amd as ea

    inp = workloads.make_varlen_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    cu = inp["cu"].to(dev)
    lens = inp["lens"]
    step, _, _ = ea.prepare_varlen_call(q, k, v, cu, cu, inp["max_len"], causal=w.causal,
                                        scale=inp["scale"])

    # the padded rectangle: [B, H, cap, d] with keys past each length masked
    L = w.Nq
    qp = torch.zeros(w.B, w.H, L, w.d, dtype=q.dtype, device=dev)
    kp = torch.zeros(w.B, w.kv_heads, L, w.d, dtype=q.dtype, device=dev)
    vp = torch.zeros_like(kp)
    c = inp["cu"].tolist()
    for b in range(w.B):
        n = c[b + 1] - c[b]
        qp[b, :, :n] = q[c[b]:c[b + 1]].transpose(0, 1)
        kp[b, :, :n] = k[c[b]:c[b + 1]].transpose(0, 1)
        vp[b, :, :n] = v[c[b]:c[b + 1]].transpose(0, 1)
    kv_len = lens.to(torch.int32).to(dev)
    step_p = None
    if not args.no_padded:
        step_p, _, _ = ea.prepare_call(qp, kp, vp, kv_len=kv_len, causal=w.causal,
                                       scale=inp["scale"])

    def timed(fn):
        warm_up(fn, args)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    ms = timed(step)
    ms_padded = timed(step_p) if step_p is not None else None
    flops = varlen_flops(w, lens)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_varlen(inp, w, args.cpu_budget)
        cpu["value"] = round(cpu["value"], 6)
    out = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak at 1 MI355X (N=4096,d=128)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {**w.describe(), "total_tokens": int(lens.sum()),
                   "lens": [int(x) for x in lens], "flops_per_step": flops,
                   "padded_ms_per_step": round(ms_padded, 4) if ms_padded else None,
                   "speedup_vs_padded": round(ms_padded / ms, 3) if ms_padded else None,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": _traffic(w.name, w.dtype)},
        "cpu_baseline": cpu, "clock_settle": args.clock_settle,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_backward(args, w):
    """One step = one attn_bwd call (preprocess, dK/dV and dQ kernels) on the
    workload, with Q, K, V, O, LSE and dO resident. FLOPs: 2.5 times the
    forward's (five tile products against two), the pages' accounting."""
    import torch
    import workloads
    import exact_io_aware_06_amd as ea

    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    bias = inp["bias"].to(dev) if inp["bias"] is not None else None
    kv_len = inp["kv_len"].to(dev) if inp["kv_len"] is not None else None
    g = torch.Generator().manual_seed(w.seed + 1000)
    do = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
    o, lse = ea.attn_fwd(q, k, v, bias=bias, kv_len=kv_len, causal=w.causal, scale=inp["scale"],
                         window=w.window)
    step, _, _, _ = ea.prepare_bwd_call(q, k, v, o, lse, do, bias=bias, kv_len=kv_len,
                                        causal=w.causal, scale=inp["scale"], window=w.window)
    warm_up(step, args)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    fwd_flops = w.flops() if w.window is None else window_flops(w)
    flops = 2.5 * fwd_flops
    tflops = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        rep = w.H // w.kv_heads
        done, t0 = 0, time.perf_counter()
        do_c = do.cpu()
        for b, h in heads:
            sl = lambda t, hh: t[b:b + 1, hh:hh + 1].double().numpy()
            oracle.attention_backward(sl(inp["q"], h), sl(inp["k"], h // rep), sl(inp["v"], h // rep),
                                      sl(do_c, h), scale=inp["scale"], causal=w.causal,
                                      window=w.window)
            done += 1
            if time.perf_counter() - t0 >= args.cpu_budget:
                break
        dt = time.perf_counter() - t0
        cpu = {"value": round(flops * done / len(heads) / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": _blas_threads(), "kind": "oracle",
               "sample": f"{done} of {len(heads)} (b,h) heads of {w.name} backward at full "
                         f"Nq={w.Nq}, Nk={w.Nk}, fp64 materialising S, P, dP, dS, {dt:.1f} s"}
    out = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak at 1 MI355X (N=4096,d=128)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {**w.describe(), "pass": "backward", "flops_per_step": flops,
                   "flops_rule": "2.5 x forward (5 tile products vs 2)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "timed": "preprocess + dK/dV + dQ (whole step)"},
        "cpu_baseline": cpu, "clock_settle": args.clock_settle,
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_varlen(inp, w, budget_s=15.0):
    """The oracle on whole (sequence, head) pairs of the packed batch until
    the time budget is spent; TFLOP/s over the pairs done."""
    import oracle
    c = inp["cu"].tolist()
    rep = w.H // w.kv_heads
    done_flops, done, total = 0.0, 0, w.B * w.H
    t0 = time.perf_counter()
    for s in range(w.B):
        n = c[s + 1] - c[s]
        for h in range(w.H):
            hk = h // rep
            qs = inp["q"][c[s]:c[s + 1], h].double().numpy()[None, None]
            ks = inp["k"][c[s]:c[s + 1], hk].double().numpy()[None, None]
            vs = inp["v"][c[s]:c[s + 1], hk].double().numpy()[None, None]
            oracle.attention_forward(qs, ks, vs, scale=inp["scale"], causal=w.causal)
            done_flops += 4.0 * w.d * n * n * (0.5 if w.causal else 1.0)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{done} of {total} (sequence, head) pairs of {w.name}, fp64 "
                      f"materialising S and P, {dt:.1f} s"}


def warm_up(fn, args):
    """Untimed calls before a timed region, in two parts.

    Clock settling: the GPU's clocks ramp over the first ~20 launches and
    keep rising for about 100 ms of sustained load (a d = 64 call of 80 us
    measured 15% slower after 30 calls than after 300), so first the step
    runs for about 150 ms (at least 10 calls, at most 5000). Then exactly
    args.warmup warm-up steps (default 30). The JSON line reports both:
    `warmup` is the warm-up steps, `clock_settle` the settling calls."""
    import torch
    t0 = time.perf_counter()
    calls = 0
    while calls < 10 or (time.perf_counter() - t0 < 0.15 and calls < 5000):
        fn()
        calls += 1
        if calls % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    args.clock_settle = {"calls": calls, "ms": round((time.perf_counter() - t0) * 1e3, 1)}
    if args.warmup is None:
        args.warmup = 30
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()


def gemm_ms(torch, n, warmup, steps):
    """Milliseconds per plain bf16 n x n x n product through torch (the
    vendor GEMM library): the matrix throughput this board sustains."""
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(warmup):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        torch.matmul(a, b, out=c)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps before the timed ones (default 30); they "
                         "follow about 150 ms of clock-settling calls, reported apart")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (attn_bwd) of the workload instead of the forward")
    ap.add_argument("--splits", type=int, default=None,
                    help="split count for a decoding workload (default: the library's choice)")
    ap.add_argument("--cold", action="store_true",
                    help="cold caches: write a 512 MiB buffer before every timed call and "
                         "report the median call (each call timed on its own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-padded", action="store_true",
                    help="packed-sequence workloads: skip the padded-batch comparison (so "
                         "that a profile of the run holds the packed call only)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB mebibytes (the "
                         "reference kernel that scales the HBM byte counters)")
    ap.add_argument("--gemm-calibration", type=int, default=0, metavar="N",
                    help="only time a plain bf16 N x N x N matrix product through torch "
                         "(the matrix throughput this GPU sustains, for context)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the "
              "forward has no multi-GPU path", file=sys.stderr)
        return 2

    import torch
    import workloads
    import exact_io_aware_06_amd as ea

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / max(args.steps, 1)
        # the HBM rate a plain device-to-device copy sustains (read + write)
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                          "launches": max(args.steps, 1) + 1, "ms": round(ms, 4),
                          "gbps": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return 0

    if args.gemm_calibration:
        n = args.gemm_calibration
        ms = gemm_ms(torch, n, max(args.warmup or 30, 1), max(args.steps, 1))
        print(json.dumps({"gemm_bf16_n": n, "ms": round(ms, 4),
                          "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}), flush=True)
        return 0

    name = args.workload or workloads.HEADLINE
    w = workloads.ALL[name]
    split = name in workloads.DECODE
    if name in workloads.VARLEN:
        return bench_varlen(args, w)
    if args.backward:
        return bench_backward(args, w)
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    bias = inp["bias"].to(dev) if inp["bias"] is not None else None
    kv_len = inp["kv_len"].to(dev) if inp["kv_len"] is not None else None
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device=dev)
    n_split = None
    if split:
        n_split = args.splits or ea.splitkv_num_splits(w.B, w.H, w.Nq, w.Nk, w.d, w.causal,
                                                       bias is not None, w.kv_heads)
    # arguments marshalled once: a step is the launch(es) alone
    step, _, _ = ea.prepare_call(q, k, v, bias=bias, kv_len=kv_len, causal=w.causal,
                                 scale=inp["scale"], out=o, lse=lse, split=split,
                                 num_splits=n_split, window=w.window)

    warm_up(step, args)
    stream = torch.cuda.current_stream(dev)

    def per_call(n, flush=None):
        # each call between its own pair of events (after the main timing, so
        # the recorded events do not sit between the timed launches)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            if flush is not None:
                flush.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)
        return {"median": round(t[len(t) // 2], 4), "min": round(t[0], 4), "calls": n}

    if args.cold:
        # the L2s and the MALL hold far less than 512 MiB: writing it evicts the
        # inputs, so each call reads them from HBM again
        flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
        calls = per_call(max(args.steps, 1), flush)
        ms = calls["median"]
    else:
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / args.steps
        calls = per_call(min(max(args.steps, 1), 50))

    flops = w.flops() if w.window is None else window_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    extra = {}
    if inp["kv_len"] is not None and not w.causal:
        # FLOPs of the keys inside each batch's valid length only
        kl = inp["kv_len"].clamp(0, w.Nk).double()
        useful = float(4.0 * w.H * w.Nq * w.d * kl.sum().item())
        extra = {"useful_flops_per_step": useful,
                 "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2)}
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                "traffic": _traffic(name, w.dtype)}
    if inp["bias"] is not None:
        # A dense fp32 bias of H x Nq x Nk makes the forward HBM-bound: its
        # algorithmic bytes are Q, K, V read and O written once per head, the
        # LSE written, the bias read once (it is shared by the batch) and the
        # key lengths; at 2.5 PFLOP/s and 8 TB/s the matrix work would take
        # less time than these bytes.
        eb = 2 if w.dtype == "bf16" else 4
        algo = (w.B * w.H * w.Nq * (2 * w.d * eb + 4) + 2 * w.B * w.kv_heads * w.Nk * w.d * eb
                + 4 * inp["bias"].numel()
                + (0 if inp["kv_len"] is None else 4 * w.B))
        gbps = algo / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "traffic": _traffic(name, w.dtype), "bytes_per_step": algo,
                    "mfma_context": {"achieved_tflops": round(tflops, 2), "peak": peak,
                                     "frac": round(tflops / peak, 4)}}
    if split:
        eb = 2 if w.dtype == "bf16" else 4
        algo = w.kv_bytes() + w.B * w.H * w.Nq * (2 * w.d * eb + 4)  # K, V; Q, O; LSE
        gbps = algo / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "traffic": _traffic(name, w.dtype),
                    "bytes_per_step": algo, "timed": "split forward + merge (whole step)"}
        extra = {"num_splits": n_split}

    gemm = None
    if roofline["bound"] == "mfma" and w.dtype == "bf16" and not args.cold:
        # context, after the timed region: what the vendor GEMM reaches on
        # this board (a dense contraction with none of attention's softmax)
        gms = gemm_ms(torch, 8192, 10, 20)
        gt = 2.0 * 8192 ** 3 / (gms * 1e-3) / 1e12
        gemm = {"vendor_gemm_bf16_8192_tflops": round(gt, 1),
                "vendor_gemm_frac_of_peak": round(gt / peak, 4),
                "attention_over_gemm": round(tflops / gt, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, w, args.cpu_budget)
        cpu["value"] = round(cpu["value"], 6)

    out = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak at 1 MI355X (N=4096,d=128)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {**w.describe(), "flops_per_step": flops, **extra, "parallelism": "single GPU",
                   "caches": "cold (512 MiB written before each call; value from the median call)"
                   if args.cold else "warm (inputs resident)"},
        "roofline": roofline, "cpu_baseline": cpu,
        "per_call_ms": calls, "clock_settle": args.clock_settle,
        "gemm_context": gemm,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
