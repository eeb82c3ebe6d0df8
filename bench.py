"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_8k]

One step is one forward pass (scores, mask, online softmax, P V, epilogue) of
exact attention over one batch of the named synthetic workload, with the
inputs already resident in device memory. The headline workload is the
long-context causal forward: B=1, Hq=Hkv=32, N=8192, d=128, bf16 storage,
fp32 accumulation, 1% of query rows scaled x8, seed 2.

Prints ONE JSON line: throughput in TFLOP/s (credited flops 4*B*Hq*N^2*d,
halved when causal), the roofline of the forward kernel (MFMA-bound, against
the 2.5 PFLOP/s dense bf16 peak and against the rate a back-to-back MFMA
probe reaches on the same GPU), the per-launch median and minimum over 20
trials of 10 launches, the GPU clock and power read by amd-smi under load,
the backward pass measured the same way, the three-pass materialising
baseline on the same inputs, and the CPU oracle timed on a bounded sample of
the same workload (a baseline only).
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # Enough untimed launches for the GPU clock to leave its idle state (with
    # 5 the timed region still includes the ramp: about 8% lower).
    ap.add_argument("--warmup", type=int, default=50)
    # Before the warmup launches: launches back to back for this long (untimed),
    # so that the GPU clock has left its idle state whatever --warmup is.
    ap.add_argument("--ramp-seconds", type=float, default=1.5)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the headline one); the general-forward workloads "
                         "(decode_32k, chunk_2k_8k, chunk_wide_2k_8k, varlen_mix) time flash_attn_fwd_kv / flash_attn_fwd_varlen")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the amd-smi clock and power sampling (seconds of extra launches; for profiler runs)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-naive", action="store_true",
                    help="skip the three-pass materialising baseline timed on the same inputs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--traffic-file", default=None,
                    help="profile summary holding the HBM bytes per launch from counter runs "
                         "(default: profiles/fwd_bf16_<workload>.md); used only if its kernel sources match")
    return ap.parse_args()


def cpu_baseline(w, inp, causal, budget_s):
    """Time the oracle (as it stands) on whole heads of the workload until the budget is spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("internal_api") == "openblas"),
                      default=os.cpu_count())
    except Exception:  # threadpoolctl missing: report the host's cores
        threads = os.cpu_count()
    G = w.Hq // w.Hkv
    heads = 0
    t0 = time.perf_counter()
    while heads < w.B * w.Hq:
        b, hq = divmod(heads, w.Hq)
        oracle.attn_fwd_head(inp.q[b, hq], inp.k[b, hq // G], inp.v[b, hq // G], w.scale, causal)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if w.bound == "hbm":  # same unit as the GPU line: the slices' share of the minimum traffic per second
        per_head, scale_to, unit, what = w.min_fwd_bytes() / (w.B * w.Hq), 1e9, "GB/s", "minimum bytes"
    else:
        per_head, scale_to, unit, what = w.fwd_flops(causal) / (w.B * w.Hq), 1e12, "TFLOP/s", "flops"
    return {
        "value": round(per_head * heads / dt / scale_to, 6),
        "unit": unit,
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{heads} of {w.B * w.Hq} (batch, head) slices of the same workload, full N x N each, "
                  f"fp64 numpy, {dt:.1f} s; {what} credited as for the GPU",
    }


def measured_mfma_peak(stream, iters=80000, blocks=1024):
    """TFLOP/s of back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD (the
    probe library built beside the attention library), one timed launch of
    about 20 ms after an untimed one; None when the probe is not built."""
    import ctypes
    import torch
    from online_softmax_flash_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        return None
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    sh = ctypes.c_void_p(stream.cuda_stream)
    if lib.fa_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), iters, blocks, sh) != 0:
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    lib.fa_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), iters, blocks, sh)
    e1.record(stream)
    e1.synchronize()
    flops = blocks * 4 * 4 * iters * 2.0 * 32 * 32 * 16
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def clock_ramp(fn, stream, seconds):
    """Untimed launches back to back for `seconds` of wall time before the
    warmup and the timed steps: the GPU clock leaves its idle state over the
    first tens of milliseconds of load, and a fixed time (not a launch count)
    covers that for any workload size."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        n += 10
        stream.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "launches": n}


def time_backward(fn, stream, flops, launches):
    """Backward pass timed like the forward steps: one untimed launch and
    0.3 s of untimed back-to-back launches (the clock is already up from the
    forward), then `launches` timed back to back with HIP events on the launch
    stream, and the median of 5 trials of 3 launches beside it."""
    import torch
    fn()
    clock_ramp(fn, stream, 0.3)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        fn()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / launches
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "tflops": round(tf, 3), "steps": launches, "credited_flops": flops,
            "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
            "timing": timing_trials(fn, stream, trials=5, per=3)}


def timing_trials(fn, stream, trials=20, per=10):
    """Per-launch time over `trials` runs of `per` back-to-back launches
    (HIP events on the launch stream): median and minimum, in ms."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(trials):
        e0.record(stream)
        for _ in range(per):
            fn()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / per)
    times.sort()
    return {"trials": trials, "launches_per_trial": per, "median_ms": round(times[len(times) // 2], 5),
            "min_ms": round(times[0], 5)}


def gpu_metrics_under_load(fn, stream, samples=3):
    """GPU clock and socket power read by `amd-smi` (a child process, queried
    `samples` times one after the other) while the kernel runs back to back
    (batches of 100 launches), after 2 s of the same load; None when amd-smi
    is unavailable or its output cannot be read."""
    import subprocess

    def query():
        try:
            return subprocess.Popen(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], stdout=subprocess.PIPE,
                                    stderr=subprocess.DEVNULL, text=True)
        except OSError:
            return None

    def parse(out):
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_") and isinstance(v, dict)
                and isinstance(v.get("clk"), dict) and isinstance(v["clk"].get("value"), (int, float))]
        return (sum(clks) / len(clks) if clks else None), g["power"]["socket_power"]["value"]

    # The driver's metrics lag the load by up to about a second: keep the
    # kernel running back to back for 2 s before the first query and for at
    # least 0.5 s around each query.
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 2.0:
        for _ in range(100):
            fn()
        n += 100
        stream.synchronize()
    got = []
    for _ in range(samples):
        proc = query()
        if proc is None:
            return None
        tq = time.perf_counter()
        while (proc.poll() is None or time.perf_counter() - tq < 0.5) and time.perf_counter() - tq < 30:
            for _ in range(100):
                fn()
            n += 100
            stream.synchronize()
        try:
            got.append(parse(proc.communicate(timeout=30)[0]))
        except Exception:  # format differences between amd-smi versions: report nothing rather than guess
            return None
    stream.synchronize()
    if not got:
        return None
    clks = [c for c, _ in got if c is not None]
    return {"source": f"amd-smi metric -c -p, {len(got)} queries during back-to-back launches", "launches": n,
            "gfx_clk_mhz": [round(c, 1) for c in clks], "socket_power_w": [p for _, p in got]}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import online_softmax_flash_amd as fa
    from online_softmax_flash_amd.inputs import make_inputs
    from online_softmax_flash_amd.workloads import HEADLINE, WORKLOADS

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    fa.load_library()  # fails loudly when the HIP library is not built

    if args.copy_calibration_mib:
        # A device copy of known size first: counter runs scale by what it reads and writes.
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    from online_softmax_flash_amd.workloads import KV_WORKLOADS
    if args.workload in KV_WORKLOADS:
        print(json.dumps(bench_kv(args, KV_WORKLOADS[args.workload])))
        return
    w = WORKLOADS[args.workload or HEADLINE]
    causal = w.causal[-1]
    inp = make_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, seed=w.seed, dtype=w.dtype, heavy_frac=w.heavy_frac,
                      with_dout=not args.no_backward)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(tdt).to(dev) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    fwd = fa.flash_attn_fwd if w.dtype == "bf16" else fa.flash_attn_fwd_f32

    stream = torch.cuda.current_stream()
    ramp = clock_ramp(lambda: fwd(q, k, v, o, lse, w.scale, causal), stream, args.ramp_seconds)
    for _ in range(args.warmup):
        fwd(q, k, v, o, lse, w.scale, causal)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        fwd(q, k, v, o, lse, w.scale, causal)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = w.fwd_flops(causal)
    tflops = flops / (ms * 1e-3) / 1e12

    traffic = _stored_traffic(args.traffic_file or os.path.join(ROOT, "profiles", f"fwd_bf16_{w.name}.md"))

    nbytes = w.min_fwd_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    kernel = (f"fwd_bf16_kernel<{w.d},64,{8 if w.d <= 128 else 4},{'true' if causal else 'false'}>"
              if w.dtype == "bf16" else f"fwd_kernel<float,{w.d}>")
    mask = "causal" if causal else "non-causal"
    if w.bound == "hbm":
        # Short sequences: the line is the minimum traffic (read Q, K, V; write
        # O, lse once) over the time, against the HBM peak.
        metric, value, unit = f"attention fwd HBM GB/s ({w.dtype}, {mask}, short sequences)", round(gbs, 3), "GB/s"
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic, "min_hbm_bytes": nbytes}
    else:
        metric, value, unit = (f"attention fwd TFLOP/s ({w.dtype}, {mask}) and % of MI355X bf16 MFMA peak",
                               round(tflops, 3), "TFLOP/s")
        roofline = {"bound": "mfma", "kernel": kernel, "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                    "min_hbm_bytes": nbytes}
    result = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": causal,
            "storage": w.dtype, "accumulate": "fp32", "seed": w.seed, "heavy_rows_frac": w.heavy_frac,
            "credited_flops": flops, "tflops": round(tflops, 3),
            "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        },
        "roofline": roofline,
        "wall_s_timed_region": round(wall_s, 4),
        "clock_ramp": ramp,
    }
    step = lambda: fwd(q, k, v, o, lse, w.scale, causal)  # noqa: E731
    result["timing"] = timing_trials(step, stream)
    if not args.no_clock:
        result["gpu"] = gpu_metrics_under_load(step, stream)
    if roofline["bound"] == "mfma":
        mp = measured_mfma_peak(stream)
        if mp:
            roofline["measured_peak"] = round(mp, 1)
            roofline["frac_of_measured_peak"] = round(tflops / mp, 4)
            # One 32x32x16 bf16 product per 32 cycles per SIMD, 1024 SIMDs:
            # the clock the probe ran at.
            roofline["probe_clock_ghz"] = round(mp * 1e12 / (1024 * 32768 / 32) / 1e9, 3)

    if not args.no_backward and inp.do is not None:
        do = torch.from_numpy(inp.do).to(tdt).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(max(fa.flash_attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), 256),
                         dtype=torch.uint8, device=dev)
        bwd = fa.flash_attn_bwd if w.dtype == "bf16" else fa.flash_attn_bwd_f32
        try:
            result["backward"] = time_backward(lambda: bwd(q, k, v, o, lse, do, dq, dk, dv, ws, w.scale, causal),
                                               stream, w.bwd_flops(causal), max(10, args.steps // 2))
        except fa.FlashAttnError as e:
            result["backward"] = {"error": str(e)}

    if not args.no_naive and w.dtype == "bf16":
        # The materialising baseline on the same inputs: scores and weights of
        # every pair go through HBM. Quadratic workspace, allocated here.
        nws = fa.flash_attn_naive_workspace_bytes(w.B, w.Hq, w.N)
        free, _ = torch.cuda.mem_get_info()
        if nws + (1 << 30) < free:
            ws_n = torch.empty(nws, dtype=torch.uint8, device=dev)
            o_n, lse_n = torch.empty_like(q), torch.empty_like(lse)
            fa.flash_attn_naive_fwd(q, k, v, o_n, lse_n, w.scale, causal, ws_n)
            torch.cuda.synchronize()
            nn = max(3, args.steps // 5)
            ev0.record(stream)
            for _ in range(nn):
                fa.flash_attn_naive_fwd(q, k, v, o_n, lse_n, w.scale, causal, ws_n)
            ev1.record(stream)
            torch.cuda.synchronize()
            nms = ev0.elapsed_time(ev1) / nn
            result["naive_baseline"] = {"ms": round(nms, 5), "tflops": round(flops / (nms * 1e-3) / 1e12, 3),
                                        "fused_speedup": round(nms / ms, 3), "steps": nn,
                                        "workspace_bytes": nws,
                                        "kernels": "naive_scores_kernel, naive_softmax_kernel, naive_pv_kernel"}
            del ws_n, o_n, lse_n
        else:
            result["naive_baseline"] = {"skipped": f"needs {nws} bytes of workspace"}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, causal, args.cpu_seconds)

    print(json.dumps(result))


def bench_kv(args, w):
    """One step = one general forward (all splits and the combine) over the workload."""
    import torch
    import online_softmax_flash_amd as fa
    from online_softmax_flash_amd.inputs import make_kv_inputs, make_varlen_inputs

    dev = torch.device("cuda:0")
    lens = w.lengths()
    if w.lengths_seed:
        cu = np.concatenate([[0], np.cumsum([nq for nq, _ in lens])]).astype(np.int64)
        inp = make_varlen_inputs(w.Hq, w.Hkv, cu, cu, w.d, w.seed, with_dout=not args.no_backward)
        cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
        max_q = int(max(nq for nq, _ in lens))
        max_k = int(max(nk for _, nk in lens))
        rows = w.Hq * int(cu[-1])
    else:
        inp = make_kv_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed, with_dout=not args.no_backward)
        max_q, max_k = w.Nq, w.Nk
        rows = w.B * w.Hq * w.Nq
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    B = len(lens)
    splits = w.num_splits or fa.flash_attn_fwd_kv_num_splits(B, w.Hq, w.Hkv, max_q, max_k, w.d)
    nws = fa.flash_attn_fwd_kv_workspace_bytes(rows, w.d, splits)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

    def step():
        if w.lengths_seed:
            fa.flash_attn_fwd_varlen(q, k, v, o, lse, cu_t, cu_t, max_q, max_k, w.scale, w.causal, splits, ws)
        else:
            fa.flash_attn_fwd_kv(q, k, v, o, lse, w.scale, w.causal, splits, ws)

    stream = torch.cuda.current_stream()
    ramp = clock_ramp(step, stream, args.ramp_seconds)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = w.fwd_flops()
    nbytes = w.min_bytes()
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    hbm = w.Nq * (w.Hq // w.Hkv) <= 32 and not w.lengths_seed  # decode: reading K and V is the work
    result = {
        "metric": ("attention decode HBM GB/s (bf16, split keys)" if hbm
                   else "attention fwd TFLOP/s (bf16, general forward)"),
        "value": round(gbs if hbm else tflops, 3),
        "unit": "GB/s" if hbm else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": max_q, "Nk": max_k, "d": w.d,
                   "causal": w.causal, "varlen": bool(w.lengths_seed), "num_splits": splits, "seed": w.seed,
                   "credited_flops": flops, "min_hbm_bytes": nbytes, "tflops": round(tflops, 3),
                   "gbs": round(gbs, 3)},
        "roofline": ({"bound": "hbm", "kernel": "fwd_kv_bf16_kernel + fwd_combine_kernel", "achieved": round(gbs, 3),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
                     if hbm else
                     {"bound": "mfma", "kernel": "fwd_kv_bf16_kernel", "achieved": round(tflops, 3),
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                      "traffic": None}),
        "wall_s_timed_region": round(wall_s, 4),
        "clock_ramp": ramp,
    }
    if not args.no_backward and splits == 1:
        # The general backward over the same problem (o and lse from the
        # forward above): one step = D and l2, then dK/dV and dQ (one launch
        # for variable-length batches, Nq != Nk and d = 256; two otherwise).
        do = torch.from_numpy(inp.do).to(torch.bfloat16).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        wsb = torch.empty(max(fa.flash_attn_bwd_kv_workspace_bytes(rows, w.d), 256), dtype=torch.uint8, device=dev)

        def bstep():
            if w.lengths_seed:
                fa.flash_attn_bwd_varlen(q, k, v, o, lse, do, dq, dk, dv, cu_t, cu_t, max_q, max_k, wsb, w.scale,
                                         w.causal)
            else:
                fa.flash_attn_bwd_kv(q, k, v, o, lse, do, dq, dk, dv, wsb, w.scale, w.causal)

        result["backward"] = time_backward(bstep, stream, 2.5 * flops, max(10, args.steps // 2))
        fused = bool(w.lengths_seed) or w.Nq != w.Nk or w.d == 256
        result["backward"]["kernels"] = ("bwd_prep_bf16_kernel, bwd_fused_bf16_kernel" if fused else
                                         "bwd_prep_bf16_kernel, bwd_dkdv_bf16_kernel, bwd_dq_bf16_kernel")

    if not args.no_cpu_baseline:
        import oracle
        G = w.Hq // w.Hkv
        t0 = time.perf_counter()
        done = 0
        pairs = [(b, hq) for b in range(B) for hq in range(w.Hq)]
        for b, hq in pairs:
            if w.lengths_seed:
                t_a, t_b = int(cu[b]), int(cu[b + 1])
                oracle.attn_fwd_head(inp.q[hq, t_a:t_b], inp.k[hq // G, t_a:t_b], inp.v[hq // G, t_a:t_b], w.scale,
                                     w.causal)
            else:
                oracle.attn_fwd_head(inp.q[b, hq], inp.k[b, hq // G], inp.v[b, hq // G], w.scale, w.causal)
            done += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        frac = done / len(pairs)  # heads are of equal work except in the variable-length batch
        if w.lengths_seed:
            per = [w.Hq and (nq * nk) for nq, nk in lens]
            frac = sum(per[b] for b, _ in pairs[:done]) / (w.Hq * sum(per))
        val = (nbytes * frac / dt / 1e9) if hbm else (flops * frac / dt / 1e12)
        result["cpu_baseline"] = {"value": round(val, 6), "unit": result["unit"], "cores": os.cpu_count(),
                                  "kind": "oracle",
                                  "sample": f"{done} of {len(pairs)} (sequence, head) slices, fp64 numpy, {dt:.1f} s"}
    return result


def _stored_traffic(path):
    """HBM bytes per launch recorded by the counter runs in a profile summary,
    or None when the file is missing or the kernel sources changed since."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    t = re.search(r"^traffic_bytes_per_launch = (\d+)$", text, flags=re.M)
    k = re.search(r"^kernel_sources_sha = ([0-9a-f]+)$", text, flags=re.M)
    if not t or not k or k.group(1) != _kernel_sha():
        return None
    return int(t.group(1))


# Sources and build flags of the headline forward kernel: stored counter data
# is used only while these are unchanged.
FWD_SOURCES = ("fa_device.hpp", "fa_fwd.hpp", "fa_fwd_bf16.hpp", "fa_fwd_bf16.hip")


def _kernel_sha() -> str:
    """Hash of the headline forward's sources (comments and layout left out:
    only code counts) and build flags, to tell whether stored counter data is
    current."""
    import hashlib
    import re
    from online_softmax_flash_amd import build as b
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "online_softmax_flash_amd", "csrc")
    for f in FWD_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(f.encode() + " ".join(code.split()).encode())
    flags = b.COMMON + b.DEVICE_FLAGS + b.EXTRA_FLAGS.get("fa_fwd_bf16.hip", [])
    h.update(repr([f.replace(b.ROOT, "<root>") for f in flags]).encode())  # independent of where the tree lives
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
