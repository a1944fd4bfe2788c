"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload target]

A step is one pass of the hot path over one batch of synthetic input that is
already resident in HBM. The default workload is the 16384-token sequence sweep
(H=16, d=128, bfloat16, B=16384/N) at the lengths the throughput target is set
for, N = 4096, 8192 and 16384: a step is one non-causal and one causal attn_fwd
call at each N (six calls). The line printed is the whole-job throughput in
TFLOP/s, counting 4*B*H*N^2*d flops per non-causal call (2*B*H*N_q*N_kv*(d_qk+d_v)
in general) and half that for a causal one, with the rate and share of the peak
of every call beside it.

Alongside it:
  * roofline: the dominant kernel's algorithmic flops per launch divided by its
    average launch duration, timed with HIP events on the stream it runs on,
    against the dense bf16 MFMA peak; traffic is the HBM bytes per launch from
    the committed rocprofv3 counter summary when it was taken on the current
    kernel source, else null;
  * cpu_baseline: the float64 CPU oracle timed on this host's cores over a
    bounded sample of the same workload (run before the GPU is touched, since
    its worker pool forks).
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

PEAK = {"bf16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA, TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_81_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "attn_fwd_fp8.hip", "attn_fp8.hip", "attn_decode.hip",
                            "attn_bwd.hip", "exattn_api.cpp", "device.h", "tile_io.h", "fp8_ops.h",
                            "mfma16.h", "launch.h")]
TARGET_N = (4096, 8192, 16384)  # sequence lengths of the throughput target
HBM_PEAK = 8000.0  # MI355X HBM3E, GB/s


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary."""
    from exact_attention_81_amd.profile_report import profile_stem
    path = os.path.join(PROFILES, f"{profile_stem(workload)}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None  # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's description."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def device_info(dev):
    """The GPU the line was measured on: name, architecture, compute units, memory."""
    import torch
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "memory_gib": round(p.total_memory / 2 ** 30, 1)}


def committed_counters(workload: str, variant: str):
    """Clock, matrix-core busy and related figures of one variant from the committed
    hardware-counter summary, or None once the kernels have changed since."""
    from exact_attention_81_amd.profile_report import profile_stem
    path = os.path.join(PROFILES, f"{profile_stem(workload)}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    fig = rec.get("per_variant", {}).get(variant)
    if fig is None:
        return None
    return dict(fig, source=os.path.relpath(path, ROOT))


def cpu_baseline(w_list, max_heads: int, min_seconds: float = 10.0):
    """Time the oracle (as it stands) on up to max_heads heads of each workload.

    The sample is repeated until at least min_seconds of wall time have passed, so
    that small workloads are still timed over a stable interval.
    """
    import oracle
    from exact_attention_81_amd import synth

    procs = max(1, min(16, os.cpu_count() or 1))
    data = []
    for w in w_list:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)][:max_heads]
        data.append((w, synth.qkv_for(w), heads))
    flops = 0.0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for w, (q, k, v), heads in data:
            oracle.attention_parallel(q, k, v, w.scale, w.causal, processes=procs, heads=heads)
            flops += w.flops() * len(heads) / (w.B * w.H)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    parts = [f"{len(heads)} of {w.B * w.H} heads of {w.label()}" for w, _, heads in data]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": procs, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "; ".join(parts) + f", {reps} time(s) ({dt:.1f} s wall, float64 numpy, "
                                        f"fork pool of {procs} processes, one BLAS thread each)"}


def cpu_baseline_one_core(w_list, max_heads: int = 2, min_seconds: float = 3.0):
    """The oracle in one process with one BLAS thread, on the tiny configuration (every
    head) and a few heads of each listed workload: the per-core rate beside the pooled
    baseline."""
    import oracle
    from threadpoolctl import threadpool_limits
    from exact_attention_81_amd import synth

    out = []
    with threadpool_limits(1):
        for w in [synth.workload("tiny")] + list(w_list):
            q, k, v = synth.qkv_for(w)
            q, k, v = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
            heads = [(b, h) for b in range(w.B) for h in range(w.H)][:max_heads]
            done = 0
            t0 = time.perf_counter()
            while True:
                for b, h in heads:
                    oracle.head(q[b, h], k[b, h], v[b, h], w.scale, w.causal)
                done += len(heads)
                dt = time.perf_counter() - t0
                if dt >= min_seconds / (len(w_list) + 1):
                    break
            out.append({"workload": w.label(), "heads": done, "seconds": round(dt, 2),
                        "value": w.flops() * done / (w.B * w.H) / dt / 1e12, "unit": "TFLOP/s",
                        "cores": 1, "kind": "oracle"})
    return out


def cpu_baseline_decode(w, max_heads: int, min_seconds: float = 10.0):
    """Time the oracle on up to max_heads query heads of the decode workload (GB/s of the
    call's algorithmic bytes, each query head counted as its share of them)."""
    import oracle
    from exact_attention_81_amd import synth

    q, k, v = synth.qkv_gqa(w.B, w.H, w.H_kv, w.N_q, w.N_kv, w.d, w.seed)
    q, k, v = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
    g = w.H // w.H_kv
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:max_heads]
    per_head = w.hbm_bytes() / (w.B * w.H)
    done = 0
    t0 = time.perf_counter()
    while True:
        for b, h in heads:
            oracle.head(q[b, h], k[b, h // g], v[b, h // g], w.scale, w.causal)
        done += len(heads)
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": per_head * done / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{len(heads)} of {w.B * w.H} query heads of {w.label()}, "
                      f"{done // len(heads)} time(s) ({dt:.1f} s wall, float64 numpy, one process)"}


def run_decode(args):
    """Split-KV decode with grouped KV heads: one attn_fwd_decode call per step."""
    from exact_attention_81_amd import synth

    w = synth.decode_workload()
    cpu = None if args.no_cpu_baseline else cpu_baseline_decode(w, args.cpu_heads)

    import torch

    import exact_attention_81_amd as ea

    dev = torch.device("cuda:0")
    q, k, v = synth.qkv_gqa(w.B, w.H, w.H_kv, w.N_q, w.N_kv, w.d, w.seed)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    splits = ea.attn_decode_splits(w.B, w.H, w.H_kv, w.N_q, w.N_kv, w.d)
    o = torch.empty((w.B, w.H, w.N_q, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev)
    need = ea.load_library().attn_decode_workspace_bytes(w.B, w.H, w.N_q, w.d, splits)
    ws = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev)

    def launch():
        ea.attn_fwd_decode(q, k, v, causal=w.causal, scale=w.scale, num_splits=splits, out=o,
                           lse=lse, workspace=ws)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for e0, e1 in evs:
        e0.record()
        launch()
        e1.record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    cold = []
    if args.cold_runs > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for _ in range(args.cold_runs):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    durs = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    avg_ms = sum(durs) / len(durs)
    nbytes = w.hbm_bytes()
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    rec = {"variant": w.label(), "avg_launch_us": avg_ms * 1e3,
           "median_launch_us": 0.5 * (durs[(len(durs) - 1) // 2] + durs[len(durs) // 2]) * 1e3,
           "min_launch_us": durs[0] * 1e3, "gbps": achieved, "splits": splits}
    if cold:
        cavg = sum(cold) / len(cold)
        rec["cold_avg_launch_us"] = cavg * 1e3
        rec["cold_gbps"] = nbytes / (cavg * 1e-3) / 1e9
    line = {
        "metric": "attention decode (split-KV, grouped KV heads) HBM GB/s of K, V, Q, O, LSE",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q,K,V ~ N(0,1) rounded to bf16, seeded torch CPU generator",
        "config": {"workload": w.label(), "B": w.B, "H": w.H, "H_kv": w.H_kv, "N_q": w.N_q,
                   "N_kv": w.N_kv, "d": w.d, "causal": w.causal, "splits": splits,
                   "step": "one attn_fwd_decode call (split kernel, then merge kernel)"},
        "roofline": {
            "bound": "hbm",
            "kernel": f"attn_decode_kernel + merge_splits_kernel ({w.label()})",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK, 4),
            "traffic": committed_traffic("decode"),
        },
        "per_variant": [rec],
        "kernel_source_sha": kernel_source_hash(),
        "wall_s_timed_region": round(wall, 4),
        "cpu_baseline": cpu,
    }
    line["device"] = device_info(dev)
    print(json.dumps(line))


def cpu_baseline_bwd(ws, max_heads: int, min_seconds: float = 10.0):
    """Time the gradient oracle on up to max_heads heads of each workload (TFLOP/s of the
    five products' algorithmic flops)."""
    import torch

    import oracle
    from exact_attention_81_amd import synth

    data = []
    for w in ws:
        q, k, v = synth.qkv_for(w)
        g = torch.Generator("cpu").manual_seed(w.seed + 1)
        do = torch.randn((w.B, w.H, w.N_q, w.d_v), generator=g).to(torch.bfloat16)
        f = [oracle.to_f64(x) for x in (q, k, v, do)]
        heads = [(b, h) for b in range(w.B) for h in range(w.H)][:max_heads]
        data.append((w, f, heads))
    flops = 0.0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for w, (q, k, v, do), heads in data:
            for b, h in heads:
                oracle.head_backward(q[b, h], k[b, h], v[b, h], do[b, h], w.scale, w.causal)
            flops += 2.5 * w.flops() * len(heads) / (w.B * w.H)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    parts = [f"{len(heads)} of {w.B * w.H} heads of {w.label()}" for w, _, heads in data]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "; ".join(parts) + f", {reps} time(s) ({dt:.1f} s wall, float64 numpy, "
                                        f"one process)"}


def run_bwd(args):
    """Backward of the default workload: one attn_bwd call per variant per step, the
    forward (for O and LSE) run once outside the timed region."""
    from exact_attention_81_amd import synth

    ws = [synth.workload("single", causal=c) for c in (False, True)]
    cpu = None if args.no_cpu_baseline else cpu_baseline_bwd(ws, min(args.cpu_heads, 16))

    import torch

    import exact_attention_81_amd as ea

    dev = torch.device("cuda:0")
    calls = []
    for w in ws:
        q, k, v = (x.to(dev) for x in synth.qkv_for(w))
        g = torch.Generator("cpu").manual_seed(w.seed + 1)
        do = torch.randn((w.B, w.H, w.N_q, w.d_v), generator=g).to(torch.bfloat16).to(dev)
        o, lse = ea.attn_fwd(q, k, v, causal=w.causal)
        calls.append((w, lambda q=q, k=k, v=v, o=o, lse=lse, do=do, w=w:
                      ea.attn_bwd(q, k, v, o, lse, do, causal=w.causal)))
    for _ in range(args.warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in calls] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        for i, (_, c) in enumerate(calls):
            evs[s][i][0].record()
            c()
            evs[s][i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    bwd_flops = [2.5 * w.flops() for w in ws]  # five products of 2*N_q*N_kv*d per head
    value = sum(bwd_flops) / (ms_per_step * 1e-3) / 1e12
    per = []
    for i, (w, _) in enumerate(calls):
        durs = sorted(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps))
        avg = sum(durs) / len(durs)
        per.append({"variant": "bwd " + w.label(), "avg_launch_us": avg * 1e3,
                    "tflops": bwd_flops[i] / (avg * 1e-3) / 1e12,
                    "median_launch_us": 0.5 * (durs[(len(durs) - 1) // 2] + durs[len(durs) // 2]) * 1e3,
                    "min_launch_us": durs[0] * 1e3})
    dom = max(range(len(per)), key=lambda i: per[i]["avg_launch_us"])
    achieved = per[dom]["tflops"]
    line = {
        "metric": "attention bwd TFLOP/s (10BHN^2d: five products, causal halved)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: Q,K,V,dO ~ N(0,1) rounded to bf16, seeded torch CPU generator",
        "config": {"workload": " + ".join("bwd " + w.label() for w in ws), "B": ws[0].B,
                   "H": ws[0].H, "N_q": ws[0].N_q, "N_kv": ws[0].N_kv, "d": ws[0].d_qk,
                   "causal": [w.causal for w in ws],
                   "step": "one attn_bwd call (dQ kernel, then dK/dV kernel) per variant"},
        "roofline": {"bound": "mfma", "kernel": f"attn_bwd_dq_kernel + attn_bwd_dkdv_kernel "
                                                f"({per[dom]['variant']})",
                     "achieved": round(achieved, 2), "peak": PEAK["bf16"], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK["bf16"], 4), "traffic": committed_traffic("bwd")},
        "per_variant": per,
        "kernel_source_sha": kernel_source_hash(),
        "wall_s_timed_region": round(wall, 4),
        "cpu_baseline": cpu,
    }
    line["device"] = device_info(dev)
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="target",
                    choices=["target", "single", "tiny", "asym", "fp8", "sweep512", "sweep1024",
                             "sweep2048", "sweep4096", "sweep8192", "sweep16384", "decode",
                             "bwd"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads of each variant the CPU oracle is timed on (default: 16 for "
                         "the target workload, 64 otherwise)")
    ap.add_argument("--cold-runs", type=int, default=5,
                    help="launches per variant timed after evicting the caches (0: none)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, run a plain float32 copy of this many MiB "
                         "three times (calibrates the HBM byte counters of a profiler run)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention "
              f"forward is sharded by (batch, head) with no communication, so N GPUs would each "
              f"run this same one-GPU workload.", file=sys.stderr)
        sys.exit(2)

    if args.cpu_heads is None:
        args.cpu_heads = 16 if args.workload == "target" else 64
    if args.workload == "decode":
        run_decode(args)
        return
    if args.workload == "bwd":
        run_bwd(args)
        return

    from exact_attention_81_amd import synth

    if args.workload == "target":
        ws = [synth.workload("sweep", causal=c, N=n) for n in TARGET_N for c in (False, True)]
    elif args.workload.startswith("sweep"):
        n = int(args.workload[5:])
        ws = [synth.workload("sweep", causal=c, N=n) for c in (False, True)]
    elif args.workload in ("tiny", "asym", "fp8"):
        ws = [synth.workload(args.workload)]
    else:
        ws = [synth.workload("single", causal=c) for c in (False, True)]

    cpu = None if args.no_cpu_baseline else cpu_baseline(ws, args.cpu_heads)
    # one-core oracle rate on the tiny and single configurations (single workload only)
    cpu1 = (cpu_baseline_one_core(ws) if cpu is not None and args.workload == "single" else None)

    import torch

    import exact_attention_81_amd as ea

    dev = torch.device("cuda:0")
    fp8 = ws[0].fp8
    prep = None
    inputs = []  # (workload, launch) pairs; launch() enqueues one attention forward
    for w in ws:
        o = torch.empty((w.B, w.H, w.N_q, w.d_v), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev)
        if fp8:
            # Rotation and block quantisation happen once, outside the timed region;
            # they are timed on their own below and reported as "prep".
            signs, q, k, v = synth.fp8_inputs(w.B, w.H, w.N_q, w.d_qk, w.seed)
            q, k, v, signs = q.to(dev), k.to(dev), v.to(dev), signs.to(dev)

            def quantise(q=q, k=k, v=v, signs=signs):
                return (ea.attn_quantize_fp8(q, signs=signs), ea.attn_quantize_fp8(k, signs=signs),
                        ea.attn_quantize_fp8(v, transpose=True))

            (q8, qd), (k8, kd), (v8, vd) = quantise()
            prep = quantise

            def launch(w=w, q8=q8, k8=k8, v8=v8, qd=qd, kd=kd, vd=vd, o=o, lse=lse):
                ea.attn_fwd_fp8(q8, k8, v8, qd, kd, vd, causal=w.causal, scale=w.scale, out=o,
                                lse=lse)
        else:
            q, k, v = synth.qkv_for(w)
            q, k, v = q.to(dev), k.to(dev), v.to(dev)

            def launch(w=w, q=q, k=k, v=v, o=o, lse=lse):
                ea.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        inputs.append((w, launch))

    def step(events=None):
        for i, (w, launch) in enumerate(inputs):
            if events is not None:
                events[i][0].record()
            launch()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in inputs] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    # Cold caches: after the timed region, each launch is timed once more right after a
    # 512 MiB fill that evicts L2 and the infinity cache (MALL).
    cold = [[] for _ in inputs]
    if args.cold_runs > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for _ in range(args.cold_runs):
            for i, (w, launch) in enumerate(inputs):
                flush.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                launch()
                e1.record()
                torch.cuda.synchronize()
                cold[i].append(e0.elapsed_time(e1))
        del flush

    prep_us = None
    if prep is not None:
        for _ in range(3):
            prep()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            prep()
        e1.record()
        torch.cuda.synchronize()
        prep_us = e0.elapsed_time(e1) * 100.0  # per call, microseconds

    if args.copy_mib > 0:
        # Reads and writes copy_mib MiB per launch; outside the timed region.
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    step_flops = sum(w.flops() for w in ws)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    per = []
    for i, (w, *_rest) in enumerate(inputs):
        durs = [evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)]
        avg_ms = sum(durs) / len(durs)
        srt = sorted(durs)
        med_ms = 0.5 * (srt[(len(srt) - 1) // 2] + srt[len(srt) // 2])
        rec = {"variant": w.label(), "avg_launch_us": avg_ms * 1e3,
               "tflops": w.flops() / (avg_ms * 1e-3) / 1e12,
               "median_launch_us": med_ms * 1e3, "min_launch_us": srt[0] * 1e3}
        if cold[i]:
            cavg = sum(cold[i]) / len(cold[i])
            rec["cold_avg_launch_us"] = cavg * 1e3
            rec["cold_tflops"] = w.flops() / (cavg * 1e-3) / 1e12
        per.append(rec)
    dt = "fp8" if fp8 else "bf16"
    peak = PEAK[dt]
    for p in per:
        p["pct_of_peak"] = 100.0 * p["tflops"] / peak
    dom = max(range(len(per)), key=lambda i: per[i]["avg_launch_us"])
    achieved = per[dom]["tflops"]
    traffic = committed_traffic(args.workload)

    w0 = ws[0]
    line = {
        "metric": "attention fwd TFLOP/s (4BHN^2d, causal halved) + % of MI355X MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 (fp8) operands, f32 accumulation" if fp8 else "bf16",
        "data": ("synthetic: Q,K,V ~ N(0,1) with 0.5% of coordinates x30, rounded to bf16, "
                 "random-sign Hadamard rotation of Q and K, e4m3 per 128-token block"
                 if fp8 else "synthetic: Q,K,V ~ N(0,1) rounded to bf16, seeded torch CPU generator"),
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {
            "workload": ("sequence sweep of 16384 tokens (B = 16384/N, H 16, d 128, bf16) at "
                         f"N = {', '.join(str(n) for n in TARGET_N)}, non-causal and causal: "
                         if args.workload == "target" else "") + " + ".join(w.label() for w in ws),
            "B": [w.B for w in ws] if len({w.B for w in ws}) > 1 else w0.B,
            "H": w0.H,
            "N_q": [w.N_q for w in ws] if len({w.N_q for w in ws}) > 1 else w0.N_q,
            "N_kv": [w.N_kv for w in ws] if len({w.N_kv for w in ws}) > 1 else w0.N_kv,
            "d_qk": w0.d_qk, "d_v": w0.d_v, "causal": [w.causal for w in ws],
            "step": ("one attn_fwd_fp8 call on prepared e4m3 inputs" if fp8
                     else "one attn_fwd call per listed variant"),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": f"{'attn_fwd_fp8_kernel' if fp8 else 'attn_fwd_kernel'} "
                      f"({per[dom]['variant']})",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "per_variant": per,
        "kernel_source_sha": kernel_source_hash(),
        "fp8_prep_us": None if prep_us is None else round(prep_us, 2),
        "wall_s_timed_region": round(wall, 4),
        "cpu_baseline": cpu,
    }
    # Hardware-counter figures of the dominant kernel from the committed summary
    # (rocprofv3 --pmc runs of this workload), null once the kernels have changed.
    line["counters"] = committed_counters(args.workload, per[dom]["variant"])
    line["device"] = device_info(dev)
    if cpu1 is not None:
        line["cpu_one_core"] = cpu1
    print(json.dumps(line))


if __name__ == "__main__":
    main()
