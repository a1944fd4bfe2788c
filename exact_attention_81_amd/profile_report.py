"""Summarise rocprofv3 output of a bench.py run into text under profiles/.

    python -m exact_attention_81_amd.profile_report --workload single \\
        --bench-json RUN/bench.json --stats RUN/stats --fetch RUN/fetch --write RUN/write \\
        --copy-mib 1024 --commands RUN/commands.txt

Inputs are the directories rocprofv3 wrote with ``--output-format csv``:
  * ``--stats``: a ``--kernel-trace --stats`` run (``*kernel_stats.csv``);
  * ``--fetch`` / ``--write``: ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` runs
    (``*counter_collection.csv``, KiB per dispatch) of ``bench.py --copy-mib M``.
The copy kernel of those runs moves a known number of bytes; dividing that by what
the counter reads for it gives the factor that turns the counter into bytes. The
attention kernel's counter times that factor is its HBM traffic per launch.

Writes ``profiles/<stem>.md`` (figures and the commands that made them) and
``profiles/<stem>_traffic.json`` (read by bench.py, which uses it only while the
kernel sources hash to the recorded value); ``profile_stem`` names the kernel and
the workload.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
from collections import defaultdict

from . import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_RE = re.compile(
    r"attn_fwd_kernel<(\d+), (\d+), (true|false), (\d+), (true|false)(?:, (true|false))?>")
FP8_RE = re.compile(r"attn_fwd_fp8_kernel<(true|false)>")
DEC_RE = re.compile(r"attn_decode_kernel<(\d+), (true|false), (true|false), (\d+)>")
MERGE_RE = re.compile(r"merge_splits_kernel<(\d+), (true|false)>")
BWD_RE = re.compile(r"attn_bwd_(dq|dkdv)_kernel<(\d+), (true|false), (true|false)>")


def _one(pattern_dir: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {pattern_dir}")
    return hits[0]


def short_name(name: str) -> str:
    m = KERNEL_RE.search(name)
    if m:
        dqk, dv, causal, tau, f16, strided = m.groups()
        return (f"attn_fwd_kernel d{dqk}x{dv} {'causal' if causal == 'true' else 'noncausal'} "
                f"tau{tau} {'fp16' if f16 == 'true' else 'bf16'}"
                f"{' strided' if strided == 'true' else ''}")
    m = FP8_RE.search(name)
    if m:
        return f"attn_fwd_fp8_kernel d128x128 {'causal' if m.group(1) == 'true' else 'noncausal'} e4m3"
    m = DEC_RE.search(name)
    if m:
        d, causal, f16, nrb = m.groups()
        return (f"attn_decode_kernel d{d} {'causal' if causal == 'true' else 'noncausal'} "
                f"{'fp16' if f16 == 'true' else 'bf16'} rowblocks{nrb}")
    m = BWD_RE.search(name)
    if m:
        which, d, causal, f16 = m.groups()
        return (f"attn_bwd_{which}_kernel d{d} {'causal' if causal == 'true' else 'noncausal'} "
                f"{'fp16' if f16 == 'true' else 'bf16'}")
    m = MERGE_RE.search(name)
    if m:
        return f"merge_splits_kernel d{m.group(1)} {'fp16' if m.group(2) == 'true' else 'bf16'}"
    if "quantize_kernel" in name:
        return "quantize_kernel (e4m3 prep)"
    if "neg" in name:
        return "copy (torch.neg, float32)"
    return name[:60]


def _rows(d: str, suffix: str):
    with open(_one(d, suffix)) as fh:
        return list(csv.DictReader(fh))


def assign_variants(rows, ws):
    """{Dispatch_Id: workload label} for the attention dispatches among ``rows``.

    bench.py launches the variants of a workload in one fixed order (warm-up, timed
    steps and cold runs alike), and variants may share a kernel instance and grid
    (the target workload's three sequence lengths do), so the k-th dispatch of the
    listed kernels belongs to variant k mod len(ws). The kernel names must follow
    that cycle, else the run is not a bench.py run of this workload."""
    keys = [variant_key(w) for w in ws]
    name_of = {}
    for r in rows:
        name = short_name(r["Kernel_Name"])
        if name in keys:
            name_of[int(r["Dispatch_Id"])] = name
    out = {}
    for i, did in enumerate(sorted(name_of)):
        if name_of[did] != keys[i % len(ws)]:
            raise ValueError(f"dispatch {did} ({name_of[did]}) breaks the launch order "
                             f"{keys} of the workload")
        out[did] = ws[i % len(ws)].label()
    return out


def trace_per_variant(d: str, ws):
    """Per workload variant: mean, min and max kernel duration (us) and launch count,
    from the kernel trace of a --kernel-trace run."""
    rows = _rows(d, "kernel_trace.csv")
    lab = assign_variants(rows, ws)
    durs = defaultdict(list)
    for r in rows:
        did = int(r["Dispatch_Id"])
        if did in lab:
            durs[lab[did]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: {"avg_us": sum(v) / len(v), "min_us": min(v), "max_us": max(v), "calls": len(v)}
            for k, v in durs.items()}


def kernel_stats(d: str):
    rows = []
    with open(_one(d, "kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def counter_per_dispatch(d: str, counter: str, ws=None):
    """Mean value of one counter per dispatch, by short kernel name and, when the
    workload's variants ``ws`` are given, also by variant label (dispatch order)."""
    rows = _rows(d, "counter_collection.csv")
    lab = assign_variants(rows, ws) if ws else {}
    vals = defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            v = float(r["Counter_Value"])
            vals[short_name(r["Kernel_Name"])].append(v)
            did = int(r["Dispatch_Id"])
            if did in lab:
                vals[lab[did]].append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def algorithmic_bytes(w) -> int:
    """Q, K, V read once, O and LSE written once (fp8: 1-byte inputs plus descales)."""
    if isinstance(w, synth.DecodeWorkload):
        return w.hbm_bytes()
    bh = w.B * w.H
    ins = w.N_q * w.d_qk + w.N_kv * w.d_qk + w.N_kv * w.d_v
    if w.fp8:
        nb = lambda n: (n + 127) // 128
        return bh * (ins + 4 * (nb(w.N_q) + 2 * nb(w.N_kv)) + 2 * w.N_q * w.d_v + 4 * w.N_q)
    return bh * (2 * ins + 2 * w.N_q * w.d_v + 4 * w.N_q)


TARGET_N = (4096, 8192, 16384)


def workloads_of(name: str):
    if name == "target":
        return [synth.workload("sweep", causal=c, N=n) for n in TARGET_N for c in (False, True)]
    if name == "bwd":
        return [synth.workload("single", causal=c) for c in (False, True)]
    if name == "decode":
        return [synth.decode_workload()]
    if name.startswith("sweep"):
        n = int(name[5:])
        return [synth.workload("sweep", causal=c, N=n) for c in (False, True)]
    if name in ("tiny", "asym", "fp8"):
        return [synth.workload(name)]
    return [synth.workload("single", causal=c) for c in (False, True)]


def variant_key(w) -> str:
    mask = "causal" if w.causal else "noncausal"
    if isinstance(w, synth.DecodeWorkload):
        rows = w.H // w.H_kv * w.N_q
        return f"attn_decode_kernel d{w.d} {mask} bf16 rowblocks{1 if rows <= 32 else 2 if rows <= 64 else 4}"
    if w.fp8:
        return f"attn_fwd_fp8_kernel d128x128 {mask} e4m3"
    return f"attn_fwd_kernel d{w.d_qk}x{w.d_v} {mask} tau8 bf16"


def bwd_keys(w):
    """Both backward kernels of one call (their counters are summed)."""
    mask = "causal" if w.causal else "noncausal"
    return [f"attn_bwd_{k}_kernel d{w.d_qk} {mask} bf16" for k in ("dq", "dkdv")]


def bwd_algorithmic_bytes(w) -> int:
    """Backward: Q, K, V, O, dO read once and LSE; dQ, dK, dV and D written once."""
    bh = w.B * w.H
    reads = 2 * (3 * w.N_q * w.d_qk + 2 * w.N_kv * w.d_qk) + 4 * w.N_q
    writes = 2 * (w.N_q * w.d_qk + 2 * w.N_kv * w.d_qk) + 4 * w.N_q
    return bh * (reads + writes)


def profile_stem(workload: str) -> str:
    """File stem of a workload's summary: the kernel it profiles, then the workload."""
    return {"decode": "attn_decode_splitkv", "bwd": "attn_bwd_single"}.get(workload,
                                                                       f"attn_fwd_{workload}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--bench-json", required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--commands", required=True)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()

    with open(args.bench_json) as fh:
        bench = json.loads(fh.read().strip().splitlines()[-1])
    with open(args.commands) as fh:
        commands = fh.read().strip()
    stats = kernel_stats(args.stats)
    ws = workloads_of(args.workload)
    fwd = args.workload not in ("bwd", "decode")
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE", ws if fwd else None)
    write = counter_per_dispatch(args.write, "WRITE_SIZE", ws if fwd else None)
    per_var = trace_per_variant(args.stats, ws) if fwd else {}
    copy_name = "copy (torch.neg, float32)"
    copy_bytes = args.copy_mib << 20
    f_fetch = copy_bytes / (fetch[copy_name][0] * 1024.0)
    f_write = copy_bytes / (write[copy_name][0] * 1024.0)

    ev = {p["variant"]: p for p in bench["per_variant"]}
    traffic = {}
    stem = profile_stem(args.workload)
    lines = [f"# {stem} (bench.py --workload {args.workload})", "",
             "Workload: " + " + ".join(w.label() for w in ws) + ".", "",
             "## Commands", "", "```", commands, "```", "",
             "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['name']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['pct']:.2f} |")
    if per_var:
        lines += ["", "Per variant, from the same kernel trace (dispatches attributed to the "
                  "variants in bench.py's launch order):", "",
                  "| variant | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for w in ws:
            t = per_var.get(w.label())
            if t:
                lines.append(f"| {w.label()} | {t['calls']} | {t['avg_us']:.2f} | "
                             f"{t['min_us']:.2f} | {t['max_us']:.2f} |")
    lines += ["", "bench.py's HIP-event average of the same launches (the run under --stats):", "",
              "| variant | avg us (events) | TFLOP/s (GB/s for decode) |", "|---|---|---|"]
    for p in bench["per_variant"]:
        rate = f"{p['tflops']:.1f}" if "tflops" in p else f"{p['gbps']:.0f} GB/s"
        lines.append(f"| {p['variant']} | {p['avg_launch_us']:.2f} | {rate} |")
    lines += ["", "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"Calibration: a float32 copy of {args.copy_mib} MiB reads and writes {copy_bytes} bytes; "
              f"its FETCH_SIZE reads {fetch[copy_name][0]:.0f} KiB and WRITE_SIZE "
              f"{write[copy_name][0]:.0f} KiB per dispatch, so bytes = KiB x {f_fetch * 1024:.1f} (fetch) "
              f"and KiB x {f_write * 1024:.1f} (write).", "",
              "| variant | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (scaled) | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|"]
    bwd = args.workload == "bwd"
    for w in ws:
        keys = bwd_keys(w) if bwd else [w.label() if fwd else variant_key(w)]
        if any(k not in fetch or k not in write for k in keys):
            continue
        fk = sum(fetch[k][0] for k in keys)
        wk = sum(write[k][0] for k in keys)
        fb = fk * 1024.0 * f_fetch
        wb = wk * 1024.0 * f_write
        alg = bwd_algorithmic_bytes(w) if bwd else algorithmic_bytes(w)
        label = ("bwd " if bwd else "") + w.label()
        traffic[label] = {"fetch_bytes": fb, "write_bytes": wb, "hbm_bytes": fb + wb,
                          "algorithmic_bytes": alg}
        lines.append(f"| {label} | {fk:.0f} | {wk:.0f} | {fb + wb:.4g} | "
                     f"{alg:.4g} | {(fb + wb) / alg:.3f} |")
    lines.append("")
    os.makedirs(args.out, exist_ok=True)
    with open(os.path.join(args.out, f"{stem}.md"), "w") as fh:
        fh.write("\n".join(lines))
    dom = bench["roofline"]["kernel"]
    dom_variant = dom[dom.index("(") + 1:-1]
    rec = {"workload": args.workload, "kernel_source_sha": bench["kernel_source_sha"],
           "dominant_variant": dom_variant,
           "hbm_bytes_per_launch": traffic.get(dom_variant, {}).get("hbm_bytes"),
           "trace_avg_us_per_variant": {k: round(v["avg_us"], 3) for k, v in per_var.items()},
           "per_variant": traffic, "copy_factor_fetch": f_fetch, "copy_factor_write": f_write}
    with open(os.path.join(args.out, f"{stem}_traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
