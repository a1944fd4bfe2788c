"""Summarise rocprofv3 hardware-counter runs of a bench.py workload into profiles/.

    python -m exact_attention_81_amd.counter_report --workload single \\
        --pmc RUN/pass1 RUN/pass2 --commands RUN/commands.txt

Each ``--pmc`` directory is a ``rocprofv3 --pmc ... --kernel-trace --stats
--output-format csv`` run of ``bench.py --workload W``; the first one's kernel
trace gives the launch durations. Counters are averaged per dispatch and kernel.
Derived figures (each formula is printed beside it in the summary):

* matrix-core busy: rocprofv3's ``MfmaUtil`` (MFMA-busy cycles of all SIMDs over
  elapsed cycles times the SIMD count);
* executed matrix flops: 512 x ``SQ_INSTS_VALU_MFMA_MOPS_*``, against the counted
  flops of the metric (2 B H N_q N_kv (d_qk + d_v), halved when causal);
* shader clock: elapsed ``GRBM_GUI_ACTIVE`` cycles over the traced duration, and the
  matrix-core rate at that clock. The counter runs once per XCD and the CSV holds
  the sum of the 8 instances (``MfmaUtil`` takes their maximum), so the elapsed
  cycles are the sum over 8; the clock so obtained makes ``MfmaUtil`` agree with
  the executed matrix rate over the peak at that clock;
* vector ALU: ``VALUBusy``, instructions and transcendental (exp/log/rcp)
  instructions per score (a wave instruction covers 64 lanes);
* LDS: ``LdsUtil``, bank-conflict cycles as a share of GPU time
  (``LDSBankConflict``) and per LDS-active cycle (``LdsBankConflict``).

Writes ``profiles/<stem>_counters.md`` with the commands that made it, and
``profiles/<stem>_counters.json`` (the headline figures per variant and the kernel
source hash of the run, read by bench.py).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
from collections import defaultdict

from .profile_report import (ROOT, assign_variants, bwd_keys, kernel_stats, profile_stem, short_name,
                             trace_per_variant, variant_key, workloads_of)

CUS = 256            # MI355X compute units
XCDS = 8             # GRBM_GUI_ACTIVE instances summed in the CSV
MFMA_FLOP_PER_CLK_CU = {"bf16": 4096, "fp8": 8192}


def counters(dirs, ws=None):
    """{short kernel name: {counter: mean value per dispatch}} over all runs; with the
    workload's variants ``ws`` also keyed by variant label (dispatch order)."""
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(path) as fh:
                rows = list(csv.DictReader(fh))
            lab = assign_variants(rows, ws) if ws else {}
            for r in rows:
                v = float(r["Counter_Value"])
                vals[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(v)
                did = int(r["Dispatch_Id"])
                if did in lab:
                    vals[lab[did]][r["Counter_Name"]].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}


def counted_flops(w) -> float:
    """The metric's flop count of one launch (R5; the backward's five products)."""
    dqk, dv = getattr(w, "d_qk", None) or w.d, getattr(w, "d_v", None) or w.d
    f = 2.0 * w.B * w.H * w.N_q * w.N_kv * (dqk + dv)
    return f * (0.5 if w.causal else 1.0)


def scores(w) -> float:
    n = float(w.B * w.H * w.N_q * w.N_kv)
    return n * (0.5 if w.causal else 1.0)


def fmt(x, spec=".3g"):
    return "n/a" if x is None else format(x, spec)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--pmc", nargs="+", required=True)
    ap.add_argument("--commands", required=True)
    ap.add_argument("--bench-json", default=None,
                    help="bench.py's output of the first pass (gives the kernel source hash)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()

    stats = {r["name"]: r for r in kernel_stats(args.pmc[0])}
    ws_all = workloads_of(args.workload)
    fwd = args.workload not in ("bwd", "decode")
    cnt = counters(args.pmc, ws_all if fwd else None)
    if fwd:  # per-variant durations from the kernel trace (variants may share a kernel)
        stats.update({k: v for k, v in trace_per_variant(args.pmc[0], ws_all).items()})
    with open(args.commands) as fh:
        commands = fh.read().strip()
    stem = profile_stem(args.workload) + "_counters"
    lines = [f"# {stem} (bench.py --workload {args.workload})", "",
             "Hardware counters of the workload's kernels, averaged per dispatch "
             "(rocprofv3 derived metrics where it defines one).", "",
             "## Commands", "", "```", commands, "```", ""]

    bwd = args.workload == "bwd"
    record = {}  # per variant key: the figures bench.py attaches to its line
    for w in ws_all:
        keys = bwd_keys(w) if bwd else [w.label() if fwd else variant_key(w)]
        for key in keys:
            c = cnt.get(key)
            if c is None:
                continue
            st = stats.get(key)
            dur_us = st["avg_us"] if st else None
            get = c.get
            prec = "fp8" if "fp8" in key else "bf16"
            mops = sum(get(f"SQ_INSTS_VALU_MFMA_MOPS_{t}", 0.0) for t in ("BF16", "F16", "F8"))
            exec_flops = 512.0 * mops if mops else None
            alg = counted_flops(w)
            if bwd:
                alg = None  # the two kernels split the five products unevenly
            gui = get("GRBM_GUI_ACTIVE")
            clock_ghz = gui / XCDS / (dur_us * 1e3) if gui and dur_us else None
            peak_at_clock = (clock_ghz * 1e9 * CUS * MFMA_FLOP_PER_CLK_CU[prec] / 1e12
                             if clock_ghz else None)
            rate = exec_flops / (dur_us * 1e-6) / 1e12 if exec_flops and dur_us else None
            sc = scores(w)
            valu_per_score = get("SQ_INSTS_VALU") * 64 / sc if get("SQ_INSTS_VALU") else None
            trans_per_score = get("SQ_INSTS_VALU_TRANS_F32") * 64 / sc if get("SQ_INSTS_VALU_TRANS_F32") else None
            coexec = (get("SQ_VALU_MFMA_COEXEC_CYCLES") / get("SQ_VALU_MFMA_BUSY_CYCLES")
                      if get("SQ_VALU_MFMA_COEXEC_CYCLES") and get("SQ_VALU_MFMA_BUSY_CYCLES") else None)
            r1 = lambda v: None if v is None else round(v, 1)
            record[w.label() if not bwd else f"{key} ({w.label()})"] = {
                "clock_ghz": None if clock_ghz is None else round(clock_ghz, 3),
                "mfma_busy_pct": r1(get("MfmaUtil")),
                "rate_over_peak_at_clock_pct": (round(rate / peak_at_clock * 100, 1)
                                                if rate and peak_at_clock else None),
                "valu_busy_pct": r1(get("VALUBusy")),
                "lds_bank_conflict_pct": r1(get("LDSBankConflict")),
                "executed_over_counted": (round(exec_flops / alg, 4) if exec_flops and alg else None)}
            lines += [f"## {variant_key(w) if fwd else key} ({w.label()})", "",
                      "| figure | value | how |", "|---|---|---|",
                      f"| duration | {fmt(dur_us, '.1f')} us | kernel trace of the first pass |",
                      f"| matrix cores busy | {fmt(get('MfmaUtil'), '.1f')} % | MfmaUtil = "
                      "sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) |",
                      f"| executed matrix flops | {fmt(exec_flops, '.4g')} | 512 x SQ_INSTS_VALU_MFMA_MOPS |",
                      f"| counted flops (metric) | {fmt(alg, '.4g')} | 2 B H N_q N_kv (d_qk + d_v), x 0.5 causal |",
                      f"| executed / counted | {fmt(exec_flops / alg if exec_flops and alg else None, '.3f')} | |",
                      f"| executed matrix rate | {fmt(rate, '.1f')} TFLOP/s | executed flops / duration |",
                      f"| GRBM_GUI_ACTIVE | {fmt(gui, '.4g')} cycles | elapsed GPU cycles, summed over the {XCDS} XCDs |",
                      f"| shader clock | {fmt(clock_ghz, '.3f')} GHz | GRBM_GUI_ACTIVE / {XCDS} / duration |",
                      f"| {prec} peak at that clock | {fmt(peak_at_clock, '.0f')} TFLOP/s | clock x {CUS} CUs x "
                      f"{MFMA_FLOP_PER_CLK_CU[prec]} flop/clk |",
                      f"| executed rate / peak at clock | {fmt(rate / peak_at_clock * 100 if rate and peak_at_clock else None, '.1f')} % | |",
                      f"| vector ALU busy | {fmt(get('VALUBusy'), '.1f')} % | VALUBusy = sum SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE |",
                      f"| MFMA cycles with a co-issued VALU op | {fmt(coexec * 100 if coexec else None, '.1f')} % | "
                      "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES |",
                      f"| VALU instructions per score | {fmt(valu_per_score, '.2f')} | SQ_INSTS_VALU x 64 / scores |",
                      f"| transcendental instructions per score | {fmt(trans_per_score, '.3f')} | "
                      "SQ_INSTS_VALU_TRANS_F32 x 64 / scores (one exp2 per score, plus rescales) |",
                      f"| MFMA instructions | {fmt(get('SQ_INSTS_MFMA'), '.4g')} | SQ_INSTS_MFMA |",
                      f"| LDS instructions | {fmt(get('SQ_INSTS_LDS'), '.4g')} | SQ_INSTS_LDS |",
                      f"| LDS busy | {fmt(get('LdsUtil'), '.1f')} % | LdsUtil = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE x CUs) |",
                      f"| LDS bank-conflict cycles, share of GPU time | {fmt(get('LDSBankConflict'), '.2f')} % | "
                      "LDSBankConflict |",
                      f"| LDS bank-conflict cycles per conflict-free LDS cycle | {fmt(get('LdsBankConflict'), '.4f')} | "
                      "LdsBankConflict |",
                      ""]
    os.makedirs(args.out, exist_ok=True)
    path = os.path.join(args.out, f"{stem}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    sha = None
    if args.bench_json:
        with open(args.bench_json) as fh:
            sha = json.loads(fh.read().strip().splitlines()[-1]).get("kernel_source_sha")
    with open(os.path.join(args.out, f"{stem}.json"), "w") as fh:
        json.dump({"workload": args.workload, "kernel_source_sha": sha, "per_variant": record}, fh,
                  indent=1)
    print(path)


if __name__ == "__main__":
    main()
