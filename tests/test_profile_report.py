"""profile_report: parsing of rocprofv3 CSV output and the copy calibration."""
import csv
import json
import os

from exact_attention_81_amd import profile_report, synth

KNAME = "void exattn::(anonymous namespace)::attn_fwd_kernel<128, 128, {c}, 8, false, false>(exattn::FwdParams)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>(...)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_short_names():
    assert profile_report.short_name(KNAME.format(c="true")) == \
        "attn_fwd_kernel d128x128 causal tau8 bf16"
    assert profile_report.short_name(
        "void exattn::(anonymous namespace)::attn_fwd_fp8_kernel<false>(exattn::FwdParams)") == \
        "attn_fwd_fp8_kernel d128x128 noncausal e4m3"
    assert profile_report.short_name(COPY) == "copy (torch.neg, float32)"
    assert profile_report.short_name(KNAME.replace("false, false>", "false, true>").format(c="false")) \
        == "attn_fwd_kernel d128x128 noncausal tau8 bf16 strided"
    assert profile_report.short_name(
        "void exattn::(anonymous namespace)::attn_decode_kernel<128, false, false, 1>"
        "(exattn::DecodeParams)") == "attn_decode_kernel d128 noncausal bf16 rowblocks1"
    assert profile_report.short_name(
        "void exattn::(anonymous namespace)::merge_splits_kernel<64, true>(float const*, "
        "float const*, void*, float*, int, int)") == "merge_splits_kernel d64 fp16"
    w = synth.decode_workload()
    assert profile_report.variant_key(w) == "attn_decode_kernel d128 noncausal bf16 rowblocks1"


def test_algorithmic_bytes():
    dw = synth.decode_workload()
    assert profile_report.algorithmic_bytes(dw) == (2 * 8 * 8 * 16384 * 128 * 2
                                                    + 2 * 8 * 64 * 1 * 128 * 2 + 4 * 8 * 64)
    w = synth.workload("single", causal=False)
    assert profile_report.algorithmic_bytes(w) == 4 * 16 * (2048 * 128 * 2 * 4 + 2048 * 4)
    f = synth.workload("fp8")
    bh = 4 * 16
    assert profile_report.algorithmic_bytes(f) == bh * (4096 * 128 * 3 + 4 * 3 * 32 + 2 * 4096 * 128 + 4 * 4096)


TRACE_HEAD = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def test_report_end_to_end(tmp_path):
    d = str(tmp_path)
    _write(f"{d}/stats/run_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[KNAME.format(c="false"), 2, 2.6e5, 1.3e5, 60.0, 1.25e5, 1.35e5, 1.0],
            [KNAME.format(c="true"), 2, 1.7e5, 0.85e5, 40.0, 0.8e5, 0.9e5, 1.0]])
    _write(f"{d}/stats/run_kernel_trace.csv", TRACE_HEAD,
           [["KERNEL_DISPATCH", 1, KNAME.format(c="false"), 1000, 126000],
            ["KERNEL_DISPATCH", 2, KNAME.format(c="true"), 130000, 210000],
            ["KERNEL_DISPATCH", 3, KNAME.format(c="false"), 300000, 435000],
            ["KERNEL_DISPATCH", 4, KNAME.format(c="true"), 440000, 530000]])
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    mib = 1024
    # the copy reads and writes 1 GiB; FETCH_SIZE shows half of it (as on the box)
    _write(f"{d}/fetch/run_counter_collection.csv", head,
           [[1, KNAME.format(c="false"), "FETCH_SIZE", 49000.0],
            [2, KNAME.format(c="true"), "FETCH_SIZE", 74000.0],
            [3, KNAME.format(c="false"), "FETCH_SIZE", 50000.0],
            [4, COPY, "FETCH_SIZE", mib * 1024 / 2]])
    _write(f"{d}/write/run_counter_collection.csv", head,
           [[1, KNAME.format(c="false"), "WRITE_SIZE", 33280.0],
            [2, KNAME.format(c="true"), "WRITE_SIZE", 33280.0],
            [3, COPY, "WRITE_SIZE", mib * 1024]])
    w0 = synth.workload("single", causal=False)
    w1 = synth.workload("single", causal=True)
    bench = {"kernel_source_sha": "abc", "roofline": {"kernel": f"attn_fwd_kernel ({w0.label()})"},
             "per_variant": [{"variant": w0.label(), "avg_launch_us": 131.0, "tflops": 1000.0},
                             {"variant": w1.label(), "avg_launch_us": 86.0, "tflops": 800.0}]}
    with open(f"{d}/bench.json", "w") as fh:
        fh.write("noise\n" + json.dumps(bench) + "\n")
    with open(f"{d}/commands.txt", "w") as fh:
        fh.write("python3 bench.py\n")
    out = f"{d}/profiles"
    import sys
    argv = sys.argv
    sys.argv = ["profile_report", "--workload", "single", "--bench-json", f"{d}/bench.json",
                "--stats", f"{d}/stats", "--fetch", f"{d}/fetch", "--write", f"{d}/write",
                "--copy-mib", str(mib), "--commands", f"{d}/commands.txt", "--out", out]
    try:
        profile_report.main()
    finally:
        sys.argv = argv
    rec = json.load(open(f"{out}/attn_fwd_single_traffic.json"))
    assert rec["copy_factor_fetch"] == 2.0 and rec["copy_factor_write"] == 1.0
    assert rec["kernel_source_sha"] == "abc"
    assert rec["dominant_variant"] == w0.label()
    assert rec["hbm_bytes_per_launch"] == 49500.0 * 1024 * 2 + 33280.0 * 1024
    assert rec["trace_avg_us_per_variant"] == {w0.label(): 130.0, w1.label(): 85.0}
    text = open(f"{out}/attn_fwd_single.md").read()
    assert "python3 bench.py" in text and "| 2 |" in text


def test_variants_sharing_a_kernel_follow_launch_order():
    """The target workload's three sequence lengths run the same kernel instance on the
    same grid: dispatches are attributed by bench.py's launch order, and a trace that
    does not follow it is refused."""
    import pytest

    ws = profile_report.workloads_of("target")
    assert [w.N_q for w in ws] == [4096, 4096, 8192, 8192, 16384, 16384]
    rows = []
    for step in range(3):
        for i, w in enumerate(ws):
            rows.append({"Dispatch_Id": str(100 + 6 * step + i),
                         "Kernel_Name": KNAME.format(c="true" if w.causal else "false")})
    rows.insert(4, {"Dispatch_Id": "50", "Kernel_Name": COPY})  # other kernels are ignored
    lab = profile_report.assign_variants(rows, ws)
    assert len(lab) == 18
    assert lab[100] == ws[0].label() and lab[104] == ws[4].label() and lab[117] == ws[5].label()
    bad = [dict(r) for r in rows if r["Kernel_Name"] != COPY]
    bad[1]["Kernel_Name"] = KNAME.format(c="false")   # two non-causal launches in a row
    with pytest.raises(ValueError):
        profile_report.assign_variants(bad, ws)


def test_counter_report_end_to_end(tmp_path):
    """Derived counter figures: executed flops from MOPS, the clock from the summed
    GRBM_GUI_ACTIVE of the 8 XCDs, and per-score instruction counts."""
    from exact_attention_81_amd import counter_report
    d = str(tmp_path)
    w = synth.workload("single", causal=False)
    flops = 2.0 * 4 * 16 * 2048 * 2048 * 256
    dur_ns = 1.25e5
    _write(f"{d}/p1/run_kernel_stats.csv",
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[KNAME.format(c="false"), 2, 2 * dur_ns, dur_ns, 100.0, dur_ns, dur_ns, 0.0]])
    k = KNAME.format(c="false")
    kc = KNAME.format(c="true")
    _write(f"{d}/p1/run_kernel_trace.csv", TRACE_HEAD,
           [["KERNEL_DISPATCH", 1, k, 0, int(dur_ns)], ["KERNEL_DISPATCH", 2, kc, 200000, 290000]])
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # 2.0 GHz for 125 us = 250000 cycles per XCD, summed over 8
    _write(f"{d}/p1/run_counter_collection.csv", head,
           [[1, k, "MfmaUtil", 50.0], [1, k, "GRBM_GUI_ACTIVE", 8 * 250000.0], [1, k, "VALUBusy", 40.0],
            [1, k, "LdsUtil", 20.0], [1, k, "LDSBankConflict", 0.0], [1, k, "LdsBankConflict", 0.0],
            [2, kc, "MfmaUtil", 30.0]])
    scores = 4 * 16 * 2048 * 2048
    _write(f"{d}/p2/run_counter_collection.csv", head,
           [[1, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", flops / 512], [1, k, "SQ_INSTS_VALU_TRANS_F32", scores / 64],
            [1, k, "SQ_INSTS_VALU", 5 * scores / 64], [1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1000.0],
            [1, k, "SQ_VALU_MFMA_COEXEC_CYCLES", 400.0], [2, kc, "SQ_INSTS_VALU", 1.0]])
    with open(f"{d}/commands.txt", "w") as fh:
        fh.write("rocprofv3 --pmc ...\n")
    import sys
    argv = sys.argv
    sys.argv = ["counter_report", "--workload", "single", "--pmc", f"{d}/p1", f"{d}/p2",
                "--commands", f"{d}/commands.txt", "--out", f"{d}/out"]
    try:
        counter_report.main()
    finally:
        sys.argv = argv
    text = open(f"{d}/out/attn_fwd_single_counters.md").read()
    sect = text[text.index(w.label()):]
    sect = sect[:sect.index("## ", 3)] if "## " in sect[3:] else sect
    rows = {r.split("|")[1].strip(): r.split("|")[2].strip() for r in sect.splitlines()
            if r.startswith("| ")}
    assert rows["executed / counted"] == "1.000"
    assert rows["shader clock"] == "2.000 GHz"
    assert rows["transcendental instructions per score"] == "1.000"
    assert rows["VALU instructions per score"] == "5.00"
    assert rows["MFMA cycles with a co-issued VALU op"] == "40.0 %"
    rate = flops / (dur_ns * 1e-9) / 1e12
    assert rows["executed rate / peak at clock"] == format(rate / (2.0 * 256 * 4096 / 1e3) * 100, ".1f") + " %"
    rec = json.load(open(f"{d}/out/attn_fwd_single_counters.json"))
    fig = rec["per_variant"][w.label()]
    assert rec["kernel_source_sha"] is None  # no bench output given
    assert fig["clock_ghz"] == 2.0 and fig["mfma_busy_pct"] == 50.0 and fig["executed_over_counted"] == 1.0
