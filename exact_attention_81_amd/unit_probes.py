"""Runs the gfx950 unit-rate probes of libexattn_probes.so and prints what they measure.

    python -m exact_attention_81_amd.unit_probes [--json]

Four questions the attention kernels' design depends on:

  * Do the hardware exponential (v_exp_f32) and the FMA (v_fma_f32) issue side by
    side? For each mix of independent exponential and FMA chains the probe reports
    cycles per wave instruction per SIMD; the table compares the mixed loop with the
    two bounds its parts predict: max(exp, fma) if they overlapped, exp + fma if they
    share issue.
  * How fast can a wave read LDS, alone and beside its own matrix-core stream? Bytes
    per clock per CU for ds_read_b128 and ds_read_b64_tr_b16, and cycles per
    v_mfma_f32_32x32x16_bf16 when every product is fed by 1 KB of LDS reads in the
    same wave, at one and two waves per SIMD; with the reads drained every 8 steps, and
    with reads kept in flight across steps (8 deep, or 4 products ahead of the
    product that uses them).
  * What clock does the chip hold under a pure matrix-core load? A stream of
    v_mfma_f32_32x32x16_bf16 (or the e4m3 v_mfma_f32_32x32x64_f8f6f4) on every SIMD with
    constant and with pseudo-random operands: the rate and clock the attention
    kernels' power budget is set against.
  * How fast can a plain kernel stream reads from HBM? A grid-stride loop of 16-byte
    loads over 1 GiB, at 1 to 8 workgroups per CU and 1 to 8 loads in flight per
    thread: the reference for the split-KV decode, which is bound by its K/V reads.

Needs a GPU; the library is built by ``build.build_probes()``.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libexattn_probes.so")
SYMBOLS = ("probe_exp_fma", "probe_lds", "probe_stream_read", "probe_mfma_clock")

EXP_FMA_MIXES = ((8, 0), (0, 8), (0, 16), (8, 8), (8, 16), (8, 24), (16, 16))
STREAM_WG_PER_CU = (1, 2, 4, 8)
STREAM_IN_FLIGHT = (1, 4, 8)
LDS_MODES = {0: "ds_read_b128", 1: "ds_read_b64_tr_b16 x2", 2: "mfma 32x32x16 bf16 only",
             3: "mfma + ds_read_b128", 4: "mfma + ds_read_b64_tr_b16 x2",
             5: "ds_read_b128, 8 in flight", 6: "mfma fed by ds_read_b128 issued 4 ahead"}


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run exact_attention_81_amd.build.build_probes()")
    lib = ctypes.CDLL(LIB_PATH)
    for name in SYMBOLS:
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
    lib.probe_exp_fma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.POINTER(ctypes.c_double)]
    lib.probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.probe_stream_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.probe_mfma_clock.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    return lib


def _call(fn, *args):
    out = (ctypes.c_double * 3)()
    rc = fn(*args, out)
    if rc != 0:
        raise RuntimeError(f"{fn.__name__}{args} failed with code {rc}")
    return list(out)


def run() -> dict:
    lib = load()
    res = {"exp_fma": [], "lds": [], "stream_read": [], "mfma_clock": []}
    for wps in (1, 2):
        for ne, nf in EXP_FMA_MIXES:
            per_instr, ghz, _ = _call(lib.probe_exp_fma, ne, nf, wps)
            res["exp_fma"].append({"waves_per_simd": wps, "exp": ne, "fma": nf,
                                   "cycles_per_instr": per_instr,
                                   "cycles_per_iter": per_instr * (ne + nf), "ghz": ghz})
        for mode, name in LDS_MODES.items():
            bpc, mfma_cyc, ghz = _call(lib.probe_lds, mode, wps)
            res["lds"].append({"waves_per_simd": wps, "mode": name,
                               "lds_bytes_per_clk_cu": bpc if mode != 2 else None,
                               "cycles_per_mfma": mfma_cyc if mode in (2, 3, 4, 6) else None,
                               "ghz": ghz})
    for kind, name in enumerate(("bf16, constant", "bf16, pseudo-random", "e4m3, constant",
                                 "e4m3, pseudo-random")):
        tf, ghz, frac = _call(lib.probe_mfma_clock, kind)
        res["mfma_clock"].append({"operands": name, "tflops": tf, "ghz": ghz, "of_peak_at_clock": frac})
    for wpc in STREAM_WG_PER_CU:
        for u in STREAM_IN_FLIGHT:
            best, mean, grid = _call(lib.probe_stream_read, wpc, u)
            res["stream_read"].append({"wg_per_cu": wpc, "in_flight": u, "best_gbs": best,
                                       "mean_gbs": mean, "grid": int(grid)})
    return res


def report(res: dict) -> str:
    lines = ["exp / FMA mixes (cycles per wave instruction per SIMD):", "",
             "| waves/SIMD | exp | fma | cyc/instr | cyc/iter | if overlapped | if shared |",
             "|---|---|---|---|---|---|---|"]
    for wps in (1, 2):
        rows = [r for r in res["exp_fma"] if r["waves_per_simd"] == wps]
        solo = {(r["exp"], r["fma"]): r["cycles_per_instr"] for r in rows}
        e1 = solo.get((8, 0))
        f1 = solo.get((0, 16), solo.get((0, 8)))
        for r in rows:
            ne, nf = r["exp"], r["fma"]
            over = shared = ""
            if ne and nf and e1 and f1:
                over = f"{max(ne * e1, nf * f1):.1f}"
                shared = f"{ne * e1 + nf * f1:.1f}"
            lines.append(f"| {wps} | {ne} | {nf} | {r['cycles_per_instr']:.2f} | "
                         f"{r['cycles_per_iter']:.1f} | {over} | {shared} |")
    lines += ["", "LDS reads and matrix-core products:", "",
              "| waves/SIMD | loop | LDS B/clk/CU | cycles per MFMA per SIMD |", "|---|---|---|---|"]
    for r in res["lds"]:
        b = "" if r["lds_bytes_per_clk_cu"] is None else f"{r['lds_bytes_per_clk_cu']:.1f}"
        c = "" if r["cycles_per_mfma"] is None else f"{r['cycles_per_mfma']:.1f}"
        lines.append(f"| {r['waves_per_simd']} | {r['mode']} | {b} | {c} |")
    lines += ["", "Sustained MFMA stream (v_mfma_f32_32x32x16_bf16 / 32x32x64_f8f6f4, two waves per SIMD):", "",
              "| operands | TFLOP/s | shader clock | of the peak at that clock |", "|---|---|---|---|"]
    for r in res["mfma_clock"]:
        lines.append(f"| {r['operands']} | {r['tflops']:.0f} | {r['ghz']:.2f} GHz | {100 * r['of_peak_at_clock']:.1f} % |")
    lines += ["", "HBM streaming read over 1 GiB (GB/s, best and mean of five passes):", "",
              "| workgroups per CU | loads in flight per thread | best | mean |", "|---|---|---|---|"]
    for r in res["stream_read"]:
        lines.append(f"| {r['wg_per_cu']} | {r['in_flight']} | {r['best_gbs']:.0f} | {r['mean_gbs']:.0f} |")
    ghz = sorted({round(r["ghz"], 2) for r in res["exp_fma"] + res["lds"]})
    lines += ["", f"shader clock during the probes: {', '.join(str(g) for g in ghz)} GHz"]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--json", action="store_true")
    args = ap.parse_args()
    res = run()
    print(json.dumps(res) if args.json else report(res))


if __name__ == "__main__":
    main()
