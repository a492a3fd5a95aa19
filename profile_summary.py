#!/usr/bin/env python3
"""Summaries of rocprofv3 runs of bench.py's profiling loops.

    python3 profile_summary.py DIR

DIR holds the rocprofv3 output directories and logs of the commands listed
in profiles/*.md (kernel traces and --pmc counter passes of
`bench.py --profile-loop ...`, `bench.py --kernel-loop ...` and
`bench.py --calibrate-copy`).  Each loop's launches are found by position:
the loop prints its first launch index, untimed warm-up launches and timed
launches, and only the library's own kernels are counted (the cache flush,
copies and fills torch issues are skipped).  Writes, for the current
kernel sources (their hash keys every entry; bench.py ignores entries of
other sources):
  profiles/kernel_medians.json  per-loop kernel durations (median, mean)
  profiles/traffic.json         HBM bytes per launch from FETCH_SIZE /
                                WRITE_SIZE, scaled by what the same counters
                                read for a plain copy of known size
  profiles/mfma_counters.json   MFMA-busy figures of the M = 256 GEMMs
and prints the tables the profiles/*.md summaries quote.
"""
from __future__ import annotations

import collections
import csv
import json
import os
import statistics as st
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (bench.py: algorithmic bytes, source hashes)

PROFILES = os.path.join(ROOT, "profiles")
CLOCK_GHZ = 2.4
SIMDS = 256 * 4
XCDS = 8


def loops(log):
    """The JSON lines a bench.py profiling run printed (loop bookkeeping)."""
    out = []
    with open(log) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and ("profile_loop" in line or "kernel_loop" in line or "calibrate_copy" in line):
                out.append(json.loads(line))
    return out


def ours(name):
    return "mi::" in name and "relayout" not in name


def by_dispatch(d, counters):
    """Dispatches of the library's kernels in launch order: (name, start,
    end, {counter: value})."""
    fn = "k_counter_collection.csv" if counters else "k_kernel_trace.csv"
    rows = [r for r in csv.DictReader(open(os.path.join(d, fn))) if ours(r["Kernel_Name"])]
    acc = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        e = acc.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "start": int(r["Start_Timestamp"]),
                                                    "end": int(r["End_Timestamp"]), "c": {}})
        if counters:
            e["c"][r["Counter_Name"]] = float(r["Counter_Value"])
    return list(acc.values())


def split(ds, lp):
    """Timed dispatches of each loop, by position."""
    out, i = {}, 0
    for l in lp:
        name = l.get("profile_loop") or l.get("kernel_loop")
        n = l["warmup_launches"] + l["launches"]
        out[name] = ds[i + l["warmup_launches"]:i + n]
        i += n
    if i != len(ds):
        raise SystemExit(f"{len(ds)} dispatches, loops account for {i}")
    return out


def short(name):
    """Kernel name with its template arguments, without namespace and
    parameter list."""
    n = name.replace("void mi::(anonymous namespace)::", "")
    return n[:n.rindex("(")] if "(" in n else n


def calibration(d_fetch, d_write):
    """HBM bytes per counter unit: a 64 MiB copy (bench.py --calibrate-copy)
    reads and writes 64 MiB."""
    res = {}
    for key, d in (("FETCH_SIZE", d_fetch), ("WRITE_SIZE", d_write)):
        rows = [r for r in csv.DictReader(open(os.path.join(d, "k_counter_collection.csv")))
                if r["Counter_Name"] == key and not ours(r["Kernel_Name"])]
        vals = sorted(float(r["Counter_Value"]) for r in rows)
        big = [v for v in vals if v > 0.5 * vals[-1]]
        med = st.median(big)
        res[key] = {"KiB_per_copy": med, "factor": round((64 << 20) / (med * 1024), 4), "copies": len(big)}
    return res


def main(d):
    nq_sha = bench.source_sha(*bench.NORMQUANT_SOURCES)
    gemm_sha = bench.source_sha(*bench.GEMM_SOURCES)
    K, NA, NB = 1536, 24576, 8192
    spec = {  # loop -> (kernel key, M, algorithmic bytes, sha)
        "gemm_a256": ("block_scaled_fp8_gemm_W_a", 256, bench.algorithmic_bytes_gemm(256, NA, K), gemm_sha),
        "gemm_b256": ("block_scaled_fp8_gemm_W_b", 256, bench.algorithmic_bytes_gemm(256, NB, K), gemm_sha),
        "gemm_a256_e8m0": ("block_scaled_fp8_gemm_W_a_e8m0", 256,
                           bench.algorithmic_bytes_gemm(256, NA, K) - 3 * (256 * 12 + NA // 128 * 12), gemm_sha),
        "gemm_b256_e8m0": ("block_scaled_fp8_gemm_W_b_e8m0", 256,
                           bench.algorithmic_bytes_gemm(256, NB, K) - 3 * (256 * 12 + NB // 128 * 12), gemm_sha),
        "pair64": ("block_scaled_fp8_gemm_pair", 64, bench.algorithmic_bytes_gemm_pair(64, NA, NB, K), gemm_sha),
        "tp8pair1": ("block_scaled_fp8_gemm_pair_tp8", 1, bench.algorithmic_bytes_gemm_pair(1, NA // 8, NB // 8, K),
                     gemm_sha),
        "nq8192_row": ("fused_dual_rmsnorm_group_quant_row", 8192, bench.algorithmic_bytes_normquant(8192), nq_sha),
        "nq8192_col": ("fused_dual_rmsnorm_group_quant_col", 8192, bench.algorithmic_bytes_normquant(8192), nq_sha),
        "normquant": ("fused_dual_rmsnorm_group_quant", 64, bench.algorithmic_bytes_normquant(64), nq_sha),
        "step": ("normquant_gemm_pair", 1, bench.algorithmic_bytes_normquant(1) +
                 bench.algorithmic_bytes_gemm_pair(1, NA, NB, K), gemm_sha),
        "nq1": ("fused_dual_rmsnorm_group_quant_M1", 1, bench.algorithmic_bytes_normquant(1), nq_sha),
    }
    P = lambda *a: os.path.join(d, *a)
    medians = {}
    print("## kernel durations (rocprofv3 kernel trace, timed launches)\n")
    print("| loop | kernel | launches | median us | mean us | min us | GB/s (median) |")
    print("|---|---|---|---|---|---|---|")
    for tdir, log, tag in (("trace_loops", "trace_loops.log", ""), ("trace_nq1cold", "trace_nq1cold.log", "_cold"),
                           ("trace_nq1warm", "trace_nq1warm.log", "_warm")):
        if not os.path.isdir(P(tdir)):
            continue
        for name, ds in split(by_dispatch(P(tdir), False), loops(P(log))).items():
            durs = [(e["end"] - e["start"]) / 1000 for e in ds]
            key, M, nbytes, sha = spec[name]
            med = st.median(durs)
            medians[name + tag] = {"kernel": short(ds[0]["name"]), "source_sha": sha, "M": M, "launches": len(durs),
                                   "median_us": round(med, 3), "mean_us": round(st.mean(durs), 3),
                                   "min_us": round(min(durs), 3)}
            print(f"| {name}{tag} | `{short(ds[0]['name'])}` | {len(durs)} | {med:.3f} | {st.mean(durs):.3f} | "
                  f"{min(durs):.3f} | {nbytes / med / 1e3:.1f} |")
    with open(os.path.join(PROFILES, "kernel_medians.json"), "w") as f:
        json.dump(medians, f, indent=1)

    cal = calibration(P("pmc_calib_FETCH_SIZE"), P("pmc_calib_WRITE_SIZE"))
    print(f"\ncalibration (64 MiB copy): {json.dumps(cal)}\n")
    traffic = {}
    print("## HBM traffic per launch (FETCH_SIZE / WRITE_SIZE, scaled by the copy calibration)\n")
    print("| loop | kernel | FETCH KiB | WRITE KiB | HBM bytes | algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|")
    for base in ("pmc_loops", "pmc_nq64", "pmc_step1"):
        if not os.path.isdir(P(base + "_FETCH_SIZE")):
            continue
        fe = split(by_dispatch(P(base + "_FETCH_SIZE"), True), loops(P(base + "_FETCH_SIZE.log")))
        wr = split(by_dispatch(P(base + "_WRITE_SIZE"), True), loops(P(base + "_WRITE_SIZE.log")))
        for name in fe:
            key, M, nbytes, sha = spec[name]
            fk = st.median(e["c"]["FETCH_SIZE"] for e in fe[name])
            wk = st.median(e["c"]["WRITE_SIZE"] for e in wr[name])
            rd = fk * 1024 * cal["FETCH_SIZE"]["factor"]
            wb = wk * 1024 * cal["WRITE_SIZE"]["factor"]
            traffic[key] = {"kernel": key, "loop": name, "source_sha": sha, "M": M,
                            "bytes_per_launch": int(rd + wb), "read_bytes": int(rd), "write_bytes": int(wb),
                            "algorithmic_bytes": nbytes, "ratio": round((rd + wb) / nbytes, 4),
                            "calibration": {k: v["factor"] for k, v in cal.items()}}
            print(f"| {name} | `{short(fe[name][0]['name'])}` | {fk:.1f} | {wk:.1f} | {int(rd + wb)} | {nbytes} | "
                  f"{(rd + wb) / nbytes:.3f} |")
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)

    mf = split(by_dispatch(P("pmc_mfma"), True), loops(P("pmc_mfma.log")))
    lds = split(by_dispatch(P("pmc_lds"), True), loops(P("pmc_lds.log")))
    mfma = {}
    print("\n## MFMA and LDS counters (medians over the timed launches)\n")
    print("| loop | kernel | trace us | SQ_VALU_MFMA_BUSY_CYCLES | SQ_INSTS_VALU_MFMA_MOPS_F8 | GRBM_GUI_ACTIVE / XCD | "
          "MFMA busy (counters) | MFMA busy (trace time) | SQ_INSTS_LDS | SQ_LDS_BANK_CONFLICT | SQ_WAIT_INST_LDS | "
          "SQ_WAIT_ANY | SQ_WAVE_CYCLES |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for name, ds in mf.items():
        key, M, nbytes, sha = spec[name]
        c = {k: st.median(e["c"][k] for e in ds) for k in ds[0]["c"]}
        l2 = {k: st.median(e["c"][k] for e in lds[name]) for k in lds[name][0]["c"]}
        t_us = medians.get(name, {}).get("median_us")
        gui = c["GRBM_GUI_ACTIVE"] / XCDS
        busy_c = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * gui)
        busy_t = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * t_us * 1e3 * CLOCK_GHZ) if t_us else None
        e8m0 = name.endswith("e8m0")
        N = NA + NB if name == "pair64" else NA if name.startswith("gemm_a") else NB
        mfma[name] = {"M": M, "N": N, "e8m0": e8m0, "source_sha": sha, "kernel": short(ds[0]["name"]),
                      "mfma_busy_cycles": c["SQ_VALU_MFMA_BUSY_CYCLES"], "mops_f8": c["SQ_INSTS_VALU_MFMA_MOPS_F8"],
                      "gui_active_cycles_per_xcd": gui, "mfma_busy_frac": round(busy_c, 4),
                      "mfma_busy_frac_trace": round(busy_t, 4) if busy_t else None, "trace_us": t_us,
                      "lds": l2}
        print(f"| {name} | `{short(ds[0]['name'])}` | {t_us} | {c['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} | "
              f"{c['SQ_INSTS_VALU_MFMA_MOPS_F8']:.0f} | {gui:.0f} | {busy_c:.3f} | "
              f"{busy_t if busy_t is None else round(busy_t, 3)} | {l2['SQ_INSTS_LDS']:.0f} | "
              f"{l2['SQ_LDS_BANK_CONFLICT']:.0f} | {l2['SQ_WAIT_INST_LDS']:.0f} | {l2['SQ_WAIT_ANY']:.0f} | "
              f"{l2['SQ_WAVE_CYCLES']:.0f} |")
    with open(os.path.join(PROFILES, "mfma_counters.json"), "w") as f:
        json.dump(mfma, f, indent=1)


if __name__ == "__main__":
    main(sys.argv[1])
