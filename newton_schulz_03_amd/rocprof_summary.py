"""Summaries of rocprofv3 output for the Muon kernels, as short markdown.

Usage:
    python -m newton_schulz_03_amd.rocprof_summary trace DIR --command "..." [--muon-only]
        DIR holds the CSV output of `rocprofv3 --kernel-trace --stats`:
        a per-kernel table of calls and durations (with --muon-only, of this
        library's kernels alone).
    python -m newton_schulz_03_amd.rocprof_summary mfma DIR --workload NAME --command "..."
        DIR holds the CSV output of `rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16`:
        the matrix cores' busy fraction and issued bf16 flops per kernel.
    python -m newton_schulz_03_amd.rocprof_summary clock DIR --workload NAME --command "..."
        DIR holds the CSV output of `rocprofv3 --pmc GRBM_GUI_ACTIVE GRBM_COUNT
        SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY`: per kernel,
        the clock held during the dispatch, the matrix cores' busy share of its
        cycles, and the share of wave time spent waiting.
    python -m newton_schulz_03_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR
            --copy-bytes N --workload NAME --command "..."
        FETCH_DIR and WRITE_DIR hold the CSV output of two runs, one with
        `--pmc FETCH_SIZE` and one with `--pmc WRITE_SIZE`.  In both runs the
        program also ran one plain device copy of N bytes (read N, write N;
        a float32 multiply by 2 into another buffer, torch's MulFunctor kernel).
        Its counter readings give the scale from counter units to bytes.  Prints the
        per-dispatch HBM traffic of every Muon kernel and a machine-readable
        block for the product kernel, which the benchmark reads back as long
        as the kernel sources are unchanged (same digest).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))

# Sources that set the matrix-core kernels' memory traffic: their device code,
# and the host code that cuts each launch's tiles into per-XCD ranges (which
# tiles share an L2).
KERNEL_SOURCES = ("csrc/gemm_bf16.hip", "csrc/gemm_pipeline.hpp", "csrc/gemm_common.hpp",
                  "csrc/device_common.hpp", "csrc/muon_internal.hpp", "csrc/muon_abi.hip")

# The wide-tile products (256 x 384 tiles) take the labels of the products they
# replace: a call uses one kind or the other for all of its middle products.
SHORT_NAMES = (("k_gemm_bf16<0,false,false,false>", "gram"), ("k_gemm_bf16<1,false,false,false>", "poly"),
               ("k_gemm_bf16<2,false,false,false>", "prod"),
               ("k_gemm_bf16<2,false,false,true>", "prod_first"),
               ("k_gemm_bf16_wide<false>", "prod"), ("k_gemm_bf16_wide<true>", "prod_first"),
               ("k_gemm_bf16<2,true,false,false>", "prod_finish"),
               ("k_gemm_bf16<2,true,false,true>", "prod_finish_first"),
               ("k_gemm_bf16<0,false,true,false>", "gram_budget"),
               ("k_gemm_bf16<1,false,true,false>", "poly_budget"),
               ("k_gemm_bf16<2,false,true,false>", "prod_budget"),
               ("k_gemm_bf16<2,false,true,true>", "prod_first_budget"),
               ("k_gemm_bf16<2,true,true,false>", "prod_finish_budget"),
               ("k_gemm_bf16<2,true,true,true>", "prod_finish_first_budget"),
               ("k_gemm_staged", "gemm_fp32"), ("k_prepare", "prepare"), ("k_finish", "finish"),
               ("k_finalize", "norm"), ("k_adamw", "adamw"))


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(_PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def short_name(kernel: str) -> str:
    k = kernel.replace("(int)", "").replace(" ", "")
    for key, name in SHORT_NAMES:
        if key.replace(" ", "") in k:
            return name
    if "MulFunctor" in kernel:
        return "copy"
    if "FillFunctor" in kernel:
        return "fill"
    return kernel[:48]


def _one_csv(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def trace_table(d: str):
    rows = list(csv.DictReader(open(_one_csv(d, "kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append((short_name(r["Name"]), r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e6,
                    float(r["TotalDurationNs"]) / 1e6, float(r.get("Percentage", 0.0))))
    out.sort(key=lambda x: -x[4])
    return out


def counter_per_dispatch(d: str, counter: str):
    """kernel short name -> (dispatches, mean counter value per dispatch)."""
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(_one_csv(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        k = short_name(r["Kernel_Name"])
        tot[k] += float(r["Counter_Value"])
        disp[k].add(r.get("Dispatch_Id") or r.get("Correlation_Id"))
    return {k: (len(disp[k]), tot[k] / max(1, len(disp[k]))) for k in tot}


MUON_KERNELS = {name for _, name in SHORT_NAMES}


def cmd_trace(a):
    rows = trace_table(a.dir)
    if a.muon_only:
        rows = [r for r in rows if r[0] in MUON_KERNELS]
        tot = sum(r[4] for r in rows) or 1.0
        rows = [r[:5] + (100.0 * r[4] / tot,) for r in rows]
    print(f"# Kernel trace: {a.title}\n")
    print(f"Command (from the repository root):\n\n```\n{a.command}\n```\n")
    if a.muon_only:
        print("Only this library's kernels are listed (the program's other kernels, such as input "
              "generation, are left out); the last column is the share of their time.\n")
    share = "% of listed time" if a.muon_only else "% of GPU time"
    print(f"| kernel | calls | avg ms | total ms | {share} |")
    print("|---|---|---|---|---|")
    for short, _, calls, avg, total, pct in rows:
        print(f"| {short} | {calls} | {avg:.4f} | {total:.2f} | {pct:.1f} |")
    print("\nFull kernel names:\n")
    for short, name, *_ in rows:
        print(f"- {short}: `{name[:160]}`")


def counter_means(d: str):
    """kernel short name -> {counter: mean value per dispatch}, dispatches."""
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in csv.DictReader(open(_one_csv(d, "counter_collection.csv"))):
        k = short_name(r["Kernel_Name"])
        tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r.get("Dispatch_Id") or r.get("Correlation_Id"))
    return {k: ({c: v / max(1, len(disp[k])) for c, v in tot[k].items()}, len(disp[k])) for k in tot}


def cmd_mfma(a):
    means = counter_means(a.dir)
    print(f"# Matrix-core utilisation: {a.workload}\n")
    print(f"Command (from the repository root):\n\n```\n{a.command}\n```\n")
    print("MfmaUtil is rocprofv3's derived metric: the cycles the matrix cores were busy, "
          "summed over all SIMDs, over the kernel's active cycles times the SIMD count.  It is "
          "taken at whatever clock the chip ran, so it is the fraction of the matrix-core peak "
          "at the sustained clock.  bf16 MFMA flops count every MFMA the kernel issued "
          "(SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), the redundant lower-triangle blocks of "
          "diagonal tiles and the identity-fragment terms included.\n")
    print("| kernel | dispatches | MfmaUtil % | bf16 MFMA flops per dispatch |")
    print("|---|---|---|---|")
    rows = sorted(means.items(), key=lambda kv: -kv[1][0].get("MfmaUtil", 0.0))
    for k, (c, n) in rows:
        if k not in MUON_KERNELS:
            continue
        util = c.get("MfmaUtil")
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        print(f"| {k} | {n} | {'' if util is None else f'{util:.1f}'} | "
              f"{'' if mops is None else f'{mops * 512:.4g}'} |")


def cmd_traffic(a):
    fetch = counter_per_dispatch(a.fetch_dir, "FETCH_SIZE")
    write = counter_per_dispatch(a.write_dir, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("the calibration copy kernel is missing from the counter output")
    ff = a.copy_bytes / (fetch["copy"][1] * 1024.0)
    wf = a.copy_bytes / (write["copy"][1] * 1024.0)
    print(f"# HBM traffic per dispatch: {a.workload}\n")
    print("Commands (from the repository root, each a run of its own):\n")
    print(f"```\n{a.command}\n```\n")
    print(f"Calibration: one device copy of {a.copy_bytes} bytes reads "
          f"{fetch['copy'][1]:.0f} KiB by FETCH_SIZE and writes {write['copy'][1]:.0f} KiB by "
          f"WRITE_SIZE; scale factors {ff:.4f} (fetch) and {wf:.4f} (write).\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes (scaled) |")
    print("|---|---|---|---|---|")
    traffic = {}
    for k in sorted(set(fetch) & set(write)):
        b = fetch[k][1] * 1024.0 * ff + write[k][1] * 1024.0 * wf
        traffic[k] = b
        print(f"| {k} | {fetch[k][0]} | {fetch[k][1]:.0f} | {write[k][1]:.0f} | {b:.4g} |")
    if "prod" in traffic:
        print("\nProduct kernel, read back by the benchmark:\n")
        print("```")
        print("kernel: prod")
        print(f"workload: {a.workload}")
        print(f"source_sha256: {kernel_source_digest()}")
        print(f"fetch_kib_per_dispatch: {fetch['prod'][1]:.1f}")
        print(f"write_kib_per_dispatch: {write['prod'][1]:.1f}")
        print(f"fetch_factor: {ff:.6f}")
        print(f"write_factor: {wf:.6f}")
        print(f"traffic_bytes_per_launch: {traffic['prod']:.0f}")
        print("```")


# XCDs whose GRBM counts rocprofv3 sums per dispatch, and SIMDs of the chip.
N_XCD = 8
N_SIMD = 256 * 4


def cmd_clock(a):
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(dict)
    for r in csv.DictReader(open(_one_csv(a.dir, "counter_collection.csv"))):
        k = short_name(r["Kernel_Name"])
        d = r.get("Dispatch_Id") or r.get("Correlation_Id")
        sums[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k][d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    print(f"# Clock and matrix-core busy share: {a.workload}\n")
    print(f"Command (from the repository root):\n\n```\n{a.command}\n```\n")
    print(f"Clock: GRBM_GUI_ACTIVE (GPU cycles, summed over the {N_XCD} XCDs) over the dispatch's "
          f"duration.  Busy: SQ_VALU_MFMA_BUSY_CYCLES over those cycles x {N_SIMD} SIMDs.  "
          "Waiting: SQ_WAIT_ANY over SQ_WAVE_CYCLES (waves stopped at s_waitcnt or a barrier); "
          "issue-blocked: SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES.  Under counter collection the "
          "dispatches run one at a time.\n")
    print("| kernel | dispatches | avg ms | clock GHz | matrix cores busy | waves waiting | issue-blocked |")
    print("|---|---|---|---|---|---|---|")
    rows = []
    for k, c in sums.items():
        if k not in MUON_KERNELS or "GRBM_GUI_ACTIVE" not in c:
            continue
        n = len(disp[k])
        dur = sum(disp[k].values()) / n
        if dur < 1e-4:  # too short for its timestamps to give a clock
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / n / N_XCD
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n / (cyc * N_SIMD)
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        wait = c.get("SQ_WAIT_ANY", 0.0) / wc if wc else 0.0
        blk = c.get("SQ_WAIT_INST_ANY", 0.0) / wc if wc else 0.0
        rows.append((dur * n, f"| {k} | {n} | {dur * 1e3:.3f} | {cyc / dur / 1e9:.2f} | "
                              f"{100 * busy:.1f}% | {100 * wait:.1f}% | {100 * blk:.1f}% |"))
    for _, line in sorted(rows, reverse=True):
        print(line)


def read_traffic(path: str, workload: str):
    """traffic_bytes_per_launch from a summary written by `traffic`, or None when the
    summary is missing, names another workload, or predates the current kernel sources."""
    try:
        text = open(path).read()
    except OSError:
        return None
    kv = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith(("#", "|", "-")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("workload") != workload or kv.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", default="")
    t.add_argument("--command", required=True)
    t.add_argument("--muon-only", action="store_true",
                   help="list this library's kernels only (drops input generation and the like)")
    f = sub.add_parser("traffic")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--command", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("dir")
    m.add_argument("--workload", required=True)
    m.add_argument("--command", required=True)
    k = sub.add_parser("clock")
    k.add_argument("dir")
    k.add_argument("--workload", required=True)
    k.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "mfma": cmd_mfma, "clock": cmd_clock}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
