"""Profile summaries for libmoe kernels: rocprofv3 output -> short markdown
files, and the HBM traffic figure that bench.py reports beside a kernel's
roofline.

HBM traffic comes from two counter runs (FETCH_SIZE, then WRITE_SIZE; both in
KiB per dispatch, read at the L2's fabric interface) of the benchmark, each
scaled by what the same counter reads for a plain device copy of known size.
The figure is tied to a digest of the kernel's source files: once the source
changes, the stored counters no longer describe the kernel and bench.py
reports no traffic for it.

    python -m sparse_moe_layer_gemv_amd.profiling copy          # the calibration copy (run under rocprofv3 --pmc)
    python -m sparse_moe_layer_gemv_amd.profiling traffic ...   # counters -> profiles/hbm_traffic_*.md
    python -m sparse_moe_layer_gemv_amd.profiling stats ...     # --stats csv -> markdown table
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")

# Source files that define each profiled kernel (kernel body, launcher and the
# device helpers it inlines).
KERNEL_SOURCES = {
    "grouped_up": ["csrc/moe_gemm.hip", "csrc/moe_device.hpp", "csrc/moe_internal.hpp"],
    "grouped_down": ["csrc/moe_gemm.hip", "csrc/moe_device.hpp", "csrc/moe_internal.hpp"],
    "decode_up": ["csrc/moe_decode.hip", "csrc/moe_device.hpp", "csrc/moe_internal.hpp"],
    "decode_down": ["csrc/moe_decode.hip", "csrc/moe_device.hpp", "csrc/moe_internal.hpp"],
    "router_fused": ["csrc/moe_router.hip", "csrc/moe_device.hpp", "csrc/moe_internal.hpp"],
}

COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read, 1 GiB written


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_{kernel}_{workload}.md")


def load_traffic(kernel: str, workload: str):
    """Stored per-launch HBM bytes of `kernel` on `workload`, or None when there
    is no record or the kernel's sources changed since it was taken."""
    p = traffic_path(kernel, workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_digest") != source_digest(kernel):
        return None
    return rec


# ---------------------------------------------------------------------------
# rocprofv3 csv readers
# ---------------------------------------------------------------------------
def _counter_csv(d: str) -> str:
    fs = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not fs:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    return fs[0]


def read_counter(d: str, counter: str, name_regex: str):
    """Per-dispatch values (KiB) of `counter` for kernels matching name_regex,
    in dispatch order, with the dispatch durations in microseconds."""
    rows = []
    with open(_counter_csv(d)) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not re.search(name_regex, r["Kernel_Name"]):
                continue
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"]), dur, r["Kernel_Name"]))
    rows.sort()
    return rows


def copy_factor(d: str, counter: str) -> float:
    """Bytes moved by the calibration copy / what `counter` reports for it."""
    rows = read_counter(d, counter, r"copyBuffer|copy_kernel|elementwise_kernel.*copy")
    big = [v for _, v, _, _ in rows if v * 1024 > COPY_BYTES / 4]
    if not big:
        raise RuntimeError(f"calibration copy not found in {d}")
    return COPY_BYTES / (statistics.median(big) * 1024)


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("moe::", "").replace("void ", "")
    return name.split("(")[0]


# ---------------------------------------------------------------------------
# commands
# ---------------------------------------------------------------------------
def cmd_copy(_args) -> int:
    import torch
    a = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes 3 times", flush=True)
    return 0


def cmd_traffic(a) -> int:
    ff = copy_factor(a.cal_fetch, "FETCH_SIZE")
    fw = copy_factor(a.cal_write, "WRITE_SIZE")
    fr = read_counter(a.fetch, "FETCH_SIZE", a.regex)
    wr = read_counter(a.write, "WRITE_SIZE", a.regex)
    if not fr or not wr:
        raise RuntimeError("no dispatch of the kernel in the counter runs")
    # steady state: drop the first dispatch (cold caches), take the median
    fv = statistics.median([v for _, v, _, _ in (fr[1:] or fr)])
    wv = statistics.median([v for _, v, _, _ in (wr[1:] or wr)])
    fetch_b = fv * 1024 * ff
    write_b = wv * 1024 * fw
    rec = {"kernel": a.kernel, "workload": a.workload, "source_digest": source_digest(a.kernel),
           "fetch_kib_raw": fv, "write_kib_raw": wv, "fetch_scale": ff, "write_scale": fw,
           "read_bytes": fetch_b, "write_bytes": write_b, "bytes_per_launch": fetch_b + write_b,
           "dispatches": len(fr)}
    lines = [
        f"# HBM traffic, `{a.kernel}` on the {a.workload} workload",
        "",
        "Commands (on the MI355X box, from the repository root; $REPO is the repository path):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
    ]
    lines += a.command
    lines += [
        "```",
        "",
        "Counter scale (bytes moved by a 1 GiB device copy / bytes the counter reports for it):",
        f"FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {fw:.3f}.",
        "",
        "| dispatch | kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | duration (us) |",
        "|---|---|---|---|---|",
    ]
    for (i, f_kib, dur, name), (_, w_kib, _, _) in zip(fr, wr):
        lines.append(f"| {i} | `{_short(name)}` | {f_kib:.1f} | {w_kib:.1f} | {dur:.1f} |")
    lines += [
        "",
        f"Per launch (median of the dispatches after the first): read {fetch_b / 1e9:.3f} GB, "
        f"written {write_b / 1e9:.3f} GB.",
        "",
        "```json",
        json.dumps(rec, indent=1),
        "```",
        "",
    ]
    out = traffic_path(a.kernel, a.workload)
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


# bf16 dense matrix-core rate of one compute unit per clock (MI355X: 2.5 PF/s
# published = 256 CUs x 4096 FLOP/clk x 2.4 GHz)
BF16_FLOP_PER_CU_CLK = 4096
N_CU = 256
SIMD_PER_CU = 4


def read_counters(d: str, name_regex: str):
    """{dispatch: {"kernel", "dur_us", counter: value}} for kernels matching name_regex."""
    out = {}
    with open(_counter_csv(d)) as f:
        for r in csv.DictReader(f):
            if not re.search(name_regex, r["Kernel_Name"]):
                continue
            i = int(r["Dispatch_Id"])
            rec = out.setdefault(i, {"kernel": _short(r["Kernel_Name"]),
                                     "dur_us": (int(r["End_Timestamp"]) -
                                                int(r["Start_Timestamp"])) / 1e3})
            rec[r["Counter_Name"]] = rec.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return dict(sorted(out.items()))


def cmd_mfma(a) -> int:
    """Matrix-core evidence of one kernel from a --pmc run of SQ_INSTS_VALU_MFMA_MOPS_BF16
    (bf16 MFMA work in units of 512 FLOP), SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and
    GRBM_GUI_ACTIVE: FLOPs issued (padding rows included) against the algorithmic
    count, the achieved rate, the clock GRBM_GUI_ACTIVE / duration implies, and the
    fraction of the matrix-core peak at that clock."""
    rows = read_counters(a.dir, a.regex)
    if not rows:
        raise RuntimeError("no dispatch of the kernel in the counter run")
    keys = [k for k in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
                        "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE") if k in next(iter(rows.values()))]
    lines = [f"# Matrix-core counters, `{a.kernel}` on the {a.workload} workload", "",
             "Command (on the MI355X box, from the repository root; $REPO is the repository path):",
             "", "```", "cd /tmp && export TMPDIR=/tmp"] + a.command + ["```", "",
             "| dispatch | kernel | duration (us) | " + " | ".join(keys) + " |",
             "|---|---|---|" + "---|" * len(keys)]
    for i, r in rows.items():
        lines.append(f"| {i} | `{r['kernel']}` | {r['dur_us']:.1f} | " +
                     " | ".join(f"{r.get(k, 0):.0f}" for k in keys) + " |")
    steady = list(rows.values())[1:] or list(rows.values())
    med = {k: statistics.median([r.get(k, 0.0) for r in steady]) for k in keys + ["dur_us"]}
    dur = med["dur_us"] * 1e-6
    summary = {"kernel": a.kernel, "workload": a.workload, "dispatches": len(rows),
               "duration_us": med["dur_us"], "algorithmic_flop": a.algorithmic_flop,
               "raw_median": {k: med[k] for k in keys}, "grbm_scale": a.grbm_scale}
    lines += ["", "Medians over the dispatches after the first:", ""]
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        flop = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        summary.update(issued_flop=flop, issued_tflops=flop / dur / 1e12,
                       issued_over_algorithmic=flop / a.algorithmic_flop if a.algorithmic_flop else None)
        lines.append(f"- bf16 matrix-core work issued: {flop / 1e12:.4f} TFLOP "
                     f"({flop / a.algorithmic_flop:.4f} x the algorithmic {a.algorithmic_flop / 1e12:.4f}"
                     " TFLOP; the excess is padding rows)" if a.algorithmic_flop else "")
        lines.append(f"- issued rate: {flop / dur / 1e12:.1f} TFLOP/s; algorithmic rate "
                     f"{a.algorithmic_flop / dur / 1e12:.1f} TFLOP/s "
                     f"({a.algorithmic_flop / dur / 1e12 / 2500:.3f} of the published 2.5 PF/s)")
    if "GRBM_GUI_ACTIVE" in med:
        cycles = med["GRBM_GUI_ACTIVE"] / a.grbm_scale
        clk = cycles / dur
        summary.update(gpu_cycles=cycles, clock_ghz=clk / 1e9)
        lines.append(f"- GRBM_GUI_ACTIVE / {a.grbm_scale:g} = {cycles:.0f} cycles over "
                     f"{med['dur_us']:.1f} us: {clk / 1e9:.3f} GHz")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
            peak_at_clk = N_CU * BF16_FLOP_PER_CU_CLK * cycles
            summary["issued_over_peak_at_clock"] = flop / peak_at_clk
            lines.append(f"- issued work over the matrix-core peak at that clock "
                         f"({N_CU} CUs x {BF16_FLOP_PER_CU_CLK} FLOP/clk x {cycles:.0f} cycles): "
                         f"{flop / peak_at_clk:.3f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            # the busy count is summed over the SIMDs (4 per CU), each of
            # which owns a matrix core
            busy = med["SQ_VALU_MFMA_BUSY_CYCLES"]
            simds = N_CU * SIMD_PER_CU
            summary["mfma_busy_over_simd_cycles"] = busy / (cycles * simds)
            lines.append(f"- SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {simds} SIMDs): "
                         f"{busy / (cycles * simds):.3f} of the matrix cores' cycles busy")
    lines += ["", "```json", json.dumps(summary, indent=1), "```", ""]
    out = os.path.join(PROFILES, f"mfma_{a.kernel}_{a.workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(l for l in lines if l is not None) + "\n")
    print("\n".join(lines))
    return 0


def cmd_counters(a) -> int:
    """Any --pmc pass: per-dispatch values and medians of every counter for one
    kernel, into profiles/<name>.md."""
    rows = read_counters(a.dir, a.regex)
    if not rows:
        raise RuntimeError("no dispatch of the kernel in the counter run")
    keys = [k for k in next(iter(rows.values())) if k not in ("kernel", "dur_us")]
    lines = [f"# {a.title}", "",
             "Command (on the MI355X box, from the repository root; $REPO is the repository path):",
             "", "```", "cd /tmp && export TMPDIR=/tmp"] + a.command + ["```", "",
             "| dispatch | kernel | duration (us) | " + " | ".join(keys) + " |",
             "|---|---|---|" + "---|" * len(keys)]
    for i, r in rows.items():
        lines.append(f"| {i} | `{r['kernel']}` | {r['dur_us']:.1f} | " +
                     " | ".join(f"{r.get(k, 0):.0f}" for k in keys) + " |")
    steady = list(rows.values())[1:] or list(rows.values())
    med = {k: statistics.median([r.get(k, 0.0) for r in steady]) for k in keys + ["dur_us"]}
    lines += ["", "Medians over the dispatches after the first:", "", "```json",
              json.dumps(med, indent=1), "```", ""] + a.note + [""]
    out = os.path.join(PROFILES, f"{a.name}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def cmd_stats(a) -> int:
    with open(a.csv) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# {a.title}", "",
             "Command (on the MI355X box, from the repository root; $REPO is the repository path):", "",
             "```", "cd /tmp && export TMPDIR=/tmp"] + a.command + ["```", "",
             f"`rocprofv3 --stats` kernel summary (`{os.path.basename(a.csv)}`):", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="libmoe profile summaries")
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("copy", help="run the 1 GiB calibration copy on cuda:0")
    t = sub.add_parser("traffic", help="write profiles/hbm_traffic_<kernel>_<workload>.md")
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--workload", required=True)
    t.add_argument("--regex", required=True, help="kernel-name regex for the dispatches")
    t.add_argument("--fetch", required=True, help="rocprofv3 -d folder of the FETCH_SIZE run")
    t.add_argument("--write", required=True, help="rocprofv3 -d folder of the WRITE_SIZE run")
    t.add_argument("--cal-fetch", required=True, help="FETCH_SIZE run of the calibration copy")
    t.add_argument("--cal-write", required=True, help="WRITE_SIZE run of the calibration copy")
    t.add_argument("--command", action="append", default=[], help="command line to record")
    m = sub.add_parser("mfma", help="matrix-core counters -> profiles/mfma_<kernel>_<workload>.md")
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--regex", required=True)
    m.add_argument("--dir", required=True, help="rocprofv3 -d folder of the counter run")
    m.add_argument("--algorithmic-flop", type=float, default=0.0)
    m.add_argument("--grbm-scale", type=float, default=1.0,
                   help="divide GRBM_GUI_ACTIVE by this (instances summed into the counter)")
    m.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters", help="any --pmc pass of one kernel -> profiles/<name>.md")
    c.add_argument("--name", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--regex", required=True)
    c.add_argument("--dir", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--note", action="append", default=[], help="line of interpretation to append")
    s = sub.add_parser("stats", help="rocprofv3 --stats csv -> markdown")
    s.add_argument("--csv", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    return {"copy": cmd_copy, "traffic": cmd_traffic, "mfma": cmd_mfma, "counters": cmd_counters,
            "stats": cmd_stats}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
