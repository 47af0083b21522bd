"""Summaries of rocprofv3 output for the profiles folder.

Reads the CSV files rocprofv3 writes (`--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` counter
collections, `--pmc` SQ counter collections, `--kernel-trace --stats` kernel statistics and
traces) and prints markdown tables; `decode-json` writes the calibrated per-call HBM bytes of
the decode workload that `bench.py` reports as `roofline.traffic`; `mfma` turns one SQ counter
pass into matrix-core utilisation per kernel.

Calibration: the counter run first copies 64 MiB device to device (`__amd_rocclr_copyBuffer`,
reading and writing exactly 64 MiB); each counter is scaled by 64 MiB / its reading for that
copy. Bytes are per dispatch: the median over the workload's dispatches of each kernel.

    python profile_summary.py counters <pmc dir> <title>
    python profile_summary.py stats <kernel_stats.csv>
    python profile_summary.py trace <kernel_trace.csv> <name substring>
    python profile_summary.py decode-json <pmc dir> <out.json>   (kernel attn_decode_kernel)
    python profile_summary.py mfma <counter_collection.csv> <title>

Matrix-core utilisation (`mfma`): the pass collects SQ_INSTS_VALU_MFMA_F32 (f32 matrix
instructions issued, one per wave instruction), SQ_VALU_MFMA_BUSY_CYCLES (matrix-unit busy
cycles summed over every SIMD), GRBM_GUI_ACTIVE (GPU-busy cycles summed over the 8 XCDs) and
SQ_BUSY_CYCLES. Per dispatch: busy fraction = MFMA busy cycles / (GRBM_GUI_ACTIVE / 8 x 1024
SIMDs), the share of all matrix-unit cycles of the dispatch's lifetime that did work; and the
issued instructions times the flops of one instruction (`--flops-per-inst`) against the
algorithmic flops, which shows padding and masked work.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

COPY_BYTES = 64 << 20
COPY_KERNEL = "__amd_rocclr_copyBuffer"
WINATTN = "winattn::"


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_values(pmc_dir: str, counter: str):
    """(calibration reading in KiB, {kernel name: [KiB per dispatch]}) for one counter pass."""
    files = glob.glob(os.path.join(pmc_dir, counter, "*counter_collection.csv"))
    if not files:
        raise FileNotFoundError(f"no {counter} counter collection under {pmc_dir}")
    per = {}
    calib = None
    for r in _rows(files[0]):
        if r["Counter_Name"] != counter:
            continue
        name, v = r["Kernel_Name"], float(r["Counter_Value"])
        if name == COPY_KERNEL and calib is None:
            calib = v
        elif WINATTN in name:
            per.setdefault(name, []).append(v)
    if calib is None:
        raise ValueError(f"{files[0]}: no calibration copy dispatch")
    return calib, per


def calibrated(pmc_dir: str):
    """{kernel: (dispatches, fetch KiB, read bytes, write KiB, write bytes)} and the factors."""
    fcal, fetch = counter_values(pmc_dir, "FETCH_SIZE")
    wcal, write = counter_values(pmc_dir, "WRITE_SIZE")
    ff = COPY_BYTES / (fcal * 1024.0)
    wf = COPY_BYTES / (wcal * 1024.0)
    out = {}
    for name in fetch:
        fk = statistics.median(fetch[name])
        wk = statistics.median(write.get(name, [0.0]))
        out[name] = (len(fetch[name]), fk, fk * 1024.0 * ff, wk, wk * 1024.0 * wf)
    return out, (fcal, ff), (wcal, wf)


def counters_md(pmc_dir: str, title: str) -> str:
    data, (fcal, ff), (wcal, wf) = calibrated(pmc_dir)
    lines = [f"### {title}", "",
             f"Calibration copy (64 MiB device-to-device, `{COPY_KERNEL}`): FETCH_SIZE "
             f"{fcal:.1f} KiB (factor {ff:.4f}), WRITE_SIZE {wcal:.1f} KiB (factor {wf:.4f}).", "",
             "| kernel | dispatches | FETCH_SIZE KiB (median) | HBM read MB | WRITE_SIZE KiB (median) | HBM write MB |",
             "|---|---|---|---|---|---|"]
    for name, (n, fk, rb, wk, wb) in data.items():
        lines.append(f"| `{name}` | {n} | {fk:.1f} | {rb / 1e6:.3f} | {wk:.1f} | {wb / 1e6:.3f} |")
    return "\n".join(lines) + "\n"


def stats_md(path: str) -> str:
    lines = ["| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in _rows(path):
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |")
    return "\n".join(lines) + "\n"


def trace_durations(path: str, needle: str):
    """Durations (ns) of every dispatch whose kernel name contains `needle`, in launch order."""
    out = []
    for r in _rows(path):
        if needle in r["Kernel_Name"]:
            out.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def decode_json(pmc_dir: str, out_path: str, digest: str,
                kernels=("attn_decode_kernel",)) -> dict:
    """The calibrated bytes of one decode call: the dispatches of every kernel whose name holds
    one of `kernels` (all the call's launches)."""
    data, (_, ff), (_, wf) = calibrated(pmc_dir)
    per = {name: {"read_bytes": int(round(rb)), "write_bytes": int(round(wb))}
           for name, (_, _, rb, _, wb) in data.items()
           if any(k in name for k in kernels)}
    doc = {
        "kernel_source_digest": digest,
        "hbm_bytes_per_launch": sum(v["read_bytes"] + v["write_bytes"] for v in per.values()),
        "launch": "one attn_window_chunk call on the decode workload: " + " + ".join(kernels),
        "per_kernel": per,
        "fetch_factor": ff,
        "write_factor": wf,
        "source": "profiles/hbm_traffic_counters.md",
    }
    with open(out_path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    return doc


XCDS = 8
SIMDS = 1024
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_F32", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
                 "SQ_BUSY_CYCLES")


def mfma_values(path: str):
    """{kernel: {counter: [value per dispatch]}} of the winattn kernels in one SQ pass."""
    per = {}
    for r in _rows(path):
        name = r["Kernel_Name"]
        if WINATTN not in name or r["Counter_Name"] not in MFMA_COUNTERS:
            continue
        per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return per


def mfma_md(path: str, title: str, expected=None) -> str:
    """Markdown table of matrix-core use per kernel. `expected` maps a kernel-name substring to
    (flops of one matrix instruction, algorithmic flops per dispatch)."""
    lines = [f"### {title}", "",
             "| kernel | dispatches | MFMA instructions | MFMA busy cycles | GPU-busy cycles per XCD "
             "| busy fraction | issued flops / algorithmic |",
             "|---|---|---|---|---|---|---|"]
    for name, c in mfma_values(path).items():
        med = {k: statistics.median(v) for k, v in c.items()}
        n = len(c.get("SQ_INSTS_VALU_MFMA_F32", []))
        inst = med.get("SQ_INSTS_VALU_MFMA_F32", 0.0)
        busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        gui = med.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        frac = busy / (gui * SIMDS) if gui > 0 else 0.0
        ratio = "—"
        for needle, (fpi, alg) in (expected or {}).items():
            if needle in name and alg > 0:
                ratio = f"{inst * fpi / alg:.3f}"
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {n} | {inst:.0f} | {busy:.0f} | {gui:.0f} | {frac:.3f} | {ratio} |")
    return "\n".join(lines) + "\n"


def main(argv):
    if len(argv) < 2:
        print(__doc__)
        return 2
    cmd = argv[1]
    if cmd == "counters":
        print(counters_md(argv[2], argv[3]))
    elif cmd == "stats":
        print(stats_md(argv[2]))
    elif cmd == "trace":
        d = trace_durations(argv[2], argv[3])
        print(f"{len(d)} dispatches, mean {statistics.mean(d):.0f} ns, median "
              f"{statistics.median(d):.0f} ns")
    elif cmd == "decode-json":
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        from sliding_window_gqa_group_amd.build import DECODE_SOURCES, source_digest
        print(json.dumps(decode_json(argv[2], argv[3], source_digest(DECODE_SOURCES)), indent=1))
    elif cmd == "mfma":
        ap = argparse.ArgumentParser(prog="profile_summary.py mfma")
        ap.add_argument("csv")
        ap.add_argument("title")
        ap.add_argument("--expect", nargs=3, action="append", default=[],
                        metavar=("KERNEL_SUBSTRING", "FLOPS_PER_INST", "ALG_FLOPS"))
        a = ap.parse_args(argv[2:])
        exp = {k: (float(f), float(g)) for k, f, g in a.expect}
        print(mfma_md(a.csv, a.title, exp))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
