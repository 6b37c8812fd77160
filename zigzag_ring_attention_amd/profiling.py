"""Summaries of rocprofv3 output for the committed profiles.

    python -m zigzag_ring_attention_amd.profiling stats  <kernel_stats.csv> <command...>
    python -m zigzag_ring_attention_amd.profiling traffic <fetch.csv> <write.csv> [--workload=cN] <command...>
    python -m zigzag_ring_attention_amd.profiling util <counter_collection.csv> <command...>

``stats`` turns a ``--kernel-trace --stats`` kernel_stats.csv into a markdown
table.  ``traffic`` turns two ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
counter_collection.csv files into HBM bytes per launch of each libzz kernel.
``util`` reports the MFMA utilisation and the effective clock of the three
attention kernels from one counter pass.
The counters are calibrated against the zigzag permute kernel in the same
run, a plain row copy whose bytes are known exactly: the first permute of a
bench step moves T * Hq * d * 2 bytes each way.

The traffic summary records a hash of the kernel sources; ``read_traffic``
returns nothing for a kernel once the sources have changed since the
counters were taken.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["zz_fwd.hip", "zz_bwd.hip", "zz_bwd_dq.hip", "zz_bwd.h", "zz_mfma.h", "zz_device.h",
                  "zz_util.hip", "zz_internal.h", "../build.py"]
_NAMES = ["fwd_step_kernel", "bwd_dkv_kernel", "bwd_dq_kernel", "permute_kernel", "cast_rows_kernel",
          "bwd_pre_kernel", "lse_merge_kernel", "debug_mask_kernel"]


def sources_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    for n in _NAMES:
        if n in name:
            return n
    return name[:48]


def stats_markdown(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# Kernel time, rocprofv3 --kernel-trace --stats", "",
           "Command: `%s`" % command, "",
           "| kernel | calls | total ms | average ms | min ms | max ms | % |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %s | %.3f | %.4f | %.4f | %.4f | %.2f |" % (
            short_name(r["Name"]), r["Calls"], float(r["TotalDurationNs"]) / 1e6,
            float(r["AverageNs"]) / 1e6, float(r["MinNs"]) / 1e6, float(r["MaxNs"]) / 1e6,
            float(r["Percentage"])))
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, counter: str):
    vals = collections.defaultdict(list)
    grid = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short_name(r["Kernel_Name"])
        vals[k].append(float(r["Counter_Value"]))
        grid.setdefault(k, []).append(int(r["Grid_Size"]))
    return vals, grid


def traffic_text(fetch_csv: str, write_csv: str, command: str, copy_bytes: float) -> str:
    f, _ = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w, _ = _per_dispatch(write_csv, "WRITE_SIZE")
    # calibration: the first permute of the step copies copy_bytes each way
    f_cal = copy_bytes / (f["permute_kernel"][0] * 1024.0)
    w_cal = copy_bytes / (w["permute_kernel"][0] * 1024.0)
    lines = ["# HBM traffic per launch, rocprofv3 --pmc FETCH_SIZE then --pmc WRITE_SIZE (KiB per dispatch)",
             "# command: %s" % command,
             "# calibration: first permute_kernel dispatch copies %d bytes each way;" % int(copy_bytes),
             "#   bytes = FETCH_SIZE KiB * 1024 * %.4f, WRITE_SIZE KiB * 1024 * %.4f" % (f_cal, w_cal),
             "kernel_sources_sha256 %s" % sources_hash(),
             "fetch_calibration %.6f" % f_cal,
             "write_calibration %.6f" % w_cal]
    for k in sorted(set(f) & set(w)):
        fk = sum(f[k]) / len(f[k])
        wk = sum(w[k]) / len(w[k])
        lines.append("kernel %s dispatches %d fetch_kib %.1f write_kib %.1f hbm_bytes_per_launch %.6e"
                     % (k, len(f[k]), fk, wk, fk * 1024 * f_cal + wk * 1024 * w_cal))
    return "\n".join(lines) + "\n"


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU; dense MFMA FLOPs per clock per SIMD.
XCDS, SIMDS = 8, 256 * 4
MFMA_FLOP = {"bf16": 32 * 32 * 16 * 2, "f32": 32 * 32 * 2 * 2}   # per 32x32xK instruction
FLOP_PER_CLK_SIMD = {"bf16": 1024, "f32": 64}
NOMINAL_GHZ = 2.4


def util_markdown(path: str, command: str) -> str:
    """MFMA utilisation and effective clock per libzz kernel from one
    `--pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` pass.

    SQ_INSTS_MFMA counts wave instructions (x FLOP per instruction = the
    executed matrix work); SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of
    every SIMD's matrix unit; GRBM_GUI_ACTIVE sums the active cycles of the 8
    XCDs, so GRBM_GUI_ACTIVE / 8 over the dispatch time is the clock."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = collections.defaultdict(dict)
    dtype = {}
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        if k not in ("fwd_step_kernel", "bwd_dkv_kernel", "bwd_dq_kernel"):
            continue
        d = r["Dispatch_Id"]
        per[k][(d, r["Counter_Name"])] += float(r["Counter_Value"])
        dur[k][d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        dtype[k] = "bf16" if "DF16b" in r["Kernel_Name"] else "f32"
    out = ["# MFMA utilisation and clock, rocprofv3 --pmc", "",
           "Command: `%s`" % command, "",
           "kernel_sources_sha256 %s" % sources_hash(), "",
           "Per dispatch (mean): executed matrix work = SQ_INSTS_MFMA x FLOP per instruction; "
           "busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x %d SIMDs); clock = GRBM_GUI_ACTIVE / %d XCDs / time. "
           "The clock-adjusted peak is %d FLOP/clk/SIMD x %d SIMDs x clock (2.5166 PFLOP/s at %.1f GHz)."
           % (SIMDS, XCDS, FLOP_PER_CLK_SIMD["bf16"], SIMDS, NOMINAL_GHZ), "",
           "| kernel | dispatches | ms | executed TFLOP | TFLOP/s | clock GHz | MFMA busy | of nominal peak |",
           "|---|---|---|---|---|---|---|---|"]
    for k in ("fwd_step_kernel", "bwd_dkv_kernel", "bwd_dq_kernel"):
        if k not in dur:
            continue
        ds = sorted(dur[k])
        t = sum(dur[k][d] for d in ds) / len(ds)
        inst = sum(per[k][(d, "SQ_INSTS_MFMA")] for d in ds) / len(ds)
        busy = sum(per[k][(d, "SQ_VALU_MFMA_BUSY_CYCLES")] for d in ds) / len(ds)
        gui = sum(per[k][(d, "GRBM_GUI_ACTIVE")] for d in ds) / len(ds)
        cyc = gui / XCDS
        flop = inst * MFMA_FLOP[dtype[k]]
        nominal = FLOP_PER_CLK_SIMD[dtype[k]] * SIMDS * NOMINAL_GHZ * 1e9
        out.append("| %s | %d | %.3f | %.3f | %.1f | %.3f | %.3f | %.3f |" % (
            k, len(ds), t * 1e3, flop / 1e12, flop / t / 1e12, cyc / t / 1e9, busy / (cyc * SIMDS),
            flop / t / nominal))
    return "\n".join(out) + "\n"


ISSUE_COUNTERS = (
    ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_WAVES",
     "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"),
    ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
     "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_INSTS_VALU_TRANS_F32", "GRBM_GUI_ACTIVE"),
)


def issue_markdown(paths, command: str) -> str:
    """Instruction mix and issue/wait cycles per libzz kernel from the two
    `--pmc` passes of ISSUE_COUNTERS (one CSV each).  SQ_INSTS_VALU includes
    the MFMA instructions; the SQ_*_CYCLES and SQ_ACTIVE_/SQ_WAIT_ counters
    are summed over waves in units of 4 clocks."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    nd = collections.defaultdict(set)
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"])
            if k not in ("fwd_step_kernel", "bwd_dkv_kernel", "bwd_dq_kernel"):
                continue
            per[k][r["Counter_Name"]] += float(r["Counter_Value"])
            nd[(k, path)].add(r["Dispatch_Id"])
    out = ["# Instruction mix and issue cycles, rocprofv3 --pmc (two passes)", "",
           "Command: `%s`" % command, "",
           "kernel_sources_sha256 %s" % sources_hash(), "",
           "Per MFMA instruction: vector (non-MFMA), transcendental, LDS, scalar and vector-memory instructions. "
           "Co-exec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (share of matrix-busy cycles with a "
           "vector instruction in flight beside it); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/%d x %d "
           "SIMDs); wait any / LDS wait = share of wave-cycles waiting on anything / on LDS results." % (XCDS, SIMDS), "",
           "| kernel | VALU/MFMA | trans/MFMA | LDS/MFMA | SALU/MFMA | VMEM/MFMA | MFMA busy | co-exec | wait any | LDS wait |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for k in ("fwd_step_kernel", "bwd_dkv_kernel", "bwd_dq_kernel"):
        if k not in per:
            continue
        c = per[k]
        mf = c["SQ_INSTS_MFMA"]
        if mf <= 0:
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        out.append("| %s | %.2f | %.2f | %.2f | %.2f | %.3f | %.3f | %.3f | %.3f | %.3f |" % (
            k, (c["SQ_INSTS_VALU"] - mf) / mf, c["SQ_INSTS_VALU_TRANS_F32"] / mf, c["SQ_INSTS_LDS"] / mf,
            c["SQ_INSTS_SALU"] / mf, c["SQ_INSTS_VMEM_RD"] / mf,
            c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS) if cyc else float("nan"),
            c["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(1.0, c["SQ_VALU_MFMA_BUSY_CYCLES"]),
            c["SQ_WAIT_ANY"] / max(1.0, c["SQ_WAVE_CYCLES"]),
            c["SQ_WAIT_INST_LDS"] / max(1.0, c["SQ_WAVE_CYCLES"])))
    return "\n".join(out) + "\n"


def read_util(path: str):
    """{kernel: (clock GHz, MFMA busy fraction)} from a utilisation summary,
    or None if the file is missing or the kernel sources changed since it was
    taken."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_sources_sha256 (\S+)", text, re.M)
    if not m or m.group(1) != sources_hash():
        return None
    out = {}
    for row in re.finditer(r"^\| (\w+)_kernel \| \d+ \| [\d.]+ \| [\d.]+ \| [\d.]+ \| ([\d.]+) \| ([\d.]+) \|", text, re.M):
        out[row.group(1)] = (float(row.group(2)), float(row.group(3)))
    return out or None


def read_traffic(path: str, kernel: str):
    """HBM bytes per launch of `kernel` from a traffic summary, or None if the
    file is missing or the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^kernel_sources_sha256 (\S+)", text, re.M)
    if not m or m.group(1) != sources_hash():
        return None
    m = re.search(r"^kernel %s .* hbm_bytes_per_launch (\S+)" % re.escape(kernel), text, re.M)
    return float(m.group(1)) if m else None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        sys.stdout.write(stats_markdown(sys.argv[2], " ".join(sys.argv[3:])))
    elif sys.argv[1] == "util":
        sys.stdout.write(util_markdown(sys.argv[2], " ".join(sys.argv[3:])))
    elif sys.argv[1] == "issue":
        sys.stdout.write(issue_markdown(sys.argv[2:4], " ".join(sys.argv[4:])))
    elif sys.argv[1] == "traffic":
        # copy size of the first permute of a bench step: Q of the workload
        # (c5 unless "--workload cN" follows the two files)
        import synthetic
        rest = sys.argv[4:]
        name = "c5"
        if rest and rest[0].startswith("--workload="):
            name = rest[0].split("=", 1)[1]
            rest = rest[1:]
        w = synthetic.WORKLOADS[name]
        copy_bytes = float(w.total * w.hq * w.d * (2 if w.dtype == "bf16" else 4))
        sys.stdout.write(traffic_text(sys.argv[2], sys.argv[3], " ".join(rest), copy_bytes))
    else:
        raise SystemExit("usage: profiling.py stats|util|issue|traffic ...")
