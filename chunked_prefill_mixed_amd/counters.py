"""Summaries of rocprofv3 output for profiles/.

Two kinds of record, both written from the CSV files rocprofv3 leaves behind:

* ``trace``: a kernel-trace summary (``--kernel-trace --output-format csv``):
  per kernel the number of dispatches and the mean, minimum, median and
  maximum duration in microseconds, as a short text table.
* ``traffic``: HBM traffic per dispatch from two counter runs, one with
  ``--pmc FETCH_SIZE`` and one with ``--pmc WRITE_SIZE`` (KiB per dispatch,
  summed over the counter's instances), each scaled by what the same counter
  reads for a plain device copy of known size (``bench.py
  --copy-calibration`` under the same two counters).  One JSON record per
  kernel, ``profiles/<kernel>_<workload>_counters.json``, carrying the hash of
  the library sources it was taken on; ``bench.py`` reports the traffic only
  while that hash still matches.
* ``mfma``: matrix-core and LDS use per kernel from one counter run with
  ``--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
  SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_ANY SQ_WAVE_CYCLES
  SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --kernel-trace``, one text section per
  workload appended to the output file.  Derived per dispatch, then averaged:
  clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy =
  SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); issued bf16
  flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; LDS busy = SQ_LDS_IDX_ACTIVE /
  (GRBM_GUI_ACTIVE / 8 x 256 CUs); issue wait = SQ_WAIT_INST_ANY /
  SQ_WAVE_CYCLES (both in 4-cycle units).  The bench's MFMA-only loop
  (``mfma_kernel``) in the same run is the matrix-core ceiling under the same
  clock and power limits.

Usage::

    python -m chunked_prefill_mixed_amd.counters trace KERNEL_TRACE.csv OUT.txt --command "..."
    python -m chunked_prefill_mixed_amd.counters traffic --workload heavy_mixed \\
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
        --out-dir profiles --command "..."
    python -m chunked_prefill_mixed_amd.counters mfma --workload heavy_mixed \\
        --csv PMC.csv --out OUT.txt --command "..." [--algorithmic-gflop X]
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel name prefix in the traces -> short name used in profiles/ and bench.py
KERNELS = {
    "cpa::append_kernel": "append_kernel",
    "cpa::decode_kernel": "decode_kernel",
    "cpa::chunk_kernel": "chunk_kernel",
    "cpa::merge_kernel": "merge_kernel",
    "cpa::mixed_kernel": "mixed_kernel",
}
COPY_BYTES = 1 << 30  # bytes bench.py --copy-calibration copies per launch


def _code_only(text: str) -> str:
    """The source without its comments, trailing blanks and empty lines (the
    library's sources hold no string literal with a comment marker)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def library_source_hash() -> str:
    """Hash of the code of every source that shapes what the library's
    kernels do: the kernels, their launchers and the host work planner (which
    decides the splits and with them the partial-result traffic).  Comments
    and blank lines are left out, so a record stays valid across changes to
    them alone; the bench's own ceiling probes are left out."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")) and f != "peaks.hip":
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(kernel_name: str) -> str | None:
    for prefix, short in KERNELS.items():
        if prefix in kernel_name:
            return short
    return None


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def trace_summary(path: str, by_grid: bool = False) -> dict:
    """{kernel name: [durations in us]} from a kernel-trace CSV, or with
    by_grid {(kernel name, grid size in workgroups): [durations]}."""
    out = defaultdict(list)
    for r in _rows(path):
        name = r.get("Kernel_Name", "")
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        threads = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        wg = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 1)
        key = (name, threads // max(1, wg)) if by_grid else name
        out[key].append((t1 - t0) / 1e3)
    return out


def write_trace(path: str, out: str, command: str) -> None:
    durs = trace_summary(path)
    grids = trace_summary(path, by_grid=True)
    lines = [f"command: {command}",
             "source: rocprofv3 --kernel-trace (csv), durations in microseconds; a kernel "
             "launched with several grid sizes (different work) is also listed per grid size "
             "(workgroups)", "",
             f"{'kernel':58s} {'calls':>6s} {'mean_us':>10s} {'min_us':>10s} {'median_us':>10s} "
             f"{'max_us':>10s}"]
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name[:58]:58s} {len(d):6d} {statistics.fmean(d):10.2f} {min(d):10.2f} "
                     f"{statistics.median(d):10.2f} {max(d):10.2f}")
        mine = sorted((g, v) for (n, g), v in grids.items() if n == name)
        if len(mine) > 1 and short_name(name):
            for g, v in mine:
                lines.append(f"  {'grid ' + str(g) + ' workgroups':56s} {len(v):6d} "
                             f"{statistics.fmean(v):10.2f} {min(v):10.2f} "
                             f"{statistics.median(v):10.2f} {max(v):10.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(path: str, counter: str) -> dict:
    """{kernel name: [counter value per dispatch]}, summed over instances."""
    acc = defaultdict(float)
    names = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        acc[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for key, v in acc.items():
        out[names[key]].append(v)
    return out


def _copy_factor(path: str, counter: str) -> tuple[float, float]:
    """(KiB the counter reads per copy dispatch, bytes copied per byte the
    counter reads)."""
    d = _per_dispatch(path, counter)
    vals = [v for name, vs in d.items() if "elementwise" in name or "copy" in name.lower()
            for v in vs]
    vals = [v for v in vals if v > 0.25 * (COPY_BYTES / 1024) / 4]  # the 1 GiB copies only
    kib = statistics.median(vals)
    return kib, COPY_BYTES / (kib * 1024)


def write_traffic(workload: str, fetch: str, write: str, copy_fetch: str, copy_write: str,
                  out_dir: str, command: str) -> list[str]:
    f_d, w_d = _per_dispatch(fetch, "FETCH_SIZE"), _per_dispatch(write, "WRITE_SIZE")
    cf_kib, cf = _copy_factor(copy_fetch, "FETCH_SIZE")
    cw_kib, cw = _copy_factor(copy_write, "WRITE_SIZE")
    sha = library_source_hash()
    written = []
    for name in sorted(set(f_d) & set(w_d)):
        short = short_name(name)
        if short is None:
            continue
        fk, wk = statistics.fmean(f_d[name]), statistics.fmean(w_d[name])
        rec = {
            "kernel": name.split("(")[0],
            "workload": workload,
            "library_source_sha": sha,
            "command": command,
            "dispatches": min(len(f_d[name]), len(w_d[name])),
            "fetch_kib_per_dispatch": fk,
            "write_kib_per_dispatch": wk,
            "copy_calibration": {"bytes_copied": COPY_BYTES, "fetch_kib": cf_kib,
                                 "write_kib": cw_kib, "fetch_factor": cf, "write_factor": cw},
            "read_bytes_per_launch": fk * 1024 * cf,
            "write_bytes_per_launch": wk * 1024 * cw,
            "traffic_bytes_per_launch": fk * 1024 * cf + wk * 1024 * cw,
            "note": "mean over the dispatches of the run (the workload's instances rotate); "
                    "each counter scaled by the factor that maps a plain 1 GiB device copy's "
                    "reading to 1 GiB",
        }
        path = os.path.join(out_dir, f"{short}_{workload}_counters.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        written.append(path)
    return written


def traffic_record(kernel: str, workload: str, profiles_dir: str) -> dict | None:
    """The committed traffic record of a kernel on a workload, if it was taken
    on the current library sources."""
    path = os.path.join(profiles_dir, f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("library_source_sha") != library_source_hash():
        return None
    return rec


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_IDX_ACTIVE",
                 "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")
NUM_XCDS, NUM_SIMDS, NUM_CUS = 8, 1024, 256


def mfma_summary(path: str) -> dict:
    """{kernel name: {derived figure: mean over its dispatches}} from one
    counter run (see the module docstring for the formulas)."""
    per = defaultdict(lambda: defaultdict(float))
    meta = {}
    for r in _rows(path):
        key = r["Dispatch_Id"]
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        meta[key] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9)
    acc = defaultdict(lambda: defaultdict(list))
    for key, c in per.items():
        name, dur = meta[key]
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / NUM_XCDS
        if cyc <= 0 or dur <= 0:
            continue
        a = acc[name]
        a["us"].append(dur * 1e6)
        a["ghz"].append(cyc / dur / 1e9)
        a["mfma_busy"].append(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * NUM_SIMDS))
        flops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        a["gflop"].append(flops / 1e9)
        a["tflops"].append(flops / dur / 1e12)
        a["lds_busy"].append(c.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cyc * NUM_CUS))
        a["lds_conflict"].append(c.get("SQ_LDS_BANK_CONFLICT", 0.0))
        w = c.get("SQ_WAVE_CYCLES", 0.0)
        a["issue_wait"].append(c.get("SQ_WAIT_INST_ANY", 0.0) / w if w else 0.0)
    return {name: {k: statistics.fmean(v) for k, v in a.items()} | {"dispatches": len(a["us"])}
            for name, a in acc.items()}


def write_mfma(workload: str, path: str, out: str, command: str,
               algorithmic_gflop: float | None = None) -> None:
    """Append the workload's section to out (the file starts with the
    command and the formulas when it is new)."""
    summ = mfma_summary(path)
    lines = []
    if not os.path.exists(out):
        lines += [f"command: {command}",
                  "source: pmc_counter_collection.csv of rocprofv3, counters summed over their "
                  "instances per dispatch, figures averaged over each kernel's dispatches",
                  "derived: clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); issued GFLOP = "
                  "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; LDS busy = SQ_LDS_IDX_ACTIVE / "
                  "(GRBM_GUI_ACTIVE / 8 x 256 CUs); issue wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; "
                  "busy x GHz compares matrix-core work per second across kernels at their own "
                  "clocks; mfma_kernel is the bench's MFMA-only loop on random operands",
                  ""]
    alg = f"; algorithmic chunk GFLOP per launch {algorithmic_gflop:.1f}" if algorithmic_gflop else ""
    lines += [f"workload {workload}{alg}",
              f"  {'kernel':34s} {'disp':>4s} {'avg_us':>9s} {'GHz':>5s} {'MFMA':>6s} {'busyxGHz':>8s} "
              f"{'GFLOP':>8s} {'TFLOP/s':>8s} {'LDS':>5s} {'bank_cf':>7s} {'wait':>5s}"]
    order = sorted(summ.items(), key=lambda kv: -kv[1]["us"] * kv[1]["dispatches"])
    for name, f in order:
        if f["us"] < 20:
            continue
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")[:34]
        lines.append(f"  {short:34s} {f['dispatches']:4d} {f['us']:9.1f} {f['ghz']:5.2f} "
                     f"{100 * f['mfma_busy']:5.1f}% {f['mfma_busy'] * f['ghz']:8.3f} "
                     f"{f['gflop']:8.1f} {f['tflops']:8.0f} {100 * f['lds_busy']:4.0f}% "
                     f"{f['lds_conflict']:7.0f} {100 * f['issue_wait']:4.0f}%")
    lines.append("")
    with open(out, "a") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("--workload", required=True)
    for a in ("fetch", "write", "copy_fetch", "copy_write"):
        c.add_argument("--" + a.replace("_", "-"), required=True, dest=a)
    c.add_argument("--out-dir", required=True)
    c.add_argument("--command", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--workload", required=True)
    m.add_argument("--csv", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--algorithmic-gflop", type=float, default=None)
    a = ap.parse_args()
    if a.cmd == "trace":
        write_trace(a.csv, a.out, a.command)
    elif a.cmd == "mfma":
        write_mfma(a.workload, a.csv, a.out, a.command, a.algorithmic_gflop)
    else:
        for p in write_traffic(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write,
                               a.out_dir, a.command):
            print(p)


if __name__ == "__main__":
    main()
