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

Usage::

    python -m chunked_prefill_mixed_amd.counters trace KERNEL_TRACE.csv OUT.txt --command "..."
    python -m chunked_prefill_mixed_amd.counters traffic --workload heavy_mixed \\
        --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
        --out-dir profiles --command "..."
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
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


def library_source_hash() -> str:
    """Hash of every source that shapes what the library's kernels do: the
    kernels, their launchers and the host work planner (which decides the
    splits and with them the partial-result traffic).  The bench's own
    ceiling probes are left out."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")) and f != "peaks.hip":
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def short_name(kernel_name: str) -> str | None:
    for prefix, short in KERNELS.items():
        if prefix in kernel_name:
            return short
    return None


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def trace_summary(path: str) -> dict:
    """{kernel name: [durations in us]} from a kernel-trace CSV."""
    out = defaultdict(list)
    for r in _rows(path):
        name = r.get("Kernel_Name", "")
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        out[name].append((t1 - t0) / 1e3)
    return out


def write_trace(path: str, out: str, command: str) -> None:
    durs = trace_summary(path)
    lines = [f"command: {command}",
             "source: rocprofv3 --kernel-trace (csv), durations in microseconds", "",
             f"{'kernel':58s} {'calls':>6s} {'mean_us':>10s} {'min_us':>10s} {'median_us':>10s} "
             f"{'max_us':>10s}"]
    for name, d in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name[:58]:58s} {len(d):6d} {statistics.fmean(d):10.2f} {min(d):10.2f} "
                     f"{statistics.median(d):10.2f} {max(d):10.2f}")
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
    a = ap.parse_args()
    if a.cmd == "trace":
        write_trace(a.csv, a.out, a.command)
    else:
        for p in write_traffic(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write,
                               a.out_dir, a.command):
            print(p)


if __name__ == "__main__":
    main()
