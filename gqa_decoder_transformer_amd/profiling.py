"""Turns rocprofv3 hardware-counter output into per-launch HBM traffic for one kernel.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` report, per dispatch, the KiB the
L2 fetched from and wrote to device memory. Those counts are scaled by what the same
counters read for a plain device copy of known size (run with ``bench.py
--calibrate-copy BYTES``), and averaged over the dispatches of the kernel of interest.

  python -m gqa_decoder_transformer_amd.profiling \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \\
      --kernel-regex REGEX --name decode.gate_up --workload qwen05b --precision exact \\
      --source gqa_decoder_transformer_amd/csrc/kernels_gemv.hip --out profiles/pmc_traffic.json

The record keeps the SHA-256 of the kernel's source file; bench.py reports the traffic
only while that file is unchanged.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics


def counter_values(directory, counter, kernel_regex):
    """Counter values (one per dispatch) of the kernels whose name matches."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    pat = re.compile(kernel_regex)
    per_dispatch = {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter or not pat.search(row.get("Kernel_Name", "")):
                    continue
                key = (f, row.get("Dispatch_Id"))
                per_dispatch[key] = per_dispatch.get(key, 0.0) + float(row["Counter_Value"])
    return list(per_dispatch.values())


def source_sha256(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-bytes", type=float, required=True)
    ap.add_argument("--copy-regex", default=r"copy|Copy")
    ap.add_argument("--kernel-regex", required=True)
    ap.add_argument("--name", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--precision", required=True)
    ap.add_argument("--source", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    cf = counter_values(a.copy_fetch, "FETCH_SIZE", a.copy_regex)
    cw = counter_values(a.copy_write, "WRITE_SIZE", a.copy_regex)
    kf = counter_values(a.fetch, "FETCH_SIZE", a.kernel_regex)
    kw = counter_values(a.write, "WRITE_SIZE", a.kernel_regex)
    if not (cf and cw and kf and kw):
        raise SystemExit(f"missing dispatches: copy {len(cf)}/{len(cw)}, kernel {len(kf)}/{len(kw)}")
    scale_f = a.copy_bytes / (max(cf) * 1024.0)
    scale_w = a.copy_bytes / (max(cw) * 1024.0)
    fetch = statistics.mean(kf) * 1024.0 * scale_f
    write = statistics.mean(kw) * 1024.0 * scale_w
    rec = {
        "name": a.name, "workload": a.workload, "precision": a.precision,
        "kernel_regex": a.kernel_regex, "dispatches": len(kf),
        "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
        "bytes_per_launch": fetch + write,
        "copy_bytes": a.copy_bytes, "copy_fetch_kib": max(cf), "copy_write_kib": max(cw),
        "scale_fetch": scale_f, "scale_write": scale_w,
        "source": a.source, "source_sha256": source_sha256(a.source), "command": a.command,
    }
    recs = []
    if os.path.exists(a.out):
        with open(a.out) as fh:
            recs = [r for r in json.load(fh)
                    if not (r["name"] == a.name and r["workload"] == a.workload and r["precision"] == a.precision)]
    recs.append(rec)
    with open(a.out, "w") as fh:
        json.dump(recs, fh, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
