"""Per-kernel averages of rocprofv3 counter runs, as a markdown table.

Reads every ``*counter_collection.csv`` under the given directories (one ``--pmc`` run
each), groups the dispatches by kernel name (kernels matching ``--kernel-regex``), and
prints per-dispatch means of each counter and of the dispatch duration, with derived
figures where their counters are present:

* TFLOP/s: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / duration;
* MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x duration x 2.4 GHz);
* waitcnt and LDS-issue stalls: SQ_WAIT_ANY and SQ_WAIT_INST_LDS over SQ_WAVE_CYCLES;
* LDS bank conflicts per LDS instruction;
* L2 hit rate: TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum);
* memory-side bytes: FETCH_SIZE (KiB) x the scale a plain copy calibrates.

  python -m gqa_decoder_transformer_amd.counter_summary DIR [DIR ...] \\
      --kernel-regex 'k_gemm<|k_flash_tiled' [--fetch-scale 2.0]
"""
import argparse
import csv
import glob
import os
import re
from collections import defaultdict

CLOCK_HZ = 2.4e9
SIMDS = 1024


def short_name(name):
    name = re.sub(r"void |ember::|\(anonymous namespace\)::", "", name)
    return re.sub(r"\(.*$", "", name)


def collect(directories, kernel_regex):
    """{kernel: {(run directory, counter or 'duration_us'): [per-dispatch values]}}"""
    pat = re.compile(kernel_regex)
    out = defaultdict(lambda: defaultdict(list))
    for d in directories:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter_collection.csv under {d}")
        for f in files:
            per = defaultdict(lambda: defaultdict(float))
            meta = {}
            with open(f, newline="") as fh:
                for row in csv.DictReader(fh):
                    if not pat.search(row.get("Kernel_Name", "")):
                        continue
                    key = row["Dispatch_Id"]
                    per[key][row["Counter_Name"]] += float(row["Counter_Value"])
                    meta[key] = (short_name(row["Kernel_Name"]),
                                 (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
            for key, counters in per.items():
                kname, dur = meta[key]
                for c, v in counters.items():
                    out[kname][(d, c)].append(v)
                out[kname][(d, "duration_us")].append(dur)
    return out


def derived(means, fetch_scale):
    """Figures from per-dispatch means {(run, counter): value}; rates use the duration
    measured in the same run as their counter."""
    val, run_of = {}, {}
    for (d, c), v in means.items():
        if c != "duration_us":
            val[c] = v
            run_of[c] = d
    dur = {d: v for (d, c), v in means.items() if c == "duration_us"}
    rows = {}
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in val:
        t = dur[run_of["SQ_INSTS_VALU_MFMA_MOPS_BF16"]]
        rows["TFLOP/s"] = val["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / (t * 1e-6) / 1e12
    if "SQ_VALU_MFMA_BUSY_CYCLES" in val:
        t = dur[run_of["SQ_VALU_MFMA_BUSY_CYCLES"]]
        rows["MFMA busy"] = val["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * t * 1e-6 * CLOCK_HZ)
    if "SQ_WAIT_ANY" in val and "SQ_WAVE_CYCLES" in val:
        rows["waitcnt / wave cycles"] = val["SQ_WAIT_ANY"] / val["SQ_WAVE_CYCLES"]
    if "SQ_WAIT_INST_LDS" in val and "SQ_WAVE_CYCLES" in val:
        rows["LDS issue wait / wave cycles"] = val["SQ_WAIT_INST_LDS"] / val["SQ_WAVE_CYCLES"]
    if "SQ_LDS_BANK_CONFLICT" in val and val.get("SQ_INSTS_LDS"):
        rows["LDS bank conflicts / LDS instr"] = val["SQ_LDS_BANK_CONFLICT"] / val["SQ_INSTS_LDS"]
    if "TCC_HIT_sum" in val and "TCC_MISS_sum" in val:
        tot = val["TCC_HIT_sum"] + val["TCC_MISS_sum"]
        rows["L2 hit rate"] = val["TCC_HIT_sum"] / tot if tot else 0.0
    if "FETCH_SIZE" in val:
        rows["memory-side fetch (MB)"] = val["FETCH_SIZE"] * 1024 * fetch_scale / 1e6
    return rows, dur


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--kernel-regex", required=True)
    ap.add_argument("--fetch-scale", type=float, default=2.0)
    args = ap.parse_args()
    data = collect(args.dirs, args.kernel_regex)
    print("| kernel | dispatches | avg us | figure | value |")
    print("|---|---:|---:|---|---:|")
    for k in sorted(data):
        means = {key: sum(v) / len(v) for key, v in data[k].items()}
        n = max(len(v) for v in data[k].values())
        rows, dur = derived(means, args.fetch_scale)
        t = sum(dur.values()) / len(dur) if dur else 0.0
        for fig, v in rows.items():
            print(f"| `{k}` | {n} | {t:.2f} | {fig} | {v:.3f} |")


if __name__ == "__main__":
    main()
