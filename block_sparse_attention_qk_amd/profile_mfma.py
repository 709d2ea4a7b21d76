"""Matrix-core utilisation and clock per kernel from one rocprofv3 counter run.

    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_BUSY_CYCLES \\
        --kernel-trace --stats --output-format csv -d DIR -o run -- python3 bench.py ...
    python -m block_sparse_attention_qk_amd.profile_mfma --run DIR [--run DIR ...] \\
        --out-md F.md --command "..."

Per dispatch the counters are summed over the device: GRBM_GUI_ACTIVE over
the 8 XCDs (so /8 gives the graphics-busy cycles of the dispatch) and
SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs (256 CUs x 4).  Hence, with the
dispatch's duration t from the kernel trace of the same run:

    clock     = GRBM_GUI_ACTIVE / 8 / t
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / (GRBM_GUI_ACTIVE / 8)

MFMA busy is the fraction of the busy cycles in which a SIMD's matrix unit
worked; at full rate it is the fraction of the bf16 peak at that clock.
"""

from __future__ import annotations

import argparse
import csv
import glob
import os
from collections import defaultdict

N_XCD = 8
N_SIMD = 256 * 4


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("sva::(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def _one(path_glob: str) -> str:
    files = glob.glob(path_glob, recursive=True)
    if not files:
        raise FileNotFoundError(path_glob)
    return files[0]


def summarize(run_dir: str):
    counters = defaultdict(dict)          # dispatch id -> counter -> value
    names = {}
    with open(_one(os.path.join(run_dir, "**", "*counter_collection.csv"))) as fh:
        for r in csv.DictReader(fh):
            d = int(r["Dispatch_Id"])
            counters[d][r["Counter_Name"]] = float(r["Counter_Value"])
            names[d] = _short(r["Kernel_Name"])
    # durations from the kernel trace of the same run, else from the
    # counter records' own timestamps
    dur = {}
    traces = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    src = traces[0] if traces else _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    with open(src) as fh:
        for r in csv.DictReader(fh):
            dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    per = defaultdict(list)
    for d, c in counters.items():
        if d not in dur or "GRBM_GUI_ACTIVE" not in c or c["GRBM_GUI_ACTIVE"] <= 0:
            continue
        busy = c["GRBM_GUI_ACTIVE"] / N_XCD
        per[names[d]].append((dur[d], busy / dur[d] / 1e9,
                              c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / N_SIMD / busy))
    out = {}
    for k, v in per.items():
        n = len(v)
        out[k] = {"dispatches": n, "avg_ms": sum(x[0] for x in v) / n * 1e3,
                  "clock_ghz": sum(x[1] for x in v) / n, "mfma_busy": sum(x[2] for x in v) / n}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--run", action="append", required=True,
                    help="rocprofv3 output directory; LABEL=DIR to name it")
    ap.add_argument("--out-md", required=True)
    ap.add_argument("--title", default="Matrix-core utilisation and clock per kernel")
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    lines = [f"# {a.title}", "", "Commands (from the repository root, on the machine with the GPU):", "", "```", a.command, "```", "",
             "clock = GRBM_GUI_ACTIVE / 8 / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / "
             "(GRBM_GUI_ACTIVE / 8) (counters summed over 8 XCDs and 1024 SIMDs).", "",
             "| run | kernel | dispatches | avg ms | clock GHz | MFMA busy |", "|---|---|---|---|---|---|"]
    for spec in a.run:
        label, _, path = spec.rpartition("=")
        label = label or os.path.basename(path.rstrip("/"))
        res = summarize(path)
        for k in sorted(res, key=lambda k: -res[k]["avg_ms"]):
            e = res[k]
            if k.startswith("__amd") or "elementwise" in k:
                continue
            lines.append(f"| {label} | `{k}` | {e['dispatches']} | {e['avg_ms']:.3f} | "
                         f"{e['clock_ghz']:.2f} | {100 * e['mfma_busy']:.1f} % |")
            print(f"{label:22s} {k:45s} {e['avg_ms']:9.3f} ms {e['clock_ghz']:5.2f} GHz "
                  f"MFMA {100 * e['mfma_busy']:5.1f} %")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
