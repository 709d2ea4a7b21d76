"""Per-kernel averages of one rocprofv3 counter run, as a short summary.

    rocprofv3 --pmc C1 C2 ... --kernel-trace --output-format csv -d DIR -o run -- \\
        python3 bench.py --workload W --steps 2 --warmup 1 --no-cpu-baseline \\
        --no-h3-prologue --no-copy-ref
    python -m block_sparse_attention_qk_amd.profile_counters --run DIR --out-md F.md \\
        --title "..." --command "..."

Every counter is summed over the device per dispatch (rocprofv3 reports one
value per dispatch and counter) and averaged over the dispatches of each
kernel.  When the LDS counters are present, the table adds two ratios:
bank-conflict cycles over LDS-active cycles, and cycles waves spent waiting
for LDS over wave cycles.  With SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
it adds the matrix units' busy share (busy cycles over the 1024 SIMDs, over
the graphics-active cycles of the 8 XCDs), and with
SQ_VALU_MFMA_COEXEC_CYCLES the share of those busy cycles in which vector
instructions executed beside the matrix instructions.
"""

from __future__ import annotations

import argparse
import csv
import glob
import os
from collections import defaultdict


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("sva::(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def read_run(run_dir: str) -> dict:
    """{kernel: {counter: average per dispatch}} from a counter-collection csv."""
    path = glob.glob(os.path.join(run_dir, "*counter_collection.csv"))
    assert path, f"no counter_collection.csv under {run_dir}"
    tot = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(set)
    with open(path[0]) as fh:
        for r in csv.DictReader(fh):
            k = _short(r["Kernel_Name"])
            tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[k].add(r["Dispatch_Id"])
    return {k: {c: v / len(disp[k]) for c, v in cs.items()} for k, cs in tot.items()}


def to_markdown(res: dict, title: str, command: str) -> str:
    counters = sorted({c for cs in res.values() for c in cs})
    lds = {"SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"}
    ratios = lds <= set(counters)
    mfma = {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"} <= set(counters)
    coex = mfma and "SQ_VALU_MFMA_COEXEC_CYCLES" in counters
    head = ["kernel"] + counters + (["bank conflict / LDS active", "LDS wait / wave cycles"]
                                    if ratios else []) + (["MFMA busy"] if mfma else []) + (
                                        ["vector co-exec / MFMA busy"] if coex else [])
    lines = [f"# {title}", "", "Command (from the repository root, on the machine with the GPU):", "",
             "```", command, "```", "",
             "Averages per dispatch of each counter, summed over the device.", "",
             "| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    for k, cs in sorted(res.items(), key=lambda kv: -kv[1].get("SQ_BUSY_CYCLES", 0.0)):
        row = [f"`{k}`"] + [f"{cs.get(c, 0.0):.3e}" for c in counters]
        if ratios:
            act = cs["SQ_LDS_IDX_ACTIVE"]
            row.append(f"{cs['SQ_LDS_BANK_CONFLICT'] / act:.3f}" if act > 0 else "—")
            row.append(f"{cs['SQ_WAIT_INST_LDS'] / cs['SQ_WAVE_CYCLES']:.3f}"
                       if cs["SQ_WAVE_CYCLES"] > 0 else "—")
        if mfma:
            g = cs["GRBM_GUI_ACTIVE"] / 8
            busy = cs["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024
            row.append(f"{busy / g * 100:.1f} %" if g > 0 else "—")
        if coex:
            b = cs["SQ_VALU_MFMA_BUSY_CYCLES"]
            row.append(f"{cs['SQ_VALU_MFMA_COEXEC_CYCLES'] / b * 100:.1f} %" if b > 0 else "—")
        lines.append("| " + " | ".join(row) + " |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--run", required=True)
    ap.add_argument("--out-md", required=True)
    ap.add_argument("--title", default="Counters per kernel")
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    res = read_run(a.run)
    with open(a.out_md, "w") as f:
        f.write(to_markdown(res, a.title, a.command))
    for k, cs in res.items():
        print(k, {c: f"{v:.3e}" for c, v in cs.items()})


if __name__ == "__main__":
    main()
