"""HBM bytes per kernel from two rocprofv3 counter runs.

    python -m block_sparse_attention_qk_amd.profile_traffic \\
        --fetch DIR_WITH_FETCH_SIZE_RUN --write DIR_WITH_WRITE_SIZE_RUN \\
        --calib-mib 1024 [--stats KERNEL_STATS_CSV] --out-json F.json --out-md F.md

Both runs profile ``bench.py --calib-copy-mib N``, which does one plain
device-to-device copy of N MiB (the library's streaming copy kernel, which
reads and writes exactly N MiB) next to the step's kernels.  rocprofv3 reports ``FETCH_SIZE`` and
``WRITE_SIZE`` in KiB per dispatch; the counters need not count every byte
(the read counter sees about half of a copy's reads on this part), so each
is scaled by known bytes / counted bytes of that copy.  The result is the
average HBM-side bytes per dispatch of every kernel, and, with the
kernel-trace statistics of the same command, the achieved GB/s.

The json also records the SHA-256 of every HIP source and of its compiler
options, so a reader (bench.py) can tell whether the figures still describe
the kernels that are built.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


def source_hashes() -> dict:
    """SHA-256 of every kernel source, and of each HIP source's compiler
    options (key "<source>:flags"), which shape its code as much as the
    source does."""
    from block_sparse_attention_qk_amd.build import flag_signature
    out = {}
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        name = os.path.basename(path)
        with open(path, "rb") as f:
            out[name] = hashlib.sha256(f.read()).hexdigest()
        if name.endswith(".hip"):
            out[name + ":flags"] = hashlib.sha256(flag_signature(name).encode()).hexdigest()
    return out


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("sva::(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def _counter_rows(run_dir: str, counter: str):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = defaultdict(list)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


def _is_copy(name: str) -> bool:
    """The calibration copy: the library's streaming copy kernel (or the
    runtime's blit kernel in older runs)."""
    return "stream_copy_kernel" in name or "copyBuffer" in name


def _calibration(per: dict, calib_bytes: float) -> float:
    copies = [v for k, vs in per.items() if _is_copy(k) for v in vs]
    if not copies:
        raise ValueError("no copy kernel in the counter run (run bench.py with --calib-copy-mib)")
    counted = max(copies) * 1024.0
    return calib_bytes / counted


def summarize(fetch_dir, write_dir, calib_mib, stats_csv=None):
    calib = calib_mib * float(1 << 20)
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")
    f_fac = _calibration(fetch, calib)
    w_fac = _calibration(write, calib)
    dur = {}
    if stats_csv:
        with open(stats_csv) as fh:
            for r in csv.DictReader(fh):
                dur[_short(r["Name"])] = float(r["AverageNs"]) * 1e-9
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        if _is_copy(k):
            continue
        fb = (sum(fetch.get(k, [0])) / max(1, len(fetch.get(k, [0])))) * 1024.0 * f_fac
        wb = (sum(write.get(k, [0])) / max(1, len(write.get(k, [0])))) * 1024.0 * w_fac
        e = {"fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
             "dispatches": len(fetch.get(k, []))}
        if k in dur:
            e["avg_s"] = dur[k]
            e["traffic_gbs"] = (fb + wb) / dur[k] / 1e9
        kernels[k] = e
    return {"calib_mib": calib_mib, "fetch_scale": f_fac, "write_scale": w_fac,
            "kernels": kernels, "sources_sha256": source_hashes()}


def to_markdown(res, title, command):
    lines = [f"# {title}", "", "Commands (from the repository root, on the machine with the GPU):", "", "```", command, "```", "",
             f"Calibration: one {res['calib_mib']} MiB device copy; FETCH_SIZE scaled by "
             f"{res['fetch_scale']:.3f}, WRITE_SIZE by {res['write_scale']:.3f} (known bytes / counted bytes).",
             "", "| kernel | read GB | written GB | total GB | avg ms | GB/s |", "|---|---|---|---|---|---|"]
    for k, e in res["kernels"].items():
        ms = f"{e['avg_s'] * 1e3:.3f}" if "avg_s" in e else "—"
        gbs = f"{e['traffic_gbs']:.0f}" if "traffic_gbs" in e else "—"
        lines.append(f"| `{k}` | {e['fetch_bytes'] / 1e9:.3f} | {e['write_bytes'] / 1e9:.3f} | "
                     f"{e['traffic_bytes'] / 1e9:.3f} | {ms} | {gbs} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--calib-mib", type=int, required=True)
    ap.add_argument("--stats")
    ap.add_argument("--out-json", required=True)
    ap.add_argument("--out-md")
    ap.add_argument("--title", default="HBM traffic per kernel")
    ap.add_argument("--command", default="")
    a = ap.parse_args()
    res = summarize(a.fetch, a.write, a.calib_mib, a.stats)
    res["command"] = a.command
    with open(a.out_json, "w") as f:
        json.dump(res, f, indent=1)
    if a.out_md:
        with open(a.out_md, "w") as f:
            f.write(to_markdown(res, a.title, a.command))
    for k, e in res["kernels"].items():
        print(f"{k:45s} {e['traffic_bytes'] / 1e9:8.3f} GB  {e.get('traffic_gbs', 0):8.0f} GB/s")


if __name__ == "__main__":
    main()
