"""Per-kernel times of one rocprofv3 kernel-trace run, as a short summary.

    rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o bench -- \\
        python3 bench.py --workload W --steps 5 --warmup 1 --no-cpu-baseline \\
        --no-h3-prologue --no-copy-ref
    python -m block_sparse_attention_qk_amd.profile_kernels --stats DIR/bench_kernel_stats.csv \\
        --trace DIR/bench_kernel_trace.csv --bench-json B.json --title "..." \\
        --command "..." --out-md F.md

The statistics file gives calls and average, minimum and maximum duration
per kernel; ``--bench-json`` adds the bench line of the same box (the
attention kernel's event time and its fraction of the bf16 peak) so the two
can be compared.  With ``--flop`` the attention kernel's rocprof average is
also turned into TFLOP/s and a fraction of the bf16 dense peak.
"""

from __future__ import annotations

import argparse
import csv
import json

PEAK_BF16_TFLOPS = 2516.6


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("sva::(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def read_medians(trace_path: str) -> dict:
    """Median duration (ms) per kernel from a kernel-trace csv."""
    per = {}
    with open(trace_path) as fh:
        for r in csv.DictReader(fh):
            per.setdefault(_short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
    out = {}
    for k, v in per.items():
        v = sorted(v)
        n = len(v)
        out[k] = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return out


def read_stats(path: str):
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            rows.append({
                "kernel": _short(r["Name"]),
                "calls": int(r["Calls"]),
                "avg_ms": float(r["AverageNs"]) * 1e-6,
                "min_ms": float(r["MinNs"]) * 1e-6,
                "max_ms": float(r["MaxNs"]) * 1e-6,
                "share": float(r["Percentage"]),
            })
    rows.sort(key=lambda e: -e["share"])
    return rows


def to_markdown(rows, title, command, bench=None, flop=None, medians=None):
    medians = medians or {}
    lines = [f"# {title}", "", "Command (from the repository root, on the machine with the GPU):",
             "", "```", command, "```", "",
             "| kernel | calls | avg ms | median ms | min ms | max ms | share |",
             "|---|---|---|---|---|---|---|"]
    for e in rows:
        med = medians.get(e["kernel"])
        ms = f"{med:.3f}" if med is not None else "—"
        lines.append(f"| `{e['kernel']}` | {e['calls']} | {e['avg_ms']:.3f} | {ms} | "
                     f"{e['min_ms']:.3f} | {e['max_ms']:.3f} | {e['share']:.2f}% |")
    attn = [e for e in rows if e["kernel"].startswith("attn_kernel")]
    if flop and attn:
        a = attn[0]
        for label, t in (("average", a["avg_ms"]), ("median", medians.get(a["kernel"]))):
            if t is None:
                continue
            tf = flop / (t * 1e-3) / 1e12
            lines += ["", f"Attention from this profile ({label}): {flop / 1e12:.3f} TFLOP executed / "
                          f"{t:.3f} ms = {tf:.1f} TFLOP/s = {tf / PEAK_BF16_TFLOPS:.4f} of "
                          f"{PEAK_BF16_TFLOPS} TFLOP/s (bf16 dense)."]
    if bench:
        r = bench.get("roofline", {})
        lines += ["", "bench.py on the same box (median of the per-call HIP event times):", "",
                  f"- ms/step {bench.get('ms_per_step')}, attention {bench.get('attn_ms')} ms -> "
                  f"{r.get('achieved')} TFLOP/s = {r.get('frac')} of {r.get('peak')} TFLOP/s",
                  f"- stage ms: {bench.get('stages_ms')}",
                  f"- stage GB/s: {bench.get('stages_hbm_gbs')}"]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--trace", help="kernel-trace csv of the same run (per-dispatch medians)")
    ap.add_argument("--bench-json")
    ap.add_argument("--flop", type=float, default=None,
                    help="executed attention flops per call (4 block^2 d nnz)")
    ap.add_argument("--title", default="Kernel times")
    ap.add_argument("--command", default="")
    ap.add_argument("--out-md", required=True)
    a = ap.parse_args()
    bench = None
    if a.bench_json:
        with open(a.bench_json) as fh:
            bench = json.loads(fh.read().strip().splitlines()[-1])
    flop = a.flop
    if flop is None and bench:
        flop = bench.get("config", {}).get("executed_attn_tflop", 0) * 1e12 or None
    rows = read_stats(a.stats)
    medians = read_medians(a.trace) if a.trace else None
    with open(a.out_md, "w") as fh:
        fh.write(to_markdown(rows, a.title, a.command, bench, flop, medians))
    for e in rows:
        print(f"{e['kernel']:50s} {e['calls']:4d} {e['avg_ms']:9.3f} ms")


if __name__ == "__main__":
    main()
