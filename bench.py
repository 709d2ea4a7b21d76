"""Benchmark of the whole sparse self-attention step on one MI355X.

One step = QK-RMSNorm + 3D-RoPE written straight into the attention layouts,
reorder of V into V tiles, block selection, block-sparse attention writing O
straight into raster order, in one sva_forward call whose marks time each
stage (``--staged``: one call per stage, with separate reorders of Q', K'
and O), on synthetic inputs already resident in HBM.  Default workload: Wan2.1-14B-like 720p latent
grid 21×45×80 = 75,600 tokens, 40 heads, d 128, 128-token blocks,
sparsity 0.75, same-frame key blocks always kept.

Timing follows the per-kernel method of the MiniMax-H3 benchmark page
(section "内核层"): warm-up calls, then 10 rounds of steps/10 calls, each
call's stages bracketed by HIP events on the stream they run on, and the
median over all calls.  ``steps`` is the number of timed calls.

Prints one JSON line.  ``value`` is the executed attention work of a step
(4·block²·d flops per kept block pair) divided by the step's median time;
the attention kernel alone is reported in ``roofline`` against the bf16
dense MFMA peak.  ``h3_prologue`` times the raster prologue at that page's
per-rank shape (4,722 rows, 56 heads, RoPE over 96 of 128 channels).
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
step and scales it to the same unit.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "executed attn TFLOP/s (% bf16 MFMA peak) + ms/layer at 75.6k tokens, sp=0.75"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed steps: 10 rounds of steps/10 calls (fewer than 10: one call "
                         "per round); the figures are medians of the per-call event times")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan720p_sp75")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "kernel that scales the profiler's byte counters)")
    ap.add_argument("--staged", action="store_true",
                    help="one call per stage (raster prologue, separate reorders, tile-order "
                         "attention, inverse reorder) instead of the fused step")
    ap.add_argument("--cpu-heads", type=int, default=2,
                    help="heads the CPU oracle runs the whole step on (bounded sample)")
    ap.add_argument("--no-copy-ref", action="store_true",
                    help="skip the streaming-copy reference measurement")
    ap.add_argument("--no-h3-prologue", action="store_true",
                    help="skip the prologue timing at the packed video + audio model's "
                         "per-rank shape (4,722 rows, 56 heads, RoPE over 96 of 128 channels)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the path shards by head with no exchange, "
              "and runs on more than one GPU are not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_qk_amd as S
    from block_sparse_attention_qk_amd import inputs as I

    wl = I.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    t0 = time.time()
    q, k, v = (I.full_tensor(wl, t) for t in (I.TENSOR_Q, I.TENSOR_K, I.TENSOR_V))
    wq, wk = I.norm_weights(wl)
    print(f"inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    dwq, dwk = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    plan = S.sva_plan_create_ex(S.desc_for(wl))
    info = plan.info
    buf = S.Buffers(plan)
    stream = torch.cuda.current_stream()

    if args.staged:
        names = ["prologue", "reorder_qk", "reorder_v", "select", "means", "attention", "reorder_o"]
    else:
        names = ["prologue", "reorder_v", "select", "means", "attention"]
    n_marks = len(names) + 1
    assert args.staged or n_marks == S.SVA_FORWARD_MARKS

    def step(ev=None):
        if not args.staged:
            # the whole step in one library call; its marks bracket the
            # stages: prologue, V reorder, select, means, attention
            S.forward(plan, dq, dk, dv, dwq, dwk, buf, marks=ev)
            return
        # ev: len(names) + 1 events bracketing the stages of this step
        k = [0]

        def rec():
            if ev:
                ev[k[0]].record(stream)
            k[0] += 1

        rec()
        if args.staged:
            # one call per stage: raster prologue, reorders, tile-order
            # attention, inverse reorder
            S.sva_qk_norm_rope(plan, dq, dk, dwq, dwk, buf.qn, buf.kn)
            rec()
            S.sva_reorder(plan, buf.qn, buf.q_r, S.SVA_FORWARD)
            S.sva_reorder(plan, buf.kn, buf.k_t, S.SVA_FORWARD_KT)
            rec()
        else:
            # fused: the prologue writes Q' in tile order, K' as K tiles and
            # the block means the selection ranks
            S.sva_qk_norm_rope_tiled(plan, dq, dk, dwq, dwk, buf.q_r, buf.k_t,
                                     None if info.dense else buf.ws)
            rec()
        S.sva_reorder(plan, dv, buf.v_t, S.SVA_FORWARD_VT)
        rec()
        if not info.dense:
            if args.staged:
                S.sva_select_blocks(plan, buf.q_r, buf.k_t, buf.ws, buf.col)
            else:
                S.sva_select_blocks(plan, None, None, buf.ws, buf.col)
        rec()
        if plan.compensated:
            S.sva_block_means(plan, buf.k_t, buf.v_t, buf.km_t, buf.vm_t)
        rec()
        if args.staged:
            S.sva_attention_ws(plan, buf.q_r, buf.k_t, buf.v_t, buf.col, buf.km_t, buf.vm_t,
                               buf.o_r, S.SVA_LAYOUT_TILE, buf.aws)
            rec()
            S.sva_reorder(plan, buf.o_r, buf.o, S.SVA_INVERSE)
            rec()
        else:
            # O straight into raster order
            S.sva_attention_ws(plan, buf.q_r, buf.k_t, buf.v_t, buf.col, buf.km_t, buf.vm_t,
                               buf.o, S.SVA_LAYOUT_RASTER, buf.aws)
            rec()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        # one copy of known size, to scale the profiler's byte counters
        n = args.calib_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        S.sva_stream_copy(dst, src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: exactly `steps` steps, in `rounds` rounds of `calls`
    # calls; every call brackets its stages with HIP events on the stream
    rounds = min(10, args.steps)
    calls = args.steps // rounds
    nsteps = rounds * calls
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)]
              for _ in range(nsteps)]
    for e in events:           # torch creates an event when it is first recorded
        for x in e:
            x.record(stream)
    rs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(rounds)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for r in range(rounds):
        rs[r][0].record(stream)
        for c in range(calls):
            step(events[r * calls + c])
        rs[r][1].record(stream)
        torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    region_ms = sum(a.elapsed_time(b) for a, b in rs)
    per_call = [e[0].elapsed_time(e[-1]) for e in events]
    ms_step = float(np.median(per_call))

    def med(i, j):
        return float(np.median([e[i].elapsed_time(e[j]) for e in events]))

    stage = {n: med(i, i + 1) for i, n in enumerate(names)}

    b, d, H, B = wl.block, wl.d, wl.H, wl.B
    nnz = int(info.nnz)
    attn_flop = 4.0 * b * b * d * nnz
    attn_ms = stage["attention"]
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    value = attn_flop / (ms_step * 1e-3) / 1e12
    N, Np, nB = int(info.N), int(info.Np), int(info.nB)
    pro_bytes = 4.0 * B * N * H * d * 2
    nsub = int(info.subblocks)
    sel_bytes = 2.0 * B * H * Np * d * 2 + 2.0 * B * H * nB * nsub * d * 8 + 4.0 * nnz
    stage_gbs = {
        "prologue": pro_bytes / (stage["prologue"] * 1e-3) / 1e9,
        "reorder_v": (B * H * (N + Np) * d * 2) / (stage["reorder_v"] * 1e-3) / 1e9,
    }
    if args.staged:
        stage_gbs["reorder_qk"] = 2 * (B * H * (N + Np) * d * 2) / (stage["reorder_qk"] * 1e-3) / 1e9
        stage_gbs["reorder_o"] = (B * H * (N + Np) * d * 2) / (stage["reorder_o"] * 1e-3) / 1e9
    if not info.dense:
        if args.staged:
            stage_gbs["select"] = sel_bytes / (stage["select"] * 1e-3) / 1e9
        else:
            # the fused path pools inside the prologue; its select reads the
            # block means and writes the block lists
            rank_bytes = 2.0 * B * H * nB * nsub * d * 8 + 4.0 * nnz
            stage_gbs["select"] = rank_bytes / (stage["select"] * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": {"rounds": rounds, "calls_per_round": calls,
                   "statistic": "median of the per-call HIP event times",
                   "ms_per_step_mean": round(region_ms / nsteps, 4),
                   "timed_region_ms": round(region_ms, 2)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "B": B, "H": H, "d": d,
            "grid": f"{wl.T}x{wl.Hh}x{wl.W}", "tokens": N, "n_extra": wl.n_extra,
            "block": b, "sparsity": wl.sparsity, "keep_same_frame": bool(wl.flags & I.KEEP_SAME_FRAME),
            "dense": bool(info.dense), "kept_block_pairs": nnz,
            "path": "staged" if args.staged else "fused (one sva_forward call)",
            "executed_attn_tflop": round(attn_flop / 1e12, 3),
        },
        "roofline": {
            "kernel": "attn_kernel<128,128>" if (d == 128 and b == 128) else f"attn_kernel<{d},{b}>",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(wl.name, d, b),
        },
        "stages_ms": {n: round(t, 4) for n, t in stage.items()},
        "stages_hbm_gbs": {n: round(t, 1) for n, t in stage_gbs.items()},
        "stages_hbm_frac": {n: round(t / PEAK_HBM_GBS, 4) for n, t in stage_gbs.items()},
        "attn_ms": round(attn_ms, 4),
        "wall_s_timed": round(wall, 3),
    }

    if not args.no_copy_ref:
        copy = hbm_copy(S, np, torch)
        out["hbm_copy"] = copy
        out["stages_vs_copy"] = {n: round(t / copy["gbs"], 4) for n, t in stage_gbs.items()}
    if not args.no_h3_prologue:
        out["h3_prologue"] = h3_prologue(S, I, np, torch, to_dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, q, k, v, wq, wk, info, args.cpu_heads, ms_step)
    print(json.dumps(out), flush=True)


def hbm_copy(S, np, torch, mib=1024):
    """The library's streaming copy of `mib` MiB (read + write = 2·mib MiB
    moved), timed like the step: median of 10 rounds x 20 calls.  The
    attainable read + write rate on this part, beside the data sheet's."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        S.sva_stream_copy(dst, src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(200)]
    torch.cuda.synchronize()
    for r in range(10):
        for c in range(20):
            a, b = ev[r * 20 + c]
            a.record(stream)
            S.sva_stream_copy(dst, src)
            b.record(stream)
        torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    ok = bool(torch.equal(dst[:4096], src[:4096]))
    del src, dst
    gbs = 2.0 * n / (ms * 1e-3) / 1e9
    return {"bytes_moved": 2 * n, "ms": round(ms, 4), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "copied_ok": ok,
            "kernel": "stream_copy_kernel (16-byte accesses, 4 per thread in flight)"}


def h3_prologue(S, I, np, torch, to_dev):
    """The raster prologue (QK-RMSNorm + 3D-RoPE of Q and K) at the packed
    video + audio model's per-rank shape, timed the pages' way: the median
    of the per-call event times over 10 rounds of 20 calls."""
    wl = I.WORKLOADS["h3_prologue"]
    q = to_dev(I.full_tensor(wl, I.TENSOR_Q))
    k = to_dev(I.full_tensor(wl, I.TENSOR_K))
    plan = S.sva_plan_create_ex(S.desc_for(wl))
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    stream = torch.cuda.current_stream()
    for _ in range(5):
        S.sva_qk_norm_rope(plan, q, k, None, None, qo, ko)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(200)]
    torch.cuda.synchronize()
    for r in range(10):
        for c in range(20):
            a, b = ev[r * 20 + c]
            a.record(stream)
            S.sva_qk_norm_rope(plan, q, k, None, None, qo, ko)
            b.record(stream)
        torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    nbytes = 4.0 * wl.N * wl.H * wl.d * 2
    S.sva_destroy(plan)
    return {"rows": wl.N, "heads": wl.H, "d": wl.d, "rope_dims": sum(wl.rope_split),
            "grid": f"{wl.T}x{wl.Hh}x{wl.W}", "ms": round(ms, 5),
            "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bytes": nbytes, "statistic": "median of 10 rounds x 20 calls"}


def measured_traffic(workload, d, b):
    """HBM bytes per launch of the attention kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when there is none for this workload or the attention source or its
    build options have changed since the counters were taken."""
    from block_sparse_attention_qk_amd import profile_traffic as PT
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        res = json.load(f)
    now, then = PT.source_hashes(), res.get("sources_sha256", {})
    # the attention source and the compiler options it was built with
    if any(then.get(f) != now.get(f) for f in ("k_attention.hip", "k_attention.hip:flags")):
        return None
    for name, e in res.get("kernels", {}).items():
        if name.startswith(f"attn_kernel<{d}, {b}, "):
            return round(e["traffic_bytes"], 0)
    return None


def cpu_baseline(wl, q, k, v, wq, wk, info, heads, gpu_ms):
    """Time the CPU oracle on a bounded sample: the whole step (prologue,
    reorder, pooling, selection and attention over every query block) for
    the first `heads` heads; scale to all heads and express the result in
    the same unit as ``value`` (executed attention flops per second)."""
    import oracle.sva_oracle as O

    g = O.Geometry(B=wl.B, H=wl.H, T=wl.T, Hh=wl.Hh, W=wl.W, d=wl.d, block=wl.block,
                   sparsity=wl.sparsity, flags=wl.flags, tile=wl.tile, n_extra=wl.n_extra,
                   split=wl.rope_split, scorer=wl.scorer, subblocks=wl.subblocks,
                   budget_multiple=max(1, wl.budget_multiple), theta=wl.theta_resolved,
                   eps=wl.eps_resolved)
    cores = len(os.sched_getaffinity(0))
    heads = max(1, min(heads, wl.H))
    t0 = time.perf_counter()
    perm = O.permutation(g)
    meta = O.block_meta(g, perm)
    t1 = time.perf_counter()
    for h in range(heads):
        O.run_head(O.bf16_bits_to_f64(q[0, :, h]), O.bf16_bits_to_f64(k[0, :, h]),
                   O.bf16_bits_to_f64(v[0, :, h]), wq[h], wk[h], g, perm=perm, meta=meta)
    t2 = time.perf_counter()
    layer_s = (t1 - t0) + (t2 - t1) / heads * wl.H * wl.B
    attn_flop = 4.0 * g.block ** 2 * g.d * int(info.nnz)
    return {
        "value": round(attn_flop / layer_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"whole step for {heads} of {wl.H} heads (all {g.nB} query blocks), "
                   f"measured {t2 - t0:.1f}s, scaled to {layer_s:.1f}s per step "
                   f"(GPU {gpu_ms:.2f} ms per step)"),
        "measured_s": round(t2 - t0, 2),
        "extrapolated_step_s": round(layer_s, 2),
    }


if __name__ == "__main__":
    main()
