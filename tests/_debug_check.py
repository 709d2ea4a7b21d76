"""Run the step through the debug library (device-side index checks) and the
release library in one fresh process, and compare.

    python tests/_debug_check.py [full]

For every case: the fused step (one sva_forward call) and the staged step
(one call per stage, every kernel of the library) through libsva.so, then
the same through libsva_debug.so.  The debug word must be zero after each
run, and every output (O, the block lists, the V tiles, the staged
intermediates) must equal the release library's bit for bit.  Then the
self-test kernel must set SVA_DEBUG_SELF, and reading the word clears it.
Prints one line per case and exits non-zero on the first mismatch.  Run in
a process of its own, since the binding holds one library at a time.
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import torch  # noqa: E402

import block_sparse_attention_qk_amd as S  # noqa: E402
from block_sparse_attention_qk_amd import inputs as I  # noqa: E402
from _parity import dev, workload_inputs  # noqa: E402
from test_gpu_parity import SMALL, SPLIT  # noqa: E402

CASES = ["tiny", "ragged128", "ragged64", "d64_b128", "dense128", "denseflag64", "sub64x4",
         "comp128", "comp64", "dense_d128_b64", "single", "sparse99", "split64", "split128",
         "split_comp"]
FULL_CASES = ["wan720p_sp75", "packed768p_sp80", "hunyuan720p_comp", "wan480p_subblock"]


def use(path):
    S.LIB_PATH = path
    S._lib = None


def run_once(wl, x, debug):
    """The fused and the staged step on one plan; returns the outputs and
    the debug word (None for the release library)."""
    plan = S.sva_plan_create_ex(S.desc_for(wl))
    fused, staged = S.Buffers(plan), S.Buffers(plan)
    S.forward(plan, *x, fused)
    S.forward_staged(plan, *x, staged)
    torch.cuda.synchronize()
    out = {"o": fused.o, "v_t": fused.v_t, "o_staged": staged.o, "q_r": staged.q_r,
           "k_t": staged.k_t, "o_r": staged.o_r}
    if fused.col is not None:
        out["col"] = fused.col
        out["col_staged"] = staged.col
    out = {k: v.clone() for k, v in out.items()}
    flags = S.sva_debug_flags(plan) if debug else None
    self_ok = None
    if debug:
        S.sva_debug_selftest(plan)
        self_ok = (S.sva_debug_flags(plan) == S.SVA_DEBUG_SELF and S.sva_debug_flags(plan) == 0)
    else:
        try:
            S.sva_debug_flags(plan)
            raise SystemExit("the release library accepted sva_debug_flags")
        except S.SvaError as e:
            assert e.status == S.SVA_ERR_UNSUPPORTED, e
    del fused, staged
    plan.__del__()
    return out, flags, self_ok


def main():
    torch.cuda.set_device(0)
    names = CASES + (FULL_CASES if "full" in sys.argv[1:] else [])
    for name in names:
        wl = SMALL.get(name) or SPLIT.get(name) or I.WORKLOADS[name]
        print(f"case {name}", flush=True)
        q, k, v, wq, wk = workload_inputs(wl)
        x = (dev(q), dev(k), dev(v), torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda())
        use(S.LIB_PATH_RELEASE)
        ref, _, _ = run_once(wl, x, False)
        use(S.DEBUG_LIB_PATH)
        got, flags, self_ok = run_once(wl, x, True)
        use(S.LIB_PATH_RELEASE)
        diff = [n for n in ref if not torch.equal(ref[n].view(torch.uint8), got[n].view(torch.uint8))]
        print(f"{name}: debug word {flags:#x}, self-test {'ok' if self_ok else 'FAILED'}, "
              f"outputs differing from the release library: {diff or 'none'}", flush=True)
        if flags != 0 or not self_ok or diff:
            sys.exit(1)
        del x, ref, got
        torch.cuda.empty_cache()
    print("debug check passed", flush=True)


if __name__ == "__main__":
    S.LIB_PATH_RELEASE = S.LIB_PATH
    main()
