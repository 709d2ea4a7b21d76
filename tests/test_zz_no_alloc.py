"""sva_select_blocks_noalloc (the selection on the library's fixed device
scratch, for callers that cannot allocate) against sva_select_blocks with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller plan, each list bit-identical to the workspace call's; a plan whose
block means exceed the scratch is refused before any work is enqueued."""

import numpy as np
import pytest
import torch

import block_sparse_attention_qk_amd as S
from block_sparse_attention_qk_amd import inputs as I
from _parity import GpuRun, workload_inputs

pytestmark = pytest.mark.gpu

# the larger call first: 12 heads of 512 blocks, then the small ragged one
_BIG = I.WORKLOADS["wan480p_sp75"]
_SMALL = I.custom("noalloc_small", 2, 3, 5, 13, 17, 128, 128, 0.6, flags=I.KEEP_SAME_FRAME,
                  n_extra=128, temperature=True, seed_base=12000)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def _select_both(wl):
    run = GpuRun(wl, *workload_inputs(wl))
    b = run.buf
    S.sva_qk_norm_rope_tiled(run.plan, run.q, run.k, run.wq, run.wk, b.q_r, b.k_t)
    S.sva_select_blocks(run.plan, b.q_r, b.k_t, b.ws, b.col)
    col2 = torch.full_like(b.col, -7)
    S.sva_select_blocks_noalloc(run.plan, b.q_r, b.k_t, col2)
    torch.cuda.synchronize()
    return b.col.cpu().numpy(), col2.cpu().numpy(), run


def test_noalloc_select_equals_workspace_select_twice():
    for wl in (_BIG, _SMALL):
        print(f"no-alloc select: {wl.name}", flush=True)
        want, got, run = _select_both(wl)
        assert want.size == int(run.plan.info.nnz) and np.all(want >= 0)
        assert np.array_equal(got, want), wl.name
    # the same big plan again after the small one (the scratch keeps the
    # small call's means; pooling overwrites every mean the plan reads)
    want, got, _ = _select_both(_BIG)
    assert np.array_equal(got, want)


def test_noalloc_select_refuses_plans_beyond_the_scratch():
    wl = I.WORKLOADS["wan720p_subblock"]          # 194 MB of block means
    plan = S.sva_plan_create_ex(S.desc_for(wl))
    assert plan.info.select_workspace_bytes > 128 << 20
    q_r = torch.empty(plan.tile_shape, dtype=torch.bfloat16, device="cuda")
    k_t = torch.empty(plan.kt_shape, dtype=torch.bfloat16, device="cuda")
    col = torch.empty(int(plan.info.nnz), dtype=torch.int32, device="cuda")
    with pytest.raises(S.SvaError) as e:
        S.sva_select_blocks_noalloc(plan, q_r, k_t, col)
    assert e.value.status == S.SVA_ERR_WORKSPACE
    S.sva_destroy(plan)
