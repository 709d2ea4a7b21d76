"""CPU tests of the C ABI: the library loads, exports every declared
symbol, and its host-side planning (sizes, permutation, block budget, row
offsets, forced blocks, argument errors) equals the oracle's bit for bit.
No compute call runs here (no GPU)."""

import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import block_sparse_attention_qk_amd as S
from block_sparse_attention_qk_amd import inputs as I
import oracle.sva_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "sva.h")).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(sva_\w+)\s*\(", header, re.M))
    assert declared == set(S.EXPORTED)
    L = S.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert S.sva_status_string(S.SVA_ERR_WORKSPACE) == "workspace too small"


def test_debug_library_exports_the_same_symbols():
    """libsva_debug.so (the same sources built with -DSVA_DEBUG, built
    beside libsva.so by the package's build) loads and exports every
    declared symbol; its debug bits match the header's."""
    assert os.path.exists(S.DEBUG_LIB_PATH), "libsva_debug.so is not built"
    L = ctypes.CDLL(S.DEBUG_LIB_PATH)
    for name in S.EXPORTED:
        assert hasattr(L, name), name
    header = open(os.path.join(ROOT, "include", "sva.h")).read()
    bits = dict(re.findall(r"^#define (SVA_DEBUG_\w+) (\d+)u", header, re.M))
    assert bits == {n: str(getattr(S, n)) for n in
                    ("SVA_DEBUG_TOKEN", "SVA_DEBUG_LIST", "SVA_DEBUG_ROW", "SVA_DEBUG_SELF")}


def _geom(wl):
    return O.Geometry(B=wl.B, H=wl.H, T=wl.T, Hh=wl.Hh, W=wl.W, d=wl.d, block=wl.block,
                      sparsity=wl.sparsity, flags=wl.flags, tile=wl.tile, n_extra=wl.n_extra,
                      split=wl.rope_split, scorer=wl.scorer, subblocks=wl.subblocks,
                      budget_multiple=max(1, wl.budget_multiple), theta=wl.theta_resolved,
                      eps=wl.eps_resolved)


CASES = list(I.WORKLOADS.values()) + [
    I.custom("ragged", 2, 3, 5, 13, 17, 128, 128, 0.6, flags=I.KEEP_SAME_FRAME,
             n_extra=128),
    I.custom("ragged64", 1, 2, 3, 7, 11, 64, 64, 0.5, tile=(2, 3, 4), n_extra=64),
    I.custom("subblock8", 1, 2, 5, 16, 24, 128, 64, 0.75, tile=(1, 4, 16),
             scorer=1, budget_multiple=8),
    I.custom("subblock8_wide", 1, 1, 21, 45, 80, 128, 128, 0.8, scorer=1, subblocks=2,
             budget_multiple=8, flags=I.KEEP_SAME_FRAME),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_host_plan_equals_oracle(wl):
    g = _geom(wl)
    info = S.sva_plan_query(S.desc_for(wl))
    assert (info.n_video, info.N, info.n_video_pad, info.Np) == (g.n_video, g.N, g.n_video_pad, g.Np)
    assert (info.nB, info.nB_video, info.k) == (g.nB, g.nB_video, g.k)
    assert bool(info.dense) == g.dense
    perm, row_ptr, forced = S.sva_plan_host_tables(S.desc_for(wl), forced=g.nB <= 1024)
    assert np.array_equal(perm, O.permutation(g))
    lens = O.row_lengths(g)
    assert np.array_equal(np.diff(row_ptr), lens)
    assert info.nnz_per_head == lens.sum() and info.nnz == lens.sum() * wl.B * wl.H
    assert info.max_row_len == lens.max()
    if forced is not None:
        f_o, dense_row = O.forced_blocks(g)
        want = f_o | dense_row[:, None]
        assert np.array_equal(forced.astype(bool), want)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_split_workspace_size(wl):
    """The partials workspace of sva_attention_ws: in a sparse plan every
    row longer than 1.5 times the longest video row (at least 16) is cut
    into ceil(len / that) pieces, each slot holding block x (d + 2) floats
    per (b, h); no row is split in a dense plan."""
    g = _geom(wl)
    info = S.sva_plan_query(S.desc_for(wl))
    lens = O.row_lengths(g)
    slots = 0
    if not g.dense:
        chunk = max(16, int(lens[: g.nB_video].max()))
        slots = sum(-(-int(n) // chunk) for n in lens if 2 * n > 3 * chunk)
    assert info.attention_workspace_bytes == wl.B * wl.H * slots * g.block * (g.d + 2) * 4


def test_workload_block_lists():
    """The executed block pairs of the bench workload (75,600 tokens,
    128-token blocks, sparsity 0.75): 591 rows of 148 blocks per head."""
    info = S.sva_plan_query(S.desc_for(I.WORKLOADS["wan720p_sp75"]))
    assert (info.nB, info.k, info.max_row_len, info.nnz_per_head) == (591, 148, 148, 591 * 148)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), S.SVA_ERR_UNSUPPORTED),
    (dict(block=32), S.SVA_ERR_UNSUPPORTED),
    (dict(B=0), S.SVA_ERR_INVALID_ARG),
    (dict(T=-1), S.SVA_ERR_INVALID_ARG),
    (dict(sparsity=1.0), S.SVA_ERR_INVALID_ARG),
    (dict(sparsity=-0.1), S.SVA_ERR_INVALID_ARG),
    (dict(sparsity=float("nan")), S.SVA_ERR_INVALID_ARG),
    (dict(flags=8), S.SVA_ERR_INVALID_ARG),
    (dict(n_extra=100), S.SVA_ERR_INVALID_ARG),
    (dict(tile=(0, 4, 4)), S.SVA_ERR_INVALID_ARG),
    (dict(rope_split=(43, 43, 42)), S.SVA_ERR_INVALID_ARG),
    (dict(rope_split=(64, 64, 64)), S.SVA_ERR_INVALID_ARG),
    (dict(eps=-1.0), S.SVA_ERR_INVALID_ARG),
    (dict(rope_theta=0.5), S.SVA_ERR_INVALID_ARG),
    (dict(scorer=2), S.SVA_ERR_INVALID_ARG),
    (dict(scorer=1, subblocks=3), S.SVA_ERR_UNSUPPORTED),
    (dict(scorer=1, subblocks=8), S.SVA_ERR_UNSUPPORTED),
    (dict(scorer=0, subblocks=4), S.SVA_ERR_INVALID_ARG),
    (dict(budget_multiple=-1), S.SVA_ERR_INVALID_ARG),
])
def test_argument_errors(kw, status):
    base = dict(B=1, H=2, T=4, Hh=8, W=8, d=128, block=128, sparsity=0.5)
    extra = {k: kw.pop(k) for k in list(kw) if k in ("tile", "n_extra", "rope_split", "eps",
                                                     "rope_theta", "flags", "scorer",
                                                     "subblocks", "budget_multiple")}
    base.update(kw)
    desc = S.sva_plan_desc_init(base["B"], base["H"], base["T"], base["Hh"], base["W"],
                                base["d"], base["block"], base["sparsity"],
                                extra.pop("flags", 0), **extra)
    with pytest.raises(S.SvaError) as e:
        S.sva_plan_query(desc)
    assert e.value.status == status
    assert S.sva_last_error()


def test_null_arguments_rejected_on_host():
    L = S.lib()
    assert L.sva_plan_query(None, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_plan_get_info(None, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_qk_norm_rope(None, None, None, None, None, None, None, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_reorder(None, None, None, 0, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_select_blocks(None, None, None, None, 0, None, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_attention(None, None, None, None, None, None, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_qk_norm_rope_tiled(None, None, None, None, None, None, None, None, 0,
                                    None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_block_means(None, None, None, None, None, None) == S.SVA_ERR_INVALID_ARG
    assert L.sva_destroy(None) == S.SVA_OK
    assert L.sva_plan_create_ex(None, None) == S.SVA_ERR_INVALID_ARG


def test_partial_rope_split_accepted():
    # 96 of 128 channels rotated (the packed H3 shape on the benchmark page)
    desc = S.sva_plan_desc_init(1, 2, 4, 8, 8, 128, 128, 0.5, rope_split=(32, 32, 32))
    info = S.sva_plan_query(desc)
    assert list(info.rope_split) == [32, 32, 32]


def test_c_program_host_calls(tmp_path):
    """The header compiles as C99 and the library links from C: a plain C
    program (tests/c_abi_host.c) runs the host-only calls and checks the
    tile order, budget, row offsets and error codes written out by hand."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    S.lib()                                   # the library must be built
    libdir = os.path.dirname(S.LIB_PATH)
    exe = str(tmp_path / "c_abi_host")
    subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_host.c"),
                    "-L", libdir, "-lsva", "-Wl,-rpath," + libdir, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: with the library absent the binding raises before any
    call runs."""
    monkeypatch.setattr(S, "LIB_PATH", str(tmp_path / "libsva.so"))
    monkeypatch.setattr(S, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        S.lib()
    with pytest.raises(RuntimeError):
        S.sva_plan_query(S.sva_plan_desc())


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus N > 1 exits with status 2 and a
    message, before it touches a device."""
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
