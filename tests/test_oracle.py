"""Pins of the CPU oracle against things other than itself: hand-worked
fixtures, closed forms, invariants, library routines and brute force.

Every check here runs on the CPU in a few seconds.  ``test_pins_catch_*``
plants plausible mistakes in the oracle (on the CPU, through monkeypatch) and
asserts that a pin fails, so a wrong oracle cannot pass silently.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle.sva_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- bf16 rounding

def check_bf16_golden():
    # spacing of bf16 at 1.0 is 2**-7
    assert O.to_bf16(1.0) == 1.0
    assert O.to_bf16(1.0 + 2.0 ** -8) == 1.0                       # tie -> even
    assert O.to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6        # tie -> even
    assert O.to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert O.to_bf16(-3.0) == -3.0
    assert O.to_bf16(2.0 ** -130) == 2.0 ** -130                   # subnormal, exact
    assert O.to_bf16(2.0 ** -134) == 0.0                           # tie -> even (0)
    assert O.to_bf16(3 * 2.0 ** -134) == 2.0 ** -132               # tie -> even


def test_bf16_golden_values():
    check_bf16_golden()


def test_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.to_bf16(x.astype(np.float64)), ref)
    bits = O.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(O.bf16_bits_to_f64(bits), ref)


# ---------------------------------------------------------------- RMSNorm

def check_rmsnorm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)) * 3.0
    eps = 1e-6
    y = O.rms_norm(x, np.ones(128), eps)
    ms = np.mean(x * x, axis=1)
    # closed form: mean(y^2) = ms / (ms + eps)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)
    # direction preserved, positive scale
    cos = np.sum(x * y, axis=1) / np.linalg.norm(x, axis=1) / np.linalg.norm(y, axis=1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-12)
    # scale invariance f(a x) = f(x) (eps negligible)
    np.testing.assert_allclose(O.rms_norm(7.5 * x, np.ones(128), 0.0),
                               O.rms_norm(x, np.ones(128), 0.0), rtol=1e-13)
    # worked example: (3, 4) -> ms = 12.5 -> (3, 4)/sqrt(12.5)
    np.testing.assert_allclose(O.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0),
                               [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    # the weight multiplies each channel
    w = rng.uniform(0.5, 2.0, 128)
    np.testing.assert_allclose(O.rms_norm(x, w, eps), y * w, rtol=1e-14)
    # a large epsilon enters the same closed form
    big = 0.5
    np.testing.assert_allclose(np.mean(O.rms_norm(x, np.ones(128), big) ** 2, axis=1),
                               ms / (ms + big), rtol=1e-12)


def test_rmsnorm_closed_forms():
    check_rmsnorm()


# ---------------------------------------------------------------- RoPE

def _geom(**kw):
    base = dict(B=1, H=1, T=4, Hh=6, W=8, d=64, block=64, sparsity=0.5)
    base.update(kw)
    return O.Geometry(**base)


def check_rope_library():
    """Each axis section equals textbook 1D RoPE as implemented by the
    transformers library (LlamaRotaryEmbedding frequencies, rotate-half
    pairing), once the interleaved pairs (2i, 2i+1) are gathered into the
    half layout (evens first, then odds)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import (LlamaRotaryEmbedding,
                                                          apply_rotary_pos_emb)
    for theta in (10000.0, 500.0):
        _rope_library_case(_geom(T=5, Hh=7, W=9, d=64, split=(16, 24, 24), theta=theta),
                           LlamaConfig, LlamaRotaryEmbedding, apply_rotary_pos_emb)


def _rope_library_case(g, LlamaConfig, LlamaRotaryEmbedding, apply_rotary_pos_emb):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((g.N, g.d))
    y = O.rope_3d(x, g)
    t, h, w = O.token_positions(g)
    off = 0
    for pos, width in zip((t, h, w), g.split):
        cfg = LlamaConfig(hidden_size=width, num_attention_heads=1, head_dim=width,
                          rope_parameters={"rope_type": "default", "rope_theta": g.theta},
                          max_position_embeddings=64)
        emb = LlamaRotaryEmbedding(cfg)
        sec = torch.from_numpy(x[:, off: off + width]).float()
        half = torch.cat([sec[:, 0::2], sec[:, 1::2]], dim=1)[None, None]
        cos, sin = emb(half, torch.from_numpy(pos)[None].long())
        ref, _ = apply_rotary_pos_emb(half, half, cos, sin)
        ref = ref[0, 0].double().numpy()
        got = y[:, off: off + width]
        got_half = np.concatenate([got[:, 0::2], got[:, 1::2]], axis=1)
        np.testing.assert_allclose(got_half, ref, atol=2e-5, rtol=0)
        off += width


def test_rope_matches_library_per_section():
    check_rope_library()


def check_rope_invariants():
    g = _geom(T=4, Hh=6, W=8, d=128, split=(44, 42, 42))
    rng = np.random.default_rng(4)
    x = rng.standard_normal((g.N, g.d))
    y = O.rope_3d(x, g)
    # every rotated pair keeps its norm
    np.testing.assert_allclose(x[:, 0::2] ** 2 + x[:, 1::2] ** 2,
                               y[:, 0::2] ** 2 + y[:, 1::2] ** 2, rtol=1e-12)
    # position (0,0,0) is the identity
    np.testing.assert_array_equal(y[0], x[0])
    # relative position: q·k depends only on the coordinate difference.
    # Put one q vector and one k vector at pairs of tokens shifted by one
    # step along each axis and compare the dot products.
    q = rng.standard_normal(g.d)
    k = rng.standard_normal(g.d)

    def dot_at(n1, n2):
        z = np.zeros((g.N, g.d))
        z[n1] = q
        z[n2] = k
        r = O.rope_3d(z, g)
        return float(r[n1] @ r[n2])

    def n_of(t, h, w):
        return (t * g.Hh + h) * g.W + w

    a = dot_at(n_of(0, 1, 2), n_of(2, 4, 3))
    for dt, dh, dw in ((1, 0, 0), (0, 1, 0), (0, 0, 3), (1, 1, 1)):
        b = dot_at(n_of(0 + dt, 1 + dh, 2 + dw), n_of(2 + dt, 4 + dh, 3 + dw))
        assert abs(a - b) < 1e-10 * max(1.0, abs(a))
    # the rotation really depends on the difference (guards a no-op RoPE)
    c = dot_at(n_of(0, 1, 2), n_of(3, 4, 3))
    assert abs(a - c) > 1e-3


def test_rope_invariants():
    check_rope_invariants()


def check_rope_coordinates():
    """Each section turns by its own axis coordinate of the raster token
    n = (t·Hh + h)·W + w: on a 2×3×4 grid with one pair per section (angle =
    coordinate, frequency theta^0), the pairs (1, 0) of token 23 = (1, 2, 3)
    come out as (cos c, sin c) for c = 1, 2, 3, and those of token 6 =
    (0, 1, 2) for c = 0, 1, 2."""
    g = _geom(T=2, Hh=3, W=4, d=6, split=(2, 2, 2), tile=(1, 1, 4))
    x = np.tile([1.0, 0.0], (g.N, 3))
    y = O.rope_3d(x, g)
    for n, coords in ((23, (1, 2, 3)), (6, (0, 1, 2))):
        want = np.concatenate([[math.cos(c), math.sin(c)] for c in coords])
        np.testing.assert_allclose(y[n], want, rtol=0, atol=1e-15)


def test_rope_coordinates():
    check_rope_coordinates()


def test_rope_leaves_extra_tokens_and_tail_dims():
    g = _geom(T=2, Hh=4, W=4, d=64, split=(16, 16, 16), n_extra=64)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((g.N, g.d))
    y = O.rope_3d(x, g)
    np.testing.assert_array_equal(y[g.n_video:], x[g.n_video:])   # extra tokens
    np.testing.assert_array_equal(y[:, 48:], x[:, 48:])           # past the sections


def test_prologue_rounding_points():
    """Round after the norm, then after the rotation: at position 0 the
    rotation is the identity, so the output is the once-rounded norm."""
    g = _geom(T=2, Hh=2, W=2, d=64)
    rng = np.random.default_rng(6)
    x = O.to_bf16(rng.standard_normal((g.N, g.d)))
    y = O.qk_norm_rope(x, np.ones(g.d), g)
    assert np.array_equal(y, O.to_bf16(y))                         # bf16 values
    np.testing.assert_array_equal(y[0], O.to_bf16(O.rms_norm(x[0], np.ones(g.d), g.eps)))
    # elsewhere the output lies within one bf16 rounding of the exact value
    exact = O.rope_3d(O.to_bf16(O.rms_norm(x, np.ones(g.d), g.eps)), g)
    assert np.all(np.abs(y - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)


def check_prologue_rounding_golden():
    """The hand-worked case of tests/golden/prologue_rounding_1x1x2.txt: the
    norm is rounded to bf16 before the rotation and the result after it."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "prologue_rounding_1x1x2.txt"))
            if ln.strip() and not ln.startswith("#")]
    g = O.Geometry(B=1, H=1, T=1, Hh=1, W=2, d=2, block=64, sparsity=0.0, split=(0, 0, 2),
                   eps=1e-6, tile=(1, 1, 2))
    x = np.array([[1.0, 0.0], [1.0, 0.0]])
    w = np.array([(1.0 + 2.0 ** -8 + 2.0 ** -12) / math.sqrt(2.0), 1.0])
    y = O.qk_norm_rope(x, w, g)
    for r in rows:
        n = int(r[0])
        np.testing.assert_array_equal(y[n], [float(r[1]), float(r[2])])


def test_prologue_rounding_golden():
    check_prologue_rounding_golden()


# ---------------------------------------------------------------- permutation

def check_perm_golden():
    g = O.Geometry(B=1, H=1, T=3, Hh=3, W=3, d=64, block=8, sparsity=0.5, tile=(2, 2, 2))
    perm = O.permutation(g)
    for t, h, w, p in (map(int, r) for r in _load("perm_3x3x3_tile2.txt")):
        assert perm[(t * 3 + h) * 3 + w] == p, (t, h, w, p)
    valid, tmin, tmax, extra = O.block_meta(g)
    forced, _ = O.forced_blocks(O.Geometry(B=1, H=1, T=3, Hh=3, W=3, d=64, block=8,
                                           sparsity=0.5, tile=(2, 2, 2),
                                           flags=O.SVA_KEEP_SAME_FRAME))
    for blk, nv, t0, t1, cols in _load("blocks_3x3x3_tile2.txt"):
        blk = int(blk)
        assert (valid[blk], tmin[blk], tmax[blk]) == (int(nv), int(t0), int(t1))
        assert sorted(np.nonzero(forced[blk])[0].tolist()) == [int(c) for c in cols.split(",")]


def test_permutation_golden_fixture():
    check_perm_golden()


def test_permutation_tiles_equal_blocks_tiny():
    # tiny workload: 4×16×16 grid, tile 4×4×4 = 64 tokens = one block
    g = O.Geometry(B=1, H=2, T=4, Hh=16, W=16, d=64, block=64, sparsity=0.5, tile=(4, 4, 4))
    perm = O.permutation(g)
    t, h, w = O.token_positions(g)
    tile_id = (t // 4) * 16 + (h // 4) * 4 + (w // 4)
    assert np.array_equal(perm // 64, tile_id)
    # inside a tile: (t, h, w) order
    assert np.array_equal(perm % 64, (t % 4) * 16 + (h % 4) * 4 + (w % 4))


@pytest.mark.parametrize("shape,tile,block,n_extra", [
    ((5, 13, 17), (2, 8, 8), 128, 0),
    ((21, 30, 52), (3, 4, 8), 64, 0),
    ((3, 7, 11), (2, 3, 4), 64, 128),
])
def test_permutation_bijection_and_inverse(shape, tile, block, n_extra):
    g = O.Geometry(B=2, H=3, T=shape[0], Hh=shape[1], W=shape[2], d=64, block=block,
                   sparsity=0.5, tile=tile, n_extra=n_extra)
    perm = O.permutation(g)
    assert len(set(perm.tolist())) == g.N
    assert perm[: g.n_video].max() == g.n_video - 1           # video part is dense
    assert np.all(perm[g.n_video:] >= g.n_video_pad)          # extra after the pad
    rng = np.random.default_rng(7)
    x = rng.standard_normal((g.B, g.N, g.H, g.d))
    xr = O.reorder_forward(x, g, perm)
    assert np.all(xr[:, :, g.n_video: g.n_video_pad] == 0)    # tail padding
    np.testing.assert_array_equal(O.reorder_inverse(xr, g, perm), x)
    # every tile is contiguous in the new order
    t, h, w = O.token_positions(g)
    tt, th, tw = tile
    key = ((t // tt) * (-(-g.Hh // th)) + h // th) * (-(-g.W // tw)) + w // tw
    order = np.argsort(perm[: g.n_video])
    assert np.all(np.diff(key[order]) >= 0)


# ---------------------------------------------------------------- pooling

def test_pooling_constant_block_and_valid_count():
    g = O.Geometry(B=1, H=1, T=3, Hh=3, W=3, d=64, block=8, sparsity=0.5, tile=(2, 2, 2))
    xr = np.zeros((g.Np, g.d))
    xr[0:8] = 1.5                      # constant block -> mean = value
    xr[24:27] = np.arange(3)[:, None]  # last block: 3 valid rows 0,1,2 -> mean 1
    m = O.pool_means(xr, g)
    np.testing.assert_array_equal(m[0], 1.5)
    np.testing.assert_array_equal(m[3], 1.0)


# ---------------------------------------------------------------- selection

def test_budget_golden():
    for nB, sp, k in _load("budget_k.txt"):
        assert O.budget(int(nB), float(sp)) == int(k), (nB, sp, k)
    assert O.budget(77, 0.6, O.SVA_DENSE) == 77


def _sel_setup(seed=8, flags=0, sparsity=0.75, n_extra=0, Hh=8, W=16):
    g = O.Geometry(B=1, H=1, T=4, Hh=Hh, W=W, d=64, block=64, sparsity=sparsity,
                   tile=(2, 4, 8), flags=flags, n_extra=n_extra)
    rng = np.random.default_rng(seed)
    qbar = rng.standard_normal((g.nB, g.d))
    kbar = rng.standard_normal((g.nB, g.d))
    return g, qbar, kbar


def check_selection_bruteforce(flags=O.SVA_KEEP_SAME_FRAME, n_extra=128, sparsity=0.3):
    # 32 video blocks, 16 per frame pair: with same-frame forcing 16 + 2
    # extra blocks are forced and sparsity 0.3 asks for 24, so every video
    # row ranks the remaining blocks (the check is not vacuous)
    g, qbar, kbar = _sel_setup(flags=flags, n_extra=n_extra, sparsity=sparsity, Hh=16, W=32)
    kept, scores, _, _ = O.select_blocks(qbar, kbar, g)
    forced, dense_row = O.forced_blocks(g)
    ranked_rows = 0
    for qb in range(g.nB):
        if dense_row[qb]:
            assert kept[qb].all()
            continue
        s = [sum(qbar[qb, i] * kbar[kb, i] for i in range(g.d)) for kb in range(g.nB)]
        f = [kb for kb in range(g.nB) if forced[qb, kb]]
        rest = sorted((kb for kb in range(g.nB) if not forced[qb, kb]),
                      key=lambda kb: (-s[kb], kb))
        need = max(g.k, len(f)) - len(f)
        ranked_rows += need > 0
        want = set(f) | set(rest[:need])
        assert set(np.nonzero(kept[qb])[0].tolist()) == want, qb
    assert ranked_rows >= g.nB_video


def test_selection_bruteforce():
    check_selection_bruteforce()
    check_selection_bruteforce(flags=0, n_extra=0, sparsity=0.75)


def test_selection_properties():
    g, qbar, kbar = _sel_setup(flags=O.SVA_KEEP_SAME_FRAME, n_extra=64)
    kept, _, _, _ = O.select_blocks(qbar, kbar, g)
    forced, dense_row = O.forced_blocks(g)
    lens = O.row_lengths(g)
    assert np.array_equal(kept.sum(axis=1), lens)
    assert np.all(kept[forced])                                  # F ⊆ kept
    assert np.all(kept[dense_row])                               # dense rows
    assert np.all(kept[g.nB_video:])                             # extra-token rows keep all
    assert dense_row[g.nB_video:].all() and not dense_row[: g.nB_video].any()
    assert np.all(kept[:, g.nB_video:])                          # dense columns
    # sparsity 0 keeps everything
    g0 = O.Geometry(B=1, H=1, T=4, Hh=8, W=16, d=64, block=64, sparsity=0.0, tile=(2, 4, 8))
    assert O.select_blocks(qbar[: g0.nB], kbar[: g0.nB], g0)[0].all()
    # nesting: a smaller sparsity keeps a superset
    prev = None
    for sp in (0.9, 0.75, 0.5, 0.25):
        gs = O.Geometry(B=1, H=1, T=4, Hh=8, W=16, d=64, block=64, sparsity=sp,
                        tile=(2, 4, 8))
        ks = O.select_blocks(qbar[: gs.nB], kbar[: gs.nB], gs)[0]
        if prev is not None:
            assert np.all(ks[prev])
        prev = ks


def test_budget_multiple():
    # hand-worked: ceil((1 - s)·nB) rounded up to a multiple of 8, clamped to nB
    assert O.budget(591, 0.75, 0, 8) == 152      # 148 -> 152
    assert O.budget(591, 0.80, 0, 8) == 120      # ceil(118.2) = 119 -> 120
    assert O.budget(16, 0.5, 0, 8) == 8          # 8 stays 8
    assert O.budget(10, 0.9, 0, 8) == 8          # 1 -> 8
    assert O.budget(5, 0.5, 0, 8) == 5           # 3 -> 8 -> clamped to 5
    assert O.budget(591, 0.75, 0, 1) == O.budget(591, 0.75)
    assert O.budget(40, 0.5, O.SVA_DENSE, 8) == 40


# ---------------------------------------------------------------- SubBlock scorer

def _sub_geom(n=4, n_extra=64, W=10, block=64):
    # 2×6×10 = 120 video tokens: block 1 is ragged (56 valid of 64), so its
    # sub-blocks hold 16, 16, 16 and 8 tokens; one extra-token block follows
    return O.Geometry(B=1, H=1, T=2, Hh=6, W=W, d=32, block=block, sparsity=0.5,
                      tile=(1, 6, 10), n_extra=n_extra, scorer=O.SCORER_SUBBLOCK, subblocks=n)


def check_subblock_exact():
    """Rows constant within each sub-block: the SubBlock estimate is the
    exact unnormalised softmax mass of each block pair (brute force)."""
    g = _sub_geom()
    valid, _, _, _ = O.block_meta(g)
    cnt = O.subblock_counts(g, valid)
    assert cnt.tolist()[:2] == [[16, 16, 16, 16], [16, 16, 16, 8]]
    rng = np.random.default_rng(21)
    n, sb = g.subblocks, g.block // g.subblocks
    def field():
        x = np.zeros((g.Np, g.d))
        for kb in range(g.nB):
            for a in range(n):
                c = cnt[kb, a]
                if c:
                    x[kb * g.block + a * sb: kb * g.block + a * sb + c] = rng.standard_normal(g.d)
        return x
    qr, kr = field(), field()
    sc = O.subblock_scores(O.subblock_means(qr, g, valid), O.subblock_means(kr, g, valid), g, valid)
    for qb in range(g.nB):
        for kb in range(g.nB):
            mass = 0.0
            for p in range(qb * g.block, qb * g.block + valid[qb]):
                for j in range(kb * g.block, kb * g.block + valid[kb]):
                    mass += math.exp(sum(qr[p, i] * kr[j, i] for i in range(g.d)) / math.sqrt(g.d))
            assert abs(sc[qb, kb] - math.log(mass)) <= 1e-12 * max(1.0, abs(math.log(mass))), (qb, kb)


def test_subblock_scores_exact_on_constant_subblocks():
    check_subblock_exact()


def test_subblock_one_subblock_ranks_like_mean():
    # every block full and one sub-block per block: the estimate is
    # log(b²) + q̄·k̄/sqrt(d), a monotone map of the mean scorer's q̄·k̄
    g1 = O.Geometry(B=1, H=1, T=4, Hh=8, W=16, d=64, block=64, sparsity=0.75,
                    tile=(2, 4, 8), scorer=O.SCORER_SUBBLOCK, subblocks=1)
    gm = O.Geometry(B=1, H=1, T=4, Hh=8, W=16, d=64, block=64, sparsity=0.75, tile=(2, 4, 8))
    rng = np.random.default_rng(22)
    qr = rng.standard_normal((g1.Np, g1.d))
    kr = rng.standard_normal((g1.Np, g1.d))
    sc = O.subblock_scores(O.subblock_means(qr, g1), O.subblock_means(kr, g1), g1)
    kept1 = O.select_from_scores(sc, g1)[0]
    keptm = O.select_blocks(O.pool_means(qr, gm), O.pool_means(kr, gm), gm)[0]
    assert np.array_equal(kept1, keptm)
    np.testing.assert_allclose(
        sc, np.log(64.0 * 64.0) + O.pool_means(qr, gm) @ O.pool_means(kr, gm).T / 8.0, rtol=1e-13)


def test_subblock_scores_stay_finite_for_large_logits():
    g = _sub_geom()
    rng = np.random.default_rng(23)
    qr = rng.standard_normal((g.Np, g.d)) * 300.0
    kr = rng.standard_normal((g.Np, g.d)) * 300.0
    sc = O.subblock_scores(O.subblock_means(qr, g), O.subblock_means(kr, g), g)
    assert np.all(np.isfinite(sc))


def test_selection_ties_take_lowest_index():
    g, _, _ = _sel_setup()
    z = np.zeros((g.nB, g.d))
    kept, _, _, _ = O.select_blocks(z, z, g)
    for qb in range(g.nB):
        assert np.nonzero(kept[qb])[0].tolist() == list(range(g.k))
    # a block scale that flips no order keeps the same choice (scale-free score)
    _, qbar, kbar = _sel_setup(seed=9)
    a = O.select_blocks(qbar, kbar, g)[0]
    b = O.select_blocks(3.0 * qbar, kbar, g)[0]
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- attention

def _attn_case(seed, flags=0, sparsity=0.5, n_extra=0, T=3, Hh=5, W=7, d=64, block=64):
    g = O.Geometry(B=1, H=1, T=T, Hh=Hh, W=W, d=d, block=block, sparsity=sparsity,
                   tile=(2, 4, 4), flags=flags, n_extra=n_extra)
    rng = np.random.default_rng(seed)
    qr = np.zeros((g.Np, d))
    kr = np.zeros((g.Np, d))
    vr = np.zeros((g.Np, d))
    valid, _, _, _ = O.block_meta(g)
    for blk in range(g.nB):
        n = valid[blk]
        sl = slice(blk * block, blk * block + n)
        qr[sl] = rng.standard_normal((n, d))
        kr[sl] = rng.standard_normal((n, d))
        vr[sl] = rng.standard_normal((n, d))
    return g, qr, kr, vr, valid


def _valid_rows(g, valid):
    return np.concatenate([np.arange(b * g.block, b * g.block + valid[b]) for b in range(g.nB)])


def check_dense_attention_sdpa():
    g, qr, kr, vr, valid = _attn_case(10, sparsity=0.0, n_extra=64)
    kept = np.ones((g.nB, g.nB), dtype=bool)
    out = O.block_attention(qr, kr, vr, kept, g)
    rows = _valid_rows(g, valid)
    t = lambda a: torch.from_numpy(a[rows])[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qr), t(kr), t(vr))[0, 0].numpy()
    np.testing.assert_allclose(out[rows], ref, rtol=1e-12, atol=1e-13)
    pad = np.setdiff1d(np.arange(g.Np), rows)
    assert np.all(out[pad] == 0)


def test_dense_attention_equals_library_sdpa():
    check_dense_attention_sdpa()


def check_sparse_attention_masked_sdpa():
    g, qr, kr, vr, valid = _attn_case(11, sparsity=0.6, flags=O.SVA_KEEP_SAME_FRAME,
                                      T=4, Hh=8, W=9)
    assert g.nB == 5
    rng = np.random.default_rng(12)
    kept = rng.random((g.nB, g.nB)) < 0.5
    kept[np.arange(g.nB), rng.integers(0, g.nB, g.nB)] = True    # ≥1 block per row
    kept[0] = [True, False, False, True, False]
    kept[4] = [False, False, False, False, True]                 # padded block only
    out = O.block_attention(qr, kr, vr, kept, g)
    rows = _valid_rows(g, valid)
    blk = rows // g.block
    mask = np.where(kept[blk][:, blk], 0.0, -np.inf)
    t = lambda a: torch.from_numpy(a[rows])[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(qr), t(kr), t(vr), attn_mask=torch.from_numpy(mask)[None, None])[0, 0].numpy()
    np.testing.assert_allclose(out[rows], ref, rtol=1e-12, atol=1e-13)


def test_sparse_attention_equals_masked_library_sdpa():
    check_sparse_attention_masked_sdpa()


def _online_rows(qr, kr, vr, kept, g, valid, rows, rot, lead_empty, c):
    """The softmax the attention kernel runs, in fp64: stages of 32 keys in a
    rotated walk of the row's kept blocks, a running max m (log2 units)
    started at the first stage's max, probabilities 2^(s·c − m) against a
    stale m, and the lazy rescale decided after the fact: only when one of
    the stage's two 16-key lane groups sums to 2^8 or more is the stage's max
    taken, m raised if that max exceeds it by more than 8, and the stage
    recomputed.  Returns the outputs and the largest accepted probability."""
    out = np.zeros((len(rows), g.d))
    pmax = 0.0
    rescales = 0
    # lane group of each key of a 32-key stage (the accumulator layout)
    group = np.array([(k % 8) // 4 for k in range(32)])
    for i, r in enumerate(rows):
        qb = r // g.block
        blocks = list(np.nonzero(kept[qb])[0])
        blocks = blocks[rot % len(blocks):] + blocks[:rot % len(blocks)]
        stages = []
        if lead_empty:
            stages.append(np.full(32, -np.inf))                   # an empty list entry
        vstages = [np.zeros((32, g.d))] if lead_empty else []
        for kb in blocks:
            for st in range(g.block // 32):
                k0 = kb * g.block + st * 32
                n = min(max(valid[kb] - st * 32, 0), 32)
                s = np.full(32, -np.inf)
                s[:n] = kr[k0:k0 + n] @ qr[r] * c
                stages.append(s)
                vv = np.zeros((32, g.d))
                vv[:n] = vr[k0:k0 + n]
                vstages.append(vv)
        m, l, o = -1e30, 0.0, np.zeros(g.d)
        if stages[0].max() > m + 8:
            m = stages[0].max()
        for s, vv in zip(stages, vstages):
            # after an empty first entry m is still -1e30: the first stage
            # with keys overflows to inf, which takes the slow path below
            with np.errstate(over="ignore"):
                p = np.exp2(s - m)
            if max(p[group == 0].sum(), p[group == 1].sum()) >= 256.0:
                mx = s.max()
                if mx > m + 8:
                    al = np.exp2(m - mx)
                    o *= al
                    l *= al
                    m = mx
                    rescales += 1
                p = np.exp2(s - m)
            pmax = max(pmax, p.max())
            l += p.sum()
            o += p @ vv
        out[i] = o / l
    return out, pmax, rescales


def test_online_softmax_with_lazy_rescale_equals_two_pass():
    """Reading R22 and the after-the-fact rescale: the kernel's online
    softmax (stale max within 8 log2 units, rescale decided from the lane
    groups' probability sums) equals the two-pass softmax up to fp64
    rounding, with every accepted probability at most 2^8, also when logits
    grow by tens of log2 units along the walk and the walk begins with an
    empty entry."""
    g, qr, kr, vr, valid = _attn_case(31, sparsity=0.5, T=4, Hh=8, W=9)
    qr = qr * 6.0                                   # logits ~ N(0, 36): large growth
    rng = np.random.default_rng(32)
    kept = rng.random((g.nB, g.nB)) < 0.6
    kept[np.arange(g.nB), np.arange(g.nB)] = True
    ref = O.block_attention(qr, kr, vr, kept, g)
    rows = _valid_rows(g, valid)[::7]
    c = 1.0 / math.sqrt(g.d) / math.log(2.0)        # natural logits -> log2 units
    total = 0
    for rot, lead in ((0, False), (1, True), (3, False)):
        out, pmax, rescales = _online_rows(qr, kr, vr, kept, g, valid, rows, rot, lead, c)
        np.testing.assert_allclose(out, ref[rows], rtol=1e-11, atol=1e-12)
        assert pmax <= 256.0 * (1 + 1e-12)
        total += rescales
    assert total > len(rows)                        # the rescale path really ran


def test_attention_bruteforce_loops():
    g, qr, kr, vr, valid = _attn_case(13, sparsity=0.5, T=2, Hh=3, W=3, d=8, block=8)
    assert valid.tolist() == [8, 8, 2]
    kept = np.zeros((g.nB, g.nB), dtype=bool)
    kept[0, [0, 2]] = True
    kept[1, [1]] = True
    kept[2, [0, 1, 2]] = True
    out = O.block_attention(qr, kr, vr, kept, g)
    for p in range(g.Np):
        qb = p // g.block
        if p - qb * g.block >= valid[qb]:
            assert np.all(out[p] == 0)
            continue
        keys = [j for j in range(g.Np) if kept[qb, j // g.block]
                and j - (j // g.block) * g.block < valid[j // g.block]]
        logits = [sum(qr[p, i] * kr[j, i] for i in range(g.d)) / math.sqrt(g.d) for j in keys]
        mx = max(logits)
        e = [math.exp(x - mx) for x in logits]
        for c in range(g.d):
            want = sum(e[i] * vr[keys[i], c] for i in range(len(keys))) / sum(e)
            assert abs(out[p, c] - want) < 1e-12


def check_compensation_exact():
    """Dropped blocks whose keys and values are constant: the compensated
    sparse attention is exactly dense attention (brute force)."""
    g = O.Geometry(B=1, H=1, T=2, Hh=6, W=10, d=32, block=64, sparsity=0.5, tile=(1, 6, 10),
                   n_extra=64, flags=O.SVA_COMPENSATE)
    valid, _, _, _ = O.block_meta(g)
    rng = np.random.default_rng(31)
    qr = rng.standard_normal((g.Np, g.d))
    kr = rng.standard_normal((g.Np, g.d))
    vr = rng.standard_normal((g.Np, g.d))
    kept = np.ones((g.nB, g.nB), bool)
    kept[0, 1] = False                  # query block 0 drops block 1 (ragged, 56 valid)
    kept[1, 0] = False                  # query block 1 drops block 0
    for kb in (0, 1):                   # make the dropped blocks constant
        kr[kb * g.block: kb * g.block + valid[kb]] = rng.standard_normal(g.d)
        vr[kb * g.block: kb * g.block + valid[kb]] = rng.standard_normal(g.d)
    for x in (qr, kr, vr):              # padding rows are zero, as after the reorder
        x[g.block + valid[1]: 2 * g.block] = 0.0
    got = O.block_attention(qr, kr, vr, kept, g)
    want = O.block_attention(qr, kr, vr, np.ones_like(kept), g)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # and it differs from the uncompensated sparse attention
    g0 = O.Geometry(B=1, H=1, T=2, Hh=6, W=10, d=32, block=64, sparsity=0.5, tile=(1, 6, 10),
                    n_extra=64)
    assert np.abs(O.block_attention(qr, kr, vr, kept, g0) - want).max() > 1e-3


def test_compensation_exact_on_constant_dropped_blocks():
    check_compensation_exact()


def test_compensation_brute_force():
    """Brute force with loops: every dropped block contributes |B| copies of
    (mean key, mean value) to the softmax of each query row."""
    g = O.Geometry(B=1, H=1, T=2, Hh=4, W=8, d=16, block=16, sparsity=0.5, tile=(1, 4, 4),
                   flags=O.SVA_COMPENSATE)
    valid, _, _, _ = O.block_meta(g)
    rng = np.random.default_rng(32)
    qr, kr, vr = (rng.standard_normal((g.Np, g.d)) for _ in range(3))
    kept = rng.random((g.nB, g.nB)) < 0.5
    kept[np.arange(g.nB), np.arange(g.nB)] = True
    got = O.block_attention(qr, kr, vr, kept, g)
    for qb in range(g.nB):
        for p in range(qb * g.block, qb * g.block + valid[qb]):
            num = np.zeros(g.d)
            den = 0.0
            for kb in range(g.nB):
                rows = range(kb * g.block, kb * g.block + valid[kb])
                if kept[qb, kb]:
                    for j in rows:
                        w = math.exp(sum(qr[p, i] * kr[j, i] for i in range(g.d)) / math.sqrt(g.d))
                        num += w * vr[j]
                        den += w
                else:
                    km = sum(kr[j] for j in rows) / valid[kb]
                    vm = sum(vr[j] for j in rows) / valid[kb]
                    w = valid[kb] * math.exp(sum(qr[p, i] * km[i] for i in range(g.d)) / math.sqrt(g.d))
                    num += w * vm
                    den += w
            np.testing.assert_allclose(got[p], num / den, rtol=1e-10, atol=1e-12)


def check_attention_row_sums(flags=0, sparsity=0.5):
    """Row sums of the softmax weights equal 1, read off block_attention
    itself: with V set to the identity (d = Np, one value channel per key
    position) the output row of query p is its weight vector over the key
    positions.  Every valid row's weights are non-negative and sum to 1;
    without compensation they vanish outside the row's kept blocks and on
    padding keys; with compensation a dropped block's weight is spread
    evenly (its mean value) over its valid keys.  With V = 1 on the valid
    keys the output is 1 on every valid row."""
    g = O.Geometry(B=1, H=1, T=2, Hh=4, W=6, d=64, block=16, sparsity=sparsity, tile=(1, 4, 4),
                   flags=flags, n_extra=16)
    assert g.Np == g.d
    valid, _, _, _ = O.block_meta(g)
    rng = np.random.default_rng(14 + flags)
    qr, kr = (rng.standard_normal((g.Np, g.d)) * 2.0 for _ in range(2))
    rows = _valid_rows(g, valid)
    pad = np.setdiff1d(np.arange(g.Np), rows)
    qr[pad] = kr[pad] = 0.0
    kept = rng.random((g.nB, g.nB)) < 0.4
    kept[np.arange(g.nB), np.arange(g.nB)] = True
    if g.dense:
        kept[:] = True
    eye = np.eye(g.Np)
    eye[pad] = 0.0
    P = O.block_attention(qr, kr, eye, kept, g)
    np.testing.assert_allclose(P[rows].sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(P >= 0)
    assert np.all(P[:, pad] == 0) and np.all(P[pad] == 0)
    comp = bool(flags & O.SVA_COMPENSATE)
    for qb in range(g.nB):
        r = slice(qb * g.block, qb * g.block + valid[qb])
        for kb in range(g.nB):
            c = slice(kb * g.block, kb * g.block + valid[kb])
            if kept[qb, kb]:
                assert np.all(P[r, c] > 0)
            elif comp:
                w = P[r, c]
                np.testing.assert_allclose(w, np.repeat(w[:, :1], w.shape[1], axis=1), rtol=1e-12)
                assert np.all(w > 0)
            else:
                assert np.all(P[r, c] == 0)
    ones = np.zeros((g.Np, g.d))
    ones[rows] = 1.0
    o1 = O.block_attention(qr, kr, ones, kept, g)
    np.testing.assert_allclose(o1[rows], 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("flags,sparsity", [(0, 0.5), (0, 0.0), (O.SVA_DENSE, 0.7),
                                            (O.SVA_COMPENSATE, 0.5),
                                            (O.SVA_COMPENSATE | O.SVA_KEEP_SAME_FRAME, 0.6)])
def test_attention_row_sums_are_one(flags, sparsity):
    check_attention_row_sums(flags, sparsity)


def test_attention_permutation_equivariance():
    """Dense attention on the tile-ordered sequence, mapped back to raster
    order, equals dense attention computed directly in raster order."""
    g = O.Geometry(B=1, H=1, T=3, Hh=5, W=7, d=32, block=64, sparsity=0.0, tile=(2, 2, 4))
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((g.N, g.d)) for _ in range(3))
    perm = O.permutation(g)
    qr, kr, vr = (np.zeros((g.Np, g.d)) for _ in range(3))
    qr[perm], kr[perm], vr[perm] = q, k, v
    out = O.block_attention(qr, kr, vr, np.ones((g.nB, g.nB), bool), g)[perm]
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- whole head

def test_run_head_dense_flag_equals_sparsity_zero():
    from block_sparse_attention_qk_amd import inputs as I
    wl = I.custom("t", 1, 1, 3, 8, 8, 64, 64, 0.0, tile=(2, 4, 4))
    q, k, v = (O.bf16_bits_to_f64(I.head_field(wl, t, 0, 0)) for t in range(3))
    w = np.ones(64)
    ga = O.Geometry(B=1, H=1, T=3, Hh=8, W=8, d=64, block=64, sparsity=0.0, tile=(2, 4, 4))
    gb = O.Geometry(B=1, H=1, T=3, Hh=8, W=8, d=64, block=64, sparsity=0.9, tile=(2, 4, 4),
                    flags=O.SVA_DENSE)
    ra = O.run_head(q, k, v, w, w, ga)
    rb = O.run_head(q, k, v, w, w, gb)
    assert ra["kept"].all() and rb["kept"].all()
    np.testing.assert_array_equal(ra["o"], rb["o"])
    # and the dense output equals library attention on the prologue outputs
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(ra["qn"]), t(ra["kn"]), t(v))[0, 0]
    np.testing.assert_allclose(ra["o"], ref.numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    # 1. RoPE rotating the wrong way
    orig_angles = O.rope_angles
    monkeypatch.setattr(O, "rope_angles", lambda p, w, th: -orig_angles(p, w, th))
    assert _fails(check_rope_library)
    monkeypatch.setattr(O, "rope_angles", orig_angles)
    # 2. RoPE frequency exponent without the factor 2
    def bad_angles(pos, width, theta):
        i = np.arange(width // 2, dtype=np.float64)
        return np.asarray(pos, np.float64)[:, None] * (theta ** (-i / width))[None, :]
    monkeypatch.setattr(O, "rope_angles", bad_angles)
    assert _fails(check_rope_library)
    monkeypatch.setattr(O, "rope_angles", orig_angles)
    # 2b. RoPE base ignored (always 10000)
    monkeypatch.setattr(O, "rope_angles", lambda p, w, th: orig_angles(p, w, 10000.0))
    assert _fails(check_rope_library)
    monkeypatch.setattr(O, "rope_angles", orig_angles)
    # 2c. grid coordinates with h and w swapped
    orig_pos = O.token_positions
    def swapped(g):
        t, h, w = orig_pos(g)
        n = np.arange(g.n_video)
        return t, n % g.Hh, (n // g.Hh) % g.W
    monkeypatch.setattr(O, "token_positions", swapped)
    assert _fails(check_rope_coordinates)
    monkeypatch.setattr(O, "token_positions", orig_pos)
    # 3. RMSNorm without the mean (sum of squares)
    orig_norm = O.rms_norm
    monkeypatch.setattr(O, "rms_norm", lambda x, w, eps: np.asarray(x) / np.sqrt(
        np.sum(np.asarray(x) ** 2, axis=-1, keepdims=True) + eps) * w)
    assert _fails(check_rmsnorm)
    monkeypatch.setattr(O, "rms_norm", orig_norm)
    # 3b. RMSNorm epsilon ignored
    monkeypatch.setattr(O, "rms_norm", lambda x, w, eps: orig_norm(x, w, 0.0))
    assert _fails(check_rmsnorm)
    monkeypatch.setattr(O, "rms_norm", orig_norm)
    # 3c. no rounding between the norm and the rotation
    orig_pro = O.qk_norm_rope
    monkeypatch.setattr(O, "qk_norm_rope", lambda x, w, g: O.to_bf16(
        O.rope_3d(O.rms_norm(x, w, g.eps), g)))
    assert _fails(check_prologue_rounding_golden)
    monkeypatch.setattr(O, "qk_norm_rope", orig_pro)
    # 4. bf16 rounding by truncation
    orig_bf = O.to_bf16
    def trunc(x):
        x = np.asarray(x, np.float64)
        _, e = np.frexp(x)
        e = np.maximum(e, -125)
        return np.ldexp(np.trunc(np.ldexp(x, 8 - e)), e - 8)
    monkeypatch.setattr(O, "to_bf16", trunc)
    assert _fails(check_bf16_golden)
    monkeypatch.setattr(O, "to_bf16", orig_bf)
    # 5. permutation in (w, h, t) order inside a tile
    orig_perm = O.permutation
    def bad_perm(g):
        p = orig_perm(g).copy()
        tt, th, tw = g.tile
        if tt * th * tw > 1:
            t, h, w = O.token_positions(g)
            base = p[: g.n_video] - ((t % tt) * th * tw + (h % th) * tw + (w % tw))
            inner = (w % tw) * th * tt + (h % th) * tt + (t % tt)
            full = ((t // tt) == (g.T // tt)) | ((h // th) == (g.Hh // th)) | ((w // tw) == (g.W // tw))
            p[: g.n_video] = np.where(full, p[: g.n_video], base + inner)
        return p
    monkeypatch.setattr(O, "permutation", bad_perm)
    assert _fails(check_perm_golden)
    monkeypatch.setattr(O, "permutation", orig_perm)
    # 6. selection tie-break or order reversed
    orig_sel = O.select_blocks
    def bad_sel(qbar, kbar, g, meta=None):
        return orig_sel(-np.asarray(qbar), kbar, g, meta)
    monkeypatch.setattr(O, "select_blocks", bad_sel)
    assert _fails(check_selection_bruteforce)
    monkeypatch.setattr(O, "select_blocks", orig_sel)
    # 7. attention without the 1/sqrt(d) scale
    orig_attn = O.block_attention
    def bad_attn(qr, kr, vr, kept, g, meta=None, qblocks=None):
        return orig_attn(np.asarray(qr) * math.sqrt(g.d), kr, vr, kept, g, meta, qblocks)
    monkeypatch.setattr(O, "block_attention", bad_attn)
    assert _fails(check_dense_attention_sdpa)
    # 8. sparse attention ignoring the mask (every block kept)
    def bad_attn2(qr, kr, vr, kept, g, meta=None, qblocks=None):
        return orig_attn(qr, kr, vr, np.ones_like(kept), g, meta, qblocks)
    monkeypatch.setattr(O, "block_attention", bad_attn2)
    assert _fails(check_sparse_attention_masked_sdpa)
    monkeypatch.setattr(O, "block_attention", orig_attn)
    # 9. compensation without the block-size weight (each dropped block
    #    counted once instead of |B| times)
    orig_attn2 = O.block_attention
    def bad_comp(qr, kr, vr, kept, g, meta=None, qblocks=None):
        if not (g.flags & O.SVA_COMPENSATE):
            return orig_attn2(qr, kr, vr, kept, g, meta, qblocks)
        valid = O.block_meta(g)[0]
        b, out = g.block, np.zeros((g.Np, g.d))
        for qb in range(g.nB):
            keys = np.concatenate([np.arange(kb * b, kb * b + valid[kb])
                                   for kb in np.nonzero(kept[qb])[0]])
            qs = np.asarray(qr)[qb * b: qb * b + valid[qb]]
            lg = qs @ np.asarray(kr)[keys].T / math.sqrt(g.d)
            vals = np.asarray(vr)[keys]
            for kb in np.nonzero(~kept[qb])[0]:
                km = np.asarray(kr)[kb * b: kb * b + valid[kb]].mean(axis=0)
                vm = np.asarray(vr)[kb * b: kb * b + valid[kb]].mean(axis=0)
                lg = np.concatenate([lg, (qs @ km)[:, None] / math.sqrt(g.d)], axis=1)
                vals = np.concatenate([vals, vm[None]], axis=0)
            e = np.exp(lg - lg.max(axis=1, keepdims=True))
            out[qb * b: qb * b + valid[qb]] = e @ vals / e.sum(axis=1, keepdims=True)
        return out
    monkeypatch.setattr(O, "block_attention", bad_comp)
    assert _fails(check_compensation_exact)
    monkeypatch.setattr(O, "block_attention", orig_attn2)
    # 10. SubBlock estimate without the sub-block counts
    orig_cnt = O.subblock_counts
    monkeypatch.setattr(O, "subblock_counts",
                        lambda g, valid=None: np.minimum(orig_cnt(g, valid), 1))
    assert _fails(check_subblock_exact)
    monkeypatch.setattr(O, "subblock_counts", orig_cnt)
    # 11. SubBlock estimate with the max instead of the sum over sub-block pairs
    orig_sub = O.subblock_scores
    def bad_sub(qs, ks, g, valid=None):
        cnt = O.subblock_counts(g, valid).astype(float)
        with np.errstate(divide="ignore"):
            lq = np.log(cnt)
        x = np.einsum("iad,jbd->ijab", qs, ks) / math.sqrt(g.d)
        return (x + lq[:, None, :, None] + lq[None, :, None, :]).max(axis=(2, 3))
    monkeypatch.setattr(O, "subblock_scores", bad_sub)
    assert _fails(check_subblock_exact)
    monkeypatch.setattr(O, "subblock_scores", orig_sub)
    # 12. compensation whose softmax denominator leaves the dropped blocks out
    #     (their weighted mean values added to the numerator only)
    def bad_den(qr, kr, vr, kept, g, meta=None, qblocks=None):
        if not (g.flags & O.SVA_COMPENSATE):
            return orig_attn2(qr, kr, vr, kept, g, meta, qblocks)
        valid = O.block_meta(g)[0]
        b, out = g.block, np.zeros((g.Np, g.d))
        for qb in range(g.nB):
            keys = np.concatenate([np.arange(kb * b, kb * b + valid[kb])
                                   for kb in np.nonzero(kept[qb])[0]])
            qs = np.asarray(qr)[qb * b: qb * b + valid[qb]]
            lg = qs @ np.asarray(kr)[keys].T / math.sqrt(g.d)
            m = lg.max(axis=1, keepdims=True)
            e = np.exp(lg - m)
            num = e @ np.asarray(vr)[keys]
            for kb in np.nonzero(~kept[qb])[0]:
                km = np.asarray(kr)[kb * b: kb * b + valid[kb]].mean(axis=0)
                vm = np.asarray(vr)[kb * b: kb * b + valid[kb]].mean(axis=0)
                wgt = valid[kb] * np.exp((qs @ km)[:, None] / math.sqrt(g.d) - m)
                num = num + wgt * vm[None, :]
            out[qb * b: qb * b + valid[qb]] = num / e.sum(axis=1, keepdims=True)
        return out
    monkeypatch.setattr(O, "block_attention", bad_den)
    assert _fails(lambda: check_attention_row_sums(O.SVA_COMPENSATE, 0.5))
    monkeypatch.setattr(O, "block_attention", orig_attn2)
    # 13. sparse attention whose softmax denominator runs over the valid keys
    #     of every block, kept or not (numerator over the kept ones only)
    def bad_den2(qr, kr, vr, kept, g, meta=None, qblocks=None):
        valid = O.block_meta(g)[0]
        b, out = g.block, np.zeros((g.Np, g.d))
        allk = np.concatenate([np.arange(kb * b, kb * b + valid[kb]) for kb in range(g.nB)])
        for qb in range(g.nB):
            qs = np.asarray(qr)[qb * b: qb * b + valid[qb]]
            lg = qs @ np.asarray(kr)[allk].T / math.sqrt(g.d)
            e = np.exp(lg - lg.max(axis=1, keepdims=True))
            on = kept[qb][allk // b]
            out[qb * b: qb * b + valid[qb]] = ((e * on) @ np.asarray(vr)[allk]
                                                / e.sum(axis=1, keepdims=True))
        return out
    monkeypatch.setattr(O, "block_attention", bad_den2)
    assert _fails(lambda: check_attention_row_sums(0, 0.5))
    monkeypatch.setattr(O, "block_attention", orig_attn2)
