"""Plain CPU oracle for the block-sparse video-DiT self-attention step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, tables or helpers) and imports nothing but NumPy.

What it computes, step by step, in float64 (the steps follow the pages; the
readings where the pages are silent are listed in the repository's design
notes and repeated next to each function):

1. QK-RMSNorm + 3D-RoPE on Q and K.  The MiniMax-H3 benchmark page ("MiniMax-H3
   在 8×H200 上基准测试", sections "加速从何而来" and "内核层") fuses a QK RMSNorm
   with a 3D RoPE and names the exact-rounding path round_norm_before_rope=True:
   the normalised value is stored (rounded to bf16) before the rotation, and the
   rotated value is rounded to bf16 again.
2. A permutation of the raster video tokens into 3D-tile order, padded at the
   tail to a multiple of the block size; extra (audio/text) tokens follow.
3. Mean pooling of Q' and K' per block ("SubBlock 稀疏注意力如何工作": a
   lightweight pooling step scores key blocks per query block and head).
4. Block scores, forced blocks, and top-k key blocks per (query block, head)
   at keep ratio 1 - sparsity (same section: sparsity is the fraction of key
   blocks dropped, ranking is independent per query block and head, and the
   kept indices are handed to the block-sparse kernel).  Two scorers: the mean
   scorer q̄·k̄, and the SubBlock scorer of the same section (sub-block means
   combined by log-sum-exp into an estimate of each key block's unnormalised
   softmax mass), optionally with the budget rounded to multiples of 8.
5. Exact softmax attention of each query over the valid keys of its kept
   blocks, non-causal (same section: the sparse path serves non-causal DiT
   attention and never builds the full attention matrix).  With every block
   kept this is textbook dense attention.  Optionally the dropped blocks
   enter the softmax as their mean key and value weighted by their size
   (compensation; the Sol-Attn README and the Sol blog's 4.2.2 on PISA).
6. The inverse permutation of the output.

Rounding: the only roundings modelled are the two bf16 storage points of
step 1, since Q' and K' are stored as bf16 and the block choice depends on
them.  Everything else is float64.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SVA_DENSE = 1
SVA_KEEP_SAME_FRAME = 2
SVA_COMPENSATE = 4
SCORER_MEAN = 0
SCORER_SUBBLOCK = 1


# --------------------------------------------------------------------------
# bf16 storage rounding (round to nearest, ties to even), float64 -> float64
# --------------------------------------------------------------------------

def to_bf16(x):
    """Round float64 values to the nearest bf16 value (ties to even).

    bf16 keeps 8 significant bits and the float32 exponent range, so a value
    in [2**(e-1), 2**e) is rounded to a multiple of 2**(e-8); below the
    smallest normal (2**-126) the spacing stays 2**-133.  The scaling by a
    power of two is exact, and ``np.rint`` rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> uint16 bf16 bit patterns, rounding to nearest even first."""
    r = to_bf16(x).astype(np.float32)          # exact: r is a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------
# Geometry of one attention call
# --------------------------------------------------------------------------

@dataclass
class Geometry:
    """Shapes of one call.  Grid T×Hh×W video tokens in raster order
    n = (t·Hh + h)·W + w, followed by ``n_extra`` extra tokens."""

    B: int
    H: int
    T: int
    Hh: int
    W: int
    d: int
    block: int
    sparsity: float
    flags: int = 0
    tile: tuple = (0, 0, 0)
    n_extra: int = 0
    theta: float = 10000.0
    split: tuple = (0, 0, 0)
    eps: float = 1e-6
    scorer: int = SCORER_MEAN
    subblocks: int = 0          # sub-blocks per block (SubBlock scorer); 0 = 4
    budget_multiple: int = 1    # round the budget up to a multiple of this
    # derived
    n_video: int = field(init=False)
    N: int = field(init=False)
    n_video_pad: int = field(init=False)
    Np: int = field(init=False)
    nB: int = field(init=False)
    nB_video: int = field(init=False)
    k: int = field(init=False)

    def __post_init__(self):
        if tuple(self.tile) == (0, 0, 0):
            self.tile = (4, 4, 4) if self.block == 64 else (2, 8, 8)
        if tuple(self.split) == (0, 0, 0):
            self.split = (16, 24, 24) if self.d == 64 else (44, 42, 42)
        self.tile = tuple(int(v) for v in self.tile)
        self.split = tuple(int(v) for v in self.split)
        self.n_video = self.T * self.Hh * self.W
        self.N = self.n_video + self.n_extra
        b = self.block
        self.n_video_pad = -(-self.n_video // b) * b
        self.Np = self.n_video_pad + self.n_extra
        self.nB = self.Np // b
        self.nB_video = self.n_video_pad // b
        if self.subblocks == 0:
            self.subblocks = 4 if self.scorer == SCORER_SUBBLOCK else 1
        self.k = budget(self.nB, self.sparsity, self.flags, self.budget_multiple)

    @property
    def dense(self) -> bool:
        return bool(self.flags & SVA_DENSE) or self.sparsity == 0.0


def budget(nB: int, sparsity: float, flags: int = 0, multiple: int = 1) -> int:
    """Key blocks kept per query row.

    The benchmark page ("SubBlock 稀疏注意力如何工作") defines sparsity as the
    fraction of key blocks that may be dropped, so sparsity 0.75 keeps about a
    quarter.  Reading: keep ceil((1 - sparsity)·nB) blocks (the 1e-9 guards a
    product that lands a hair above an integer), at least one, at most all;
    sparsity 0 or the dense flag keeps every block.  The same section says the
    SubBlock router's budget is rounded in units of 8 blocks; with
    ``multiple`` > 1 the budget is rounded up to a multiple of it (reading:
    up, so at least the requested fraction is kept), then clamped to nB.
    """
    if (flags & SVA_DENSE) or sparsity == 0.0:
        return nB
    k = math.ceil((1.0 - sparsity) * nB - 1e-9)
    if multiple > 1:
        k = -(-k // multiple) * multiple
    return max(1, min(nB, k))


# --------------------------------------------------------------------------
# Step 1: QK-RMSNorm + 3D-RoPE
# --------------------------------------------------------------------------

def rms_norm(x, w, eps):
    """RMS normalisation over the last axis (head dim), times weight ``w``.

    y = x / sqrt(mean(x²) + eps) · w.  Reading: per (token, head) over the
    head dimension, weight of shape [d] per head (ones when absent).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def token_positions(geom: Geometry):
    """(t, h, w) grid coordinates of every raster video token."""
    n = np.arange(geom.n_video)
    w = n % geom.W
    h = (n // geom.W) % geom.Hh
    t = n // (geom.W * geom.Hh)
    return t, h, w


def rope_angles(pos, width, theta):
    """Angles of the rotary pairs of one axis section of width ``width``:
    pair i at integer position p turns by p · theta^(-2i/width)."""
    i = np.arange(width // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / width)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope_3d(y, geom: Geometry):
    """Apply 3D rotary embedding to y of shape [..., N, d] (float64).

    Reading: the head dimension is cut into contiguous sections for the t, h
    and w axes (widths ``geom.split``); inside a section, element pairs
    (2i, 2i+1) rotate by the token's coordinate on that axis times
    theta^(-2i/width).  Dimensions past the three sections, and every extra
    token, are left unrotated.
    """
    y = np.array(y, dtype=np.float64, copy=True)
    t, h, w = token_positions(geom)
    off = 0
    for pos, width in zip((t, h, w), geom.split):
        if width == 0:
            continue
        ang = rope_angles(pos, width, geom.theta)          # [n_video, width/2]
        c, s = np.cos(ang), np.sin(ang)
        sec = y[..., : geom.n_video, off: off + width]
        a = sec[..., 0::2].copy()
        b = sec[..., 1::2].copy()
        sec[..., 0::2] = a * c - b * s
        sec[..., 1::2] = a * s + b * c
        y[..., : geom.n_video, off: off + width] = sec
        off += width
    return y


def qk_norm_rope(x, w, geom: Geometry):
    """Prologue for one tensor of one head: x [..., N, d] float64 values of
    bf16 inputs, w [d] → bf16-valued float64 [..., N, d].

    Rounding order per the page's exact-rounding path: RMSNorm → round to
    bf16 → RoPE → round to bf16.
    """
    y = to_bf16(rms_norm(x, w, geom.eps))
    return to_bf16(rope_3d(y, geom))


# --------------------------------------------------------------------------
# Step 2: 3D-tile permutation
# --------------------------------------------------------------------------

def permutation(geom: Geometry):
    """perm[n] = position of raster token n in the tile-ordered sequence.

    Reading: tiles of size tile=(tt, th, tw) cover the grid, edge tiles are
    clipped; tiles are visited in (t, h, w)-lexicographic order of their
    origin and the tokens inside a tile in (t, h, w) order.  The concatenation
    is padded once at the tail to a multiple of the block size; extra tokens
    come after the padding, in their own order.
    """
    tt, th, tw = geom.tile
    T, Hh, W = geom.T, geom.Hh, geom.W
    perm = np.empty(geom.N, dtype=np.int64)
    p = 0
    for t0 in range(0, T, tt):
        for h0 in range(0, Hh, th):
            for w0 in range(0, W, tw):
                for t in range(t0, min(t0 + tt, T)):
                    for h in range(h0, min(h0 + th, Hh)):
                        for w in range(w0, min(w0 + tw, W)):
                            perm[(t * Hh + h) * W + w] = p
                            p += 1
    assert p == geom.n_video
    perm[geom.n_video:] = geom.n_video_pad + np.arange(geom.n_extra)
    return perm


def reorder_forward(x, geom: Geometry, perm=None):
    """[B, N, H, d] raster → [B, H, Np, d] tile order, padding rows zero."""
    perm = permutation(geom) if perm is None else perm
    B, N, H, d = x.shape
    out = np.zeros((B, H, geom.Np, d), dtype=x.dtype)
    out[:, :, perm, :] = np.transpose(x, (0, 2, 1, 3))
    return out


def reorder_inverse(xr, geom: Geometry, perm=None):
    """[B, H, Np, d] tile order → [B, N, H, d] raster (padding dropped)."""
    perm = permutation(geom) if perm is None else perm
    return np.transpose(xr[:, :, perm, :], (0, 2, 1, 3))


# --------------------------------------------------------------------------
# Step 3: block metadata and pooling
# --------------------------------------------------------------------------

def block_meta(geom: Geometry, perm=None):
    """Per block: number of valid tokens, first and last frame (t) of its
    valid video tokens, and whether it holds extra tokens."""
    perm = permutation(geom) if perm is None else perm
    b = geom.block
    valid = np.zeros(geom.nB, dtype=np.int64)
    tmin = np.full(geom.nB, np.iinfo(np.int64).max)
    tmax = np.full(geom.nB, -1)
    t, _, _ = token_positions(geom)
    blk = perm[: geom.n_video] // b
    np.add.at(valid, blk, 1)
    np.minimum.at(tmin, blk, t)
    np.maximum.at(tmax, blk, t)
    extra = np.zeros(geom.nB, dtype=bool)
    extra[geom.nB_video:] = True
    valid[geom.nB_video:] = b
    tmin[geom.nB_video:] = -1
    tmax[geom.nB_video:] = -1
    return valid, tmin, tmax, extra


def pool_means(xr, geom: Geometry, valid=None):
    """Mean of each block over its valid tokens: xr [..., Np, d] → [..., nB, d].

    Padding rows hold zeros, so the block sum over all rows equals the sum
    over valid rows; the mean divides by the valid count.
    """
    if valid is None:
        valid, _, _, _ = block_meta(geom)
    x = np.asarray(xr, dtype=np.float64)
    s = x.reshape(x.shape[:-2] + (geom.nB, geom.block, geom.d)).sum(axis=-2)
    return s / valid[:, None]


def subblock_counts(geom: Geometry, valid=None):
    """Valid tokens of each sub-block: [nB, n].  A block of b tile-order
    positions is split into n runs of b/n consecutive positions; its valid
    tokens are the first ``valid`` positions."""
    if valid is None:
        valid, _, _, _ = block_meta(geom)
    n = geom.subblocks
    sb = geom.block // n
    start = np.arange(n) * sb
    return np.clip(np.asarray(valid)[:, None] - start[None, :], 0, sb)


def subblock_means(xr, geom: Geometry, valid=None):
    """Mean of every sub-block over its valid tokens: [Np, d] → [nB, n, d]
    (zero for a sub-block without valid tokens)."""
    cnt = subblock_counts(geom, valid)
    n = geom.subblocks
    x = np.asarray(xr, dtype=np.float64)
    s = x.reshape(geom.nB, n, geom.block // n, geom.d).sum(axis=2)
    return np.where(cnt[..., None] > 0, s / np.maximum(cnt, 1)[..., None], 0.0)


def subblock_scores(qsub, ksub, geom: Geometry, valid=None):
    """SubBlock block scores: [nB, nB].

    The benchmark page ("SubBlock 稀疏注意力如何工作") splits every query and
    key block into sub-blocks, pools them, and scores each key block for a
    query block by a log-sum-exp estimate of its unnormalised softmax mass.
    Reading: replace every query and key by the mean of its sub-block; the
    mass of key block kb for the query rows of qb,
        sum_{p in qb} sum_{j in kb} exp(q_p·k_j / sqrt(d)),
    becomes
        score = log sum_a sum_b c_a c_b exp(q̄_a·k̄_b / sqrt(d)),
    with c the valid counts of the sub-blocks (empty sub-blocks drop out).
    It is exact when every sub-block holds identical rows.
    """
    cnt = subblock_counts(geom, valid).astype(np.float64)
    d = geom.d
    q = np.asarray(qsub, np.float64)
    k = np.asarray(ksub, np.float64)
    with np.errstate(divide="ignore"):
        lq = np.log(cnt)                 # -inf for empty sub-blocks
    x = np.einsum("iad,jbd->ijab", q, k) / math.sqrt(d)
    x = x + lq[:, None, :, None] + lq[None, :, None, :]
    m = x.max(axis=(2, 3))
    return m + np.log(np.exp(x - m[:, :, None, None]).sum(axis=(2, 3)))


# --------------------------------------------------------------------------
# Step 4: block scores and top-k selection
# --------------------------------------------------------------------------

def forced_blocks(geom: Geometry, meta=None):
    """forced[qb, kb] for the always-kept blocks, and dense[qb] for rows
    that keep every block.

    Readings: extra-token key blocks are always kept (dense columns) and
    extra-token query blocks keep every key block (dense rows); with the
    same-frame flag, two video blocks are "same frame" when the frame
    intervals of their valid tokens intersect.
    """
    valid, tmin, tmax, extra = block_meta(geom) if meta is None else meta
    nB = geom.nB
    forced = np.zeros((nB, nB), dtype=bool)
    forced[:, extra] = True
    if geom.flags & SVA_KEEP_SAME_FRAME:
        vid = ~extra
        inter = (tmin[:, None] <= tmax[None, :]) & (tmin[None, :] <= tmax[:, None])
        forced |= inter & vid[:, None] & vid[None, :]
    dense_row = extra.copy()
    if geom.dense:
        dense_row[:] = True
    return forced, dense_row


def row_lengths(geom: Geometry, meta=None):
    """Blocks kept per query block: every block for a dense row, otherwise
    max(k, number of forced blocks) — forced blocks count toward the budget."""
    forced, dense_row = forced_blocks(geom, meta)
    nf = forced.sum(axis=1)
    return np.where(dense_row, geom.nB, np.maximum(geom.k, nf)).astype(np.int64)


def select_blocks(qbar, kbar, geom: Geometry, meta=None):
    """Kept key blocks of one (batch, head) under the mean scorer.

    qbar, kbar: [nB, d] block means.  Score s[qb, kb] = q̄_qb · k̄_kb; the
    selection is ``select_from_scores``.
    """
    scores = np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T
    return select_from_scores(scores, geom, meta)


def select_from_scores(scores, geom: Geometry, meta=None):
    """Each row keeps its forced blocks plus the best remaining blocks
    ordered by (score descending, block index ascending) until it holds
    ``row_lengths`` blocks.

    Returns (kept [nB, nB] bool, scores [nB, nB], thresh [nB], smax [nB]):
    thresh is the score of the last block taken from the ranking (nan when
    none was needed) and smax the row's largest |score|, for the tie margin.
    """
    forced, dense_row = forced_blocks(geom, meta)
    nB = geom.nB
    lens = row_lengths(geom, meta)
    scores = np.asarray(scores, np.float64)
    kept = np.zeros((nB, nB), dtype=bool)
    thresh = np.full(nB, np.nan)
    smax = np.abs(scores).max(axis=1)
    idx = np.arange(nB)
    for qb in range(nB):
        if dense_row[qb]:
            kept[qb, :] = True
            continue
        f = forced[qb]
        kept[qb, f] = True
        need = int(lens[qb] - f.sum())
        if need <= 0:
            continue
        cand = idx[~f]
        sc = scores[qb, cand]
        order = np.lexsort((cand, -sc))    # score desc, then index asc
        take = cand[order[:need]]
        kept[qb, take] = True
        thresh[qb] = scores[qb, take[-1]]
    return kept, scores, thresh, smax


# --------------------------------------------------------------------------
# Step 5: attention over the kept blocks
# --------------------------------------------------------------------------

def block_attention(qr, kr, vr, kept, geom: Geometry, meta=None, qblocks=None):
    """Attention of one (batch, head) over its kept blocks.

    qr, kr, vr: [Np, d] tile-ordered values.  For every valid query token p
    of query block qb: o_p = Σ_j softmax_j(q_p·k_j / sqrt(d)) v_j over the
    valid key tokens j of the key blocks kept for qb, with the softmax taken
    in two passes (max, then exp and sum).  Padding query rows are zero.
    Only the query blocks in ``qblocks`` (default all) are computed; the
    others are left at zero.

    With the compensate flag, every key block dropped from the row also
    enters the softmax, as its mean key and mean value (over its valid
    tokens) weighted by its valid count |B|: one extra logit
    q_p·k̄_B / sqrt(d) + ln|B| with value v̄_B per dropped block.  The pages
    name a light-weight compensation of the dropped blocks (the Sol-Attn
    README) and a first-order Taylor compensation (PISA, in the Sol blog's
    4.2.2); this is the leading term of that expansion: summed over the
    block, the first-order term of exp(q·k_j) around k̄_B vanishes, and the
    value term it leaves out would need a d×d moment per block.
    """
    valid, _, _, _ = block_meta(geom) if meta is None else meta
    b, d = geom.block, geom.d
    q = np.asarray(qr, np.float64)
    k = np.asarray(kr, np.float64)
    v = np.asarray(vr, np.float64)
    out = np.zeros((geom.Np, d), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    comp = bool(geom.flags & SVA_COMPENSATE)
    if comp:
        kbar = np.stack([k[kb * b: kb * b + valid[kb]].mean(axis=0) for kb in range(geom.nB)])
        vbar = np.stack([v[kb * b: kb * b + valid[kb]].mean(axis=0) for kb in range(geom.nB)])
    rows = range(geom.nB) if qblocks is None else qblocks
    for qb in rows:
        keys = np.concatenate([np.arange(kb * b, kb * b + valid[kb])
                               for kb in np.nonzero(kept[qb])[0]])
        qs = q[qb * b: qb * b + valid[qb]]
        logits = (qs @ k[keys].T) * scale
        vals = v[keys]
        if comp:
            drop = np.nonzero(~kept[qb])[0]
            if drop.size:
                extra = (qs @ kbar[drop].T) * scale + np.log(valid[drop].astype(np.float64))
                logits = np.concatenate([logits, extra], axis=1)
                vals = np.concatenate([vals, vbar[drop]], axis=0)
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        out[qb * b: qb * b + valid[qb]] = (e @ vals) / e.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# The whole step for one (batch, head)
# --------------------------------------------------------------------------

def run_head(q, k, v, wq, wk, geom: Geometry, qblocks=None, perm=None, meta=None):
    """The full path for one (batch, head).

    q, k, v: [N, d] float64 values of the bf16 raster inputs of that head;
    wq, wk: [d] RMSNorm weights.  Returns a dict with the bf16-valued
    prologue outputs (raster), the tile-ordered tensors, block means, the
    kept mask with its scores and tie margins, and the attention output both
    tile-ordered (``o_r``) and raster (``o``).
    """
    perm = permutation(geom) if perm is None else perm
    meta = block_meta(geom, perm) if meta is None else meta
    qn = qk_norm_rope(q, wq, geom)
    kn = qk_norm_rope(k, wk, geom)
    qr = np.zeros((geom.Np, geom.d))
    kr = np.zeros((geom.Np, geom.d))
    vr = np.zeros((geom.Np, geom.d))
    qr[perm] = qn
    kr[perm] = kn
    vr[perm] = np.asarray(v, np.float64)
    qbar = pool_means(qr, geom, meta[0])
    kbar = pool_means(kr, geom, meta[0])
    if geom.scorer == SCORER_SUBBLOCK:
        scores = subblock_scores(subblock_means(qr, geom, meta[0]),
                                 subblock_means(kr, geom, meta[0]), geom, meta[0])
        kept, scores, thresh, smax = select_from_scores(scores, geom, meta)
    else:
        kept, scores, thresh, smax = select_blocks(qbar, kbar, geom, meta)
    o_r = block_attention(qr, kr, vr, kept, geom, meta, qblocks)
    return dict(qn=qn, kn=kn, qr=qr, kr=kr, vr=vr, qbar=qbar, kbar=kbar,
                kept=kept, scores=scores, thresh=thresh, smax=smax,
                o_r=o_r, o=o_r[perm])
