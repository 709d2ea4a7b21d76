"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and lays them out; it holds none of
the attention method's arithmetic.  Both the HIP path (tests, bench) and the
CPU oracle (tests) take their inputs from here, so the two sides see the
same bits.

Field model (stands in for video-DiT activations, which are smooth in space
and time): for every (tensor, batch, head, channel) a coarse N(0,1) grid of
2×4×4 (t, h, w) points is upsampled trilinearly (align-corners mapping) to
the full T×Hh×W latent grid, then 0.5·N(0,1) noise is added at full
resolution and the result is rounded to bf16 (nearest, ties to even).
Extra (audio/text) tokens are plain N(0,1).  Each (tensor, batch, head) has
its own PCG64 stream seeded from (workload seed, tensor, batch, head), so a
single head can be regenerated without drawing the others.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

DENSE = 1
KEEP_SAME_FRAME = 2
COMPENSATE = 4

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
_STREAM_TAU = 3
_STREAM_EXTRA = 4


@dataclass(frozen=True)
class Workload:
    """One named call shape.  ``seed_base`` = 1000 × workload number."""

    name: str
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
    temperature: bool = False
    seed_base: int = 0
    rope_split: tuple = (0, 0, 0)   # t/h/w RoPE channels; zeros = the plan's default
    scorer: int = 0                 # 0 mean of each block, 1 SubBlock estimate
    subblocks: int = 0              # runs per block for the SubBlock scorer (0 = 4)
    budget_multiple: int = 0        # round the budget up to a multiple (0 = 1)
    rope_theta: float = 0.0         # RoPE base (0 = 10000)
    eps: float = 0.0                # RMSNorm epsilon (0 = 1e-6)

    @property
    def theta_resolved(self) -> float:
        return self.rope_theta if self.rope_theta else 10000.0

    @property
    def eps_resolved(self) -> float:
        return self.eps if self.eps else 1e-6

    @property
    def n_video(self) -> int:
        return self.T * self.Hh * self.W

    @property
    def N(self) -> int:
        return self.n_video + self.n_extra


WORKLOADS = {
    # tiny: 4×16×16 grid, tiles 4×4×4 = blocks of 64
    "tiny": Workload("tiny", 1, 2, 4, 16, 16, 64, 64, 0.5,
                     tile=(4, 4, 4), seed_base=0),
    # Wan2.1-1.3B-like 480p latent grid, block 64, dense and sparse
    "wan480p_dense": Workload("wan480p_dense", 1, 12, 21, 30, 52, 128, 64, 0.0,
                              tile=(3, 4, 8), seed_base=1000),
    "wan480p_sp75": Workload("wan480p_sp75", 1, 12, 21, 30, 52, 128, 64, 0.75,
                             tile=(3, 4, 8), seed_base=1000),
    # Wan2.1-14B-like 720p, 75,600 tokens, same-frame key blocks always kept
    "wan720p_sp75": Workload("wan720p_sp75", 1, 40, 21, 45, 80, 128, 128, 0.75,
                             flags=KEEP_SAME_FRAME, tile=(2, 8, 8),
                             temperature=True, seed_base=2000),
    # HunyuanVideo-like 1280×720×129f, sparse and dense-flag runs
    "hunyuan720p_sp80": Workload("hunyuan720p_sp80", 1, 24, 33, 45, 80, 128, 128, 0.80,
                                 tile=(2, 8, 8), seed_base=3000),
    "hunyuan720p_dense": Workload("hunyuan720p_dense", 1, 24, 33, 45, 80, 128, 128, 0.80,
                                  flags=DENSE, tile=(2, 8, 8), seed_base=3000),
    # packed video + 512 audio/text tokens (always-dense rows and columns)
    "packed768p_sp80": Workload("packed768p_sp80", 1, 48, 31, 48, 84, 128, 128, 0.80,
                                tile=(2, 8, 8), n_extra=512, seed_base=4000),
    # HunyuanVideo-like inputs with the dropped blocks compensated
    "hunyuan720p_comp": Workload("hunyuan720p_comp", 1, 24, 33, 45, 80, 128, 128, 0.80,
                                 flags=COMPENSATE, tile=(2, 8, 8), seed_base=3000),
    # the 720p inputs under the SubBlock scorer (4 runs of 32 tokens per
    # block, budget rounded up to a multiple of 8 blocks)
    "wan720p_subblock": Workload("wan720p_subblock", 1, 40, 21, 45, 80, 128, 128, 0.75,
                                 flags=KEEP_SAME_FRAME, tile=(2, 8, 8), temperature=True,
                                 seed_base=2000, scorer=1, budget_multiple=8),
    # the SubBlock router at the configuration that defines it: 64-token
    # blocks cut into four 16-token sub-blocks, budget rounded up to a
    # multiple of 8 blocks, on the 480p inputs at sparsity 0.75
    "wan480p_subblock": Workload("wan480p_subblock", 1, 12, 21, 30, 52, 128, 64, 0.75,
                                 tile=(3, 4, 8), seed_base=1000, scorer=1, subblocks=4,
                                 budget_multiple=8),
    # the per-rank prologue shape of the packed video + audio benchmark:
    # 4,722 rows (= 2·3·787, so the grid is 2×3×787: the pages give rows,
    # not a grid, and the prologue's work per row does not depend on it),
    # 56 heads of 128 channels, RoPE over 96 of them (32 per axis)
    "h3_prologue": Workload("h3_prologue", 1, 56, 2, 3, 787, 128, 128, 0.0,
                            seed_base=7000, rope_split=(32, 32, 32)),
    # size limits: 4096 blocks per head (the plan's maximum; 262,144 tokens in
    # 64-token blocks), and 1538 blocks (1536 video + 2 of extra tokens, whose
    # rows and columns are always kept)
    "max4096": Workload("max4096", 1, 2, 16, 128, 128, 64, 64, 0.9, tile=(4, 4, 4),
                        seed_base=5000),
    "blocks1538": Workload("blocks1538", 1, 1, 24, 64, 128, 128, 128, 0.85,
                           flags=KEEP_SAME_FRAME, tile=(2, 8, 8), n_extra=256,
                           seed_base=6000),
}


def _interp_matrix(n_fine: int, n_coarse: int) -> np.ndarray:
    """Linear interpolation weights, align-corners: fine index i sits at
    coarse coordinate i·(n_coarse-1)/(n_fine-1)."""
    m = np.zeros((n_fine, n_coarse), dtype=np.float64)
    if n_fine == 1:
        m[0, 0] = 1.0
        return m
    x = np.arange(n_fine) * (n_coarse - 1) / (n_fine - 1)
    i0 = np.minimum(np.floor(x).astype(np.int64), n_coarse - 2)
    f = x - i0
    m[np.arange(n_fine), i0] = 1.0 - f
    m[np.arange(n_fine), i0 + 1] += f
    return m


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 → bf16 bit patterns, nearest with ties to even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(wl: Workload, stream: int, tensor: int, b: int, h: int) -> np.random.Generator:
    ss = np.random.SeedSequence([wl.seed_base + stream, tensor, b, h])
    return np.random.Generator(np.random.PCG64(ss))


def head_field(wl: Workload, tensor: int, b: int, h: int) -> np.ndarray:
    """bf16 bits [N, d] of one (tensor, batch, head), raster token order."""
    rng = _rng(wl, tensor, tensor, b, h)
    coarse = rng.standard_normal((2, 4, 4, wl.d))
    noise = rng.standard_normal((wl.T, wl.Hh, wl.W, wl.d), dtype=np.float32)
    mt = _interp_matrix(wl.T, 2)
    mh = _interp_matrix(wl.Hh, 4)
    mw = _interp_matrix(wl.W, 4)
    g = np.einsum("wc,abcd->abwd", mw, coarse)
    g = np.einsum("hb,abwd->ahwd", mh, g)
    g = np.einsum("ta,ahwd->thwd", mt, g).astype(np.float32)
    g += np.float32(0.5) * noise
    out = np.empty((wl.N, wl.d), dtype=np.uint16)
    out[: wl.n_video] = f32_to_bf16_bits(g.reshape(wl.n_video, wl.d))
    if wl.n_extra:
        re = _rng(wl, _STREAM_EXTRA, tensor, b, h)
        out[wl.n_video:] = f32_to_bf16_bits(
            re.standard_normal((wl.n_extra, wl.d), dtype=np.float32))
    return out


def full_tensor(wl: Workload, tensor: int, threads: int | None = None) -> np.ndarray:
    """bf16 bits [B, N, H, d] of one tensor (heads generated in parallel)."""
    out = np.empty((wl.B, wl.N, wl.H, wl.d), dtype=np.uint16)
    jobs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    if threads is None:
        threads = max(1, min(16, len(os.sched_getaffinity(0))))

    def work(bh):
        b, h = bh
        out[b, :, h, :] = head_field(wl, tensor, b, h)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, jobs))
    return out


def norm_weights(wl: Workload):
    """RMSNorm weights (wq, wk), float32 [H, d].

    Ones, except where the workload asks for a per-head attention
    temperature τ_h ~ U[0.5, 2]: then wq[h, :] = 1/τ_h, which scales the
    head's logits by 1/τ_h (a scale on the raw input would be undone by the
    normalisation).
    """
    wq = np.ones((wl.H, wl.d), dtype=np.float32)
    wk = np.ones((wl.H, wl.d), dtype=np.float32)
    if wl.temperature:
        rng = _rng(wl, _STREAM_TAU, 0, 0, 0)
        tau = rng.uniform(0.5, 2.0, size=wl.H)
        wq[:] = (1.0 / tau).astype(np.float32)[:, None]
    return wq, wk


def custom(name: str, B: int, H: int, T: int, Hh: int, W: int, d: int, block: int,
           sparsity: float, flags: int = 0, tile=(0, 0, 0), n_extra: int = 0,
           temperature: bool = False, seed_base: int = 9000,
           rope_split=(0, 0, 0), scorer: int = 0, subblocks: int = 0,
           budget_multiple: int = 0, rope_theta: float = 0.0, eps: float = 0.0) -> Workload:
    """An ad-hoc workload (tests use these for small ragged shapes)."""
    return Workload(name, B, H, T, Hh, W, d, block, sparsity, flags, tuple(tile),
                    n_extra, temperature, seed_base, tuple(rope_split), scorer, subblocks,
                    budget_multiple, rope_theta, eps)
