"""CPU check of the attention kernel's LDS stage-buffer schedule.

The attention kernel copies K and V stages of 32 keys into rotating LDS
buffers ahead of their use and synchronises its waves with a bare barrier
every BP stages, after a wait that leaves the copies of the latest
iterations in flight.  A wrong buffer count, copy lead or wait would let a
copy overwrite a buffer that another wave still reads, or let a wave read a
buffer before every wave's copy into it has landed: races that a GPU run
need not show.  This test takes the schedule's constants from the kernel
source and checks, for every iteration of rows of many lengths, that

  - every stage a wave reads was copied (by every wave) in an iteration
    whose copies had landed at a barrier that closed before the reading
    iteration began (read after write), and
  - every copy into a buffer is issued after a barrier that followed every
    wave's last read of the stage the buffer held before (write after read),

with waves free to run ahead of one another between barriers.  The model:
before the walk, K stages 0..KLEAD-1 and V stages 0..VLEAD-1 are copied, the
V buffer of "stage -1" is zeroed, every copy lands and the workgroup
synchronises; the first stage's scores then read K stage 0 (and, with two
stages per barrier, a barrier follows).  Iteration i copies K stage i+KLEAD
and V stage i+VLEAD, reads K stage i+1 (scores) and V stage i-1 (the
product), and, on a barrier iteration, waits until the copies of the
iterations up to i-X have landed and passes the barrier.  After the walk the
last product reads V stage n-1.  Copies past the end of the row are issued
(into buffers nobody reads) and count as writes; reads of stages past the
end are masked and not checked.

Schedules with a planted mistake (one buffer fewer, a longer lead, copies
left in flight at the barrier, the barrier after the first scores missing)
fail the same check, so it is not vacuous.
"""

import os
import re
from dataclasses import dataclass, replace

import pytest

from block_sparse_attention_qk_amd import build as B

SRC = os.path.join(B.CSRC, "k_attention.hip")


@dataclass(frozen=True)
class Schedule:
    nbk: int          # K buffers
    nbv: int          # V buffers
    bp: int           # stages per barrier
    klead: int        # K copies run this many stages ahead
    vlead: int        # V copies run this many stages ahead
    x: int            # iterations whose copies may stay in flight at a barrier
    first_barrier: bool   # a barrier right after the first stage's scores


def _source():
    with open(SRC) as f:
        return f.read()


def schedules_from_source():
    """The schedule of each block size, read off the kernel source.  Any
    change to the form of these lines fails here, so the model is updated
    together with the kernel."""
    s = _source()

    def per_blk(name):
        m = re.search(name + r"\(int, int blk\) \{ return blk == 64 \? (\d+) : (\d+); \}", s)
        assert m, f"{name} not found in the form the model expects"
        return {64: int(m.group(1)), 128: int(m.group(2))}

    nbk, nbv, bp = per_blk("attn_k_buffers"), per_blk("attn_v_buffers"), per_blk("attn_barrier_period")
    m = re.search(r"constexpr int KLEAD = NBK - (\d+);", s)
    assert m
    kl = int(m.group(1))
    m = re.search(r"constexpr int VLEAD = BP == 1 \? NBV - (\d+) : (\d+);", s)
    assert m
    vl1, vl2 = int(m.group(1)), int(m.group(2))
    m = re.search(r"constexpr int kInFlight = BP == 1 \? \(NBK - (\d+) < NBV - (\d+) \? "
                  r"NBK - (\d+) : NBV - (\d+)\) \* 2 \* LPW : (\d+);", s)
    assert m and m.group(1) == m.group(3) and m.group(2) == m.group(4)
    a, b, x2 = int(m.group(1)), int(m.group(2)), int(m.group(5))
    # copies of one iteration: LPW of K, then LPW of V
    assert re.search(r"SVA_COPY_K\(kb8 \+ E\[ck / SPB\]\.off, ck % SPB, ck % NBK\);\s*"
                     r"SVA_COPY_V\(vb8 \+ E\[cv / SPB\]\.off, cv % SPB, cv % NBV\);", s)
    assert "const int ck = u + KLEAD, cv = u + VLEAD, cs = u + 1;" in s
    assert re.search(r"if \(BP == 1 \|\| \(u & 1\)\) \{\s*__builtin_amdgcn_s_waitcnt\(kWaitNext\);"
                     r"\s*__builtin_amdgcn_s_barrier\(\);", s)
    first = re.search(r"if \(BP == 2\) __builtin_amdgcn_s_barrier\(\);", s) is not None
    assert x2 % 2 == 0
    out = {}
    for blk in (64, 128):
        p = bp[blk]
        out[blk] = Schedule(
            nbk=nbk[blk], nbv=nbv[blk], bp=p, klead=nbk[blk] - kl,
            vlead=nbv[blk] - vl1 if p == 1 else vl2,
            x=min(nbk[blk] - a, nbv[blk] - b) if p == 1 else x2 // 2,
            first_barrier=first and p == 2)
    return out


def hazards(sch: Schedule, n: int):
    """Violations of the schedule for a row of n stages (n a multiple of the
    stages per block), as a list of strings; empty when it is safe."""
    # barriers: (iteration after which it stands, latest iteration whose
    # copies have landed when it is passed)
    bars = [(-2, -2)]                      # the synchronisation before the walk
    if sch.first_barrier:
        bars.append((-1, -2))
    for i in range(n):
        if sch.bp == 1 or i % 2 == 1:
            bars.append((i, i - sch.x))
    bad = []

    def visible_before(c, r):
        # a barrier standing after an iteration < r whose wait covered c
        return any(e < r and land >= c for e, land in bars)

    def barrier_between(r, c):
        # a barrier after iteration r (the read) and before iteration c
        return any(r <= e < c for e, _ in bars)

    def k_copy_iter(s):
        return -2 if s < sch.klead else s - sch.klead

    def v_copy_iter(s):
        return -2 if s < sch.vlead else s - sch.vlead

    def k_read_iter(s):
        return s - 1                      # scores of stage s in iteration s-1

    def v_read_iter(s):
        return s + 1                      # product of stage s in iteration s+1

    # read after write
    for s in range(n):
        r = k_read_iter(s)
        if not visible_before(k_copy_iter(s), r):
            bad.append(f"K stage {s} read in iteration {r} before its copy is visible")
    for s in range(-1, n):
        r = v_read_iter(s)
        c = -2 if s == -1 else v_copy_iter(s)   # stage -1: the zeroed buffer
        if not visible_before(c, r):
            bad.append(f"V stage {s} read in iteration {r} before its copy is visible")
    # write after read (every copy the loop issues, past the end included)
    for i in range(n):
        s = i + sch.klead
        prev = s - sch.nbk
        if 0 <= prev < n and not barrier_between(k_read_iter(prev), i):
            bad.append(f"K stage {s} copied in iteration {i} over stage {prev}, "
                       f"read in iteration {k_read_iter(prev)}")
        if prev >= n:
            pass                            # the previous occupant was never read
        s = i + sch.vlead
        prev = s - sch.nbv
        if -1 <= prev < n and not barrier_between(v_read_iter(prev), i):
            bad.append(f"V stage {s} copied in iteration {i} over stage {prev}, "
                       f"read in iteration {v_read_iter(prev)}")
    # every buffer holds one stage at a time: a lead no longer than the ring
    if sch.klead >= sch.nbk + 1 or sch.vlead >= sch.nbv:
        bad.append("copy lead longer than the buffer ring")
    return bad


def _lengths(blk):
    spb = blk // 32
    return [spb * e for e in range(1, 9)]


@pytest.mark.parametrize("blk", [64, 128])
def test_kernel_schedule_is_race_free(blk):
    sch = schedules_from_source()[blk]
    for n in _lengths(blk):
        assert hazards(sch, n) == [], (blk, sch, n)


def test_schedule_constants_read_from_source():
    s = schedules_from_source()
    # what the kernel's comments state: four and four buffers with one
    # barrier per two stages at 128-token blocks, three and two with a
    # barrier per stage at 64-token blocks
    assert (s[128].nbk, s[128].nbv, s[128].bp) == (4, 4, 2)
    assert (s[64].nbk, s[64].nbv, s[64].bp) == (3, 2, 1)
    assert s[128].x == 0 and s[128].first_barrier


@pytest.mark.parametrize("mistake", ["v_lead", "in_flight", "no_first_barrier", "k_buffer",
                                     "bp1_v_buffer", "bp1_in_flight"])
def test_planted_schedule_mistakes_are_caught(mistake):
    s = schedules_from_source()
    sch = {
        "v_lead": replace(s[128], vlead=2),              # V copied two stages ahead
        "in_flight": replace(s[128], x=1),                # last copies left in flight
        "no_first_barrier": replace(s[128], first_barrier=False),
        "k_buffer": replace(s[128], nbk=3, klead=2),      # one K buffer fewer
        "bp1_v_buffer": replace(s[64], nbv=1, vlead=0),   # one V buffer at a barrier per stage
        "bp1_in_flight": replace(s[64], x=1),
    }[mistake]
    blk = 128 if not mistake.startswith("bp1") else 64
    assert any(hazards(sch, n) for n in _lengths(blk)), mistake
