"""CPU check of the attention kernel's compiled code for gfx950.

The attention kernel issues its global -> LDS copies from inline asm that
writes M0 (the LDS destination) right before each copy.  The compiler is
told M0 is clobbered but does not honour that clobber for M0, so the copies
are correct only while the compiler itself neither keeps a value in M0 nor
emits an instruction that reads M0 implicitly.  This test compiles the
kernel to assembly (the same options as the library build) and checks
exactly that: every mention of M0 lies inside one of the kernel's own asm
blocks, each block is "write M0; s_nop 0; global_load_lds_dwordx4", and no
instruction that reads M0 implicitly appears anywhere else.  A compiler
change that breaks the assumption fails here, on the CPU, before a run.
"""

import os
import re
import shutil
import subprocess

import pytest

from block_sparse_attention_qk_amd import build as B

SRC = os.path.join(B.CSRC, "k_attention.hip")
# instructions that read M0 implicitly on this target
_M0_READERS = re.compile(r"^\s*(s_sendmsg|s_movrel|v_movrel|ds_gws|ds_ordered|"
                         r"buffer_load_\w*lds|global_load_lds|s_ttracedata|v_interp)")


@pytest.fixture(scope="module")
def attention_asm(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    out = str(tmp_path_factory.mktemp("asm") / "k_attention.s")
    cmd = [B.HIPCC, "-x", "hip", *B.COMMON, *B.EXTRA.get("k_attention.hip", []),
           "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    with open(out) as f:
        return f.read().splitlines()


def _code(line):
    return line.split(";")[0].strip()


def test_m0_only_in_the_copy_sequences(attention_asm):
    lines = attention_asm
    in_asm = False
    block = []
    blocks = 0
    for ln in lines:
        s = ln.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm, block = True, []
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            code = [c for c in block if c]
            if any(re.search(r"\bm0\b", c) for c in code):
                blocks += 1
                assert len(code) == 3, code
                assert re.match(r"s_(mov_b32|add_u32) m0, ", code[0]), code
                assert code[1] == "s_nop 0", code
                assert code[2].startswith("global_load_lds_dwordx4 "), code
            continue
        c = _code(ln)
        if in_asm:
            block.append(c)
            continue
        if not c or c.startswith("."):
            continue
        assert not re.search(r"\bm0\b", c), f"compiler-generated use of M0: {c}"
        assert not _M0_READERS.match(c), f"instruction reading M0 outside the copies: {c}"
    assert blocks > 100          # every instantiation's copies were seen
