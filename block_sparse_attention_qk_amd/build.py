"""Build libsva.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_qk_amd.build            # libsva.so
    python -m block_sparse_attention_qk_amd.build --debug    # libsva_debug.so

Every call recompiles every source (the objects go to ``_build/`` next to
this file, the library to ``libsva.so``).  The debug build compiles the same
sources with -DSVA_DEBUG (device-side index checks reported through the
plan's debug word, see sva_debug_flags) into ``_build_debug/`` and
``libsva_debug.so``.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsva.so")
DEBUG_OUT_DIR = os.path.join(PKG, "_build_debug")
DEBUG_LIB = os.path.join(PKG, "libsva_debug.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-result",
]


# per-source code generation options
EXTRA = {
    # MFMA results in VGPRs: the softmax reads S with VALU ops, and the
    # default AGPR form made the register allocator shuttle the Q operands
    # and S tiles between AGPRs and VGPRs every stage
    # The scheduler's own register-pressure trackers: bit-identical code
    # semantics, 1-2.5 % faster on the 64-token-block kernels (sparse 480p
    # 1.60 -> 1.56 ms), unchanged at 128-token blocks.
    "k_attention.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-use-amdgpu-trackers"],
}


def flag_signature(name: str) -> str:
    """The compiler options of source `name`, without the include path (so
    the text is the same on every machine): what a kernel's code depends on
    besides its source."""
    common, skip = [], False
    for a in COMMON:
        if skip:
            skip = False
        elif a == "-I":
            skip = True
        else:
            common.append(a)
    return " ".join(common + EXTRA.get(name, []))


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_OUT_DIR if debug else OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *(["-DSVA_DEBUG"] if debug else []),
           *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # surface real warnings (the host pass always notes the device-only
    # target feature; that line is harmless)
    warn = [ln for ln in r.stderr.splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln]
    if warn:
        print(f"warnings in {os.path.basename(src)}:\n" + "\n".join(warn))
    return obj


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _link(objs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False, debug: bool = False) -> str:
    out_dir, lib = (DEBUG_OUT_DIR, DEBUG_LIB) if debug else (OUT_DIR, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), srcs))
    return _link(objs, lib, verbose)


def build_all(verbose: bool = False) -> tuple:
    """Both libraries, their objects compiled in one pool (the slowest
    source of each build overlaps the other's)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(DEBUG_OUT_DIR, exist_ok=True)
    srcs = _sources()
    # the largest sources first, so they do not trail the pool
    jobs = sorted([(src, dbg) for dbg in (False, True) for src in srcs],
                  key=lambda j: -os.path.getsize(j[0]))
    with ThreadPoolExecutor(8) as ex:
        done = dict(zip(jobs, ex.map(lambda j: _compile(*j), jobs)))
    rel = _link([done[(src, False)] for src in srcs], LIB, verbose)
    dbg = _link([done[(src, True)] for src in srcs], DEBUG_LIB, verbose)
    return rel, dbg


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
