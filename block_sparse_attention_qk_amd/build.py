"""Build libsva.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_qk_amd.build

Every call recompiles every source (the objects go to ``_build/`` next to
this file, the library to ``libsva.so``).
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
    "k_attention.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
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


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
