"""The debug library (device-side index checks, -DSVA_DEBUG) on the GPU.

tests/_debug_check.py runs, in a process of its own, the fused and the staged
step of small cases (ragged tails, 64- and 128-token blocks, dense plans,
SubBlock ranking, compensation, split rows, a single block, sparsity 0.99)
and of four named workloads at full size through the release and the debug
library: no check may fire (the plan's debug word stays zero), every output
must equal the release library's bit for bit, and the self-test kernel must
set SVA_DEBUG_SELF, cleared on reading.
"""

import os
import subprocess
import sys

import pytest

import block_sparse_attention_qk_amd as S

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_debug_library_checks_stay_silent_and_outputs_match():
    assert os.path.exists(S.DEBUG_LIB_PATH), "libsva_debug.so is not built"
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "_debug_check.py"), "full"],
                       capture_output=True, text=True, timeout=600)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "debug check passed" in r.stdout
