"""The host planner built with AddressSanitizer and UndefinedBehaviorSanitizer.

plan_host.cpp is pure C++ (no HIP): every descriptor the library accepts goes
through it before any device work.  tests/asan_plan.cpp drives it over the
measured video shapes, a seeded spread of 400 descriptors over every option,
and one descriptor per class of invalid input; the sanitizers stop the
process at the first out-of-bounds access, use after free, leak, signed
overflow or other undefined behaviour.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def _compiler():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    return cxx


def test_planner_under_sanitizers(tmp_path):
    cxx = _compiler()
    exe = str(tmp_path / "asan_plan")
    r = subprocess.run([cxx, "-std=c++17", "-O1", "-g", *SAN, "-Wall", "-Wextra", "-Werror",
                        os.path.join(ROOT, "tests", "asan_plan.cpp"),
                        os.path.join(ROOT, "block_sparse_attention_qk_amd", "csrc", "plan_host.cpp"),
                        "-o", exe], capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("no sanitizer runtime for g++")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    words = r.stdout.split()
    assert words[0] == "ok", r.stdout
    accepted, refused = int(words[1]), int(words[2])
    assert accepted == 406 and refused == 23, r.stdout
