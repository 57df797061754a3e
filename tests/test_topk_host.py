"""The select kernel's per-row top-k (csrc/topk_wave.h) run on the host.

tests/host/topk_wave_host.cpp emulates a wave with 64 threads and runs the
same selection code the kernel runs, built with g++ under the undefined-
behaviour and address sanitizers (any report aborts).  Its cases: every score
of a window equal (zero pooled query, identical pooled keys, signed zeros,
-inf), ties at the k-th score, the k-th and (k+1)-th scores one ulp apart, a
single candidate, random and denormal scores, at every compiled candidate
width; each must equal a brute-force stable sort by (score descending, index
ascending) and fill exactly its row's keep positions.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_sparse_attention_lcsa_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_topk_wave_on_host_under_sanitizers(tmp_path):
    exe = str(tmp_path / "topk_wave_host")
    build = subprocess.run(
        ["g++", "-std=c++20", "-O1", "-g", "-fsanitize=undefined,address",
         "-fno-sanitize-recover=all", "-pthread", "-Wall", "-Wno-unknown-pragmas", "-Werror",
         "-I", CSRC, os.path.join(HERE, "host", "topk_wave_host.cpp"), "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stdout + build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "runtime error" not in out and " 0 failed" in out, out[-3000:]
