"""liblcsa from plain C: a C99 program that includes only include/lcsa.h and
links liblcsa.so is compiled with gcc -Werror and run on the host (the plan
functions need no GPU); its output must match the oracle's geometry.  The
header must also compile as C++ and declare nothing a C compiler rejects."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import lcsa_inputs as li
import oracle

lcsa = pytest.importorskip("block_sparse_attention_lcsa_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "plan_example.c")
INC = os.path.join(ROOT, "include")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("c_abi") / "plan_example")
    libdir = os.path.dirname(lcsa.lib_path())
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC, SRC,
                        "-L", libdir, "-llcsa", f"-Wl,-rpath,{libdir}", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, desc):
    args = [str(desc[k]) for k in ("batch", "heads", "grid_h", "grid_w", "q_frames", "cached_frames",
                                    "kv_ratio", "local_range")] + [repr(float(desc["topk_ratio"]))]
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=60)
    out = {}
    for line in r.stdout.splitlines():
        key, _, val = line.partition(" ")
        out[key] = val
    return r.returncode, out


@pytest.mark.parametrize("name", ["first_768x1280", "stream_768x1280", "first_768x1408",
                                  "first_2048x3840"])
def test_c_program_plans_match_oracle(program, name):
    desc = li.CONFIGS[name]
    rc, out = _run(program, desc)
    assert rc == 0, out
    g = oracle.geometry(desc)
    assert int(out["abi"]) == lcsa.abi_version()
    assert (int(out["kv_frames"]), int(out["nqb"]), int(out["nkb"]), int(out["k"])) == \
        (g.kv_frames, g.nqb, g.nkb, g.k)
    assert (int(out["block_h"]), int(out["block_w"])) == (g.block_h, g.block_w)
    counts = np.array([min(g.k, len(oracle.window(g, qb))) for qb in range(g.nqb)], dtype=np.int64)
    rp = np.concatenate([[0], np.cumsum(np.tile(counts, g.batch * g.heads))])
    assert int(out["rows"]) == len(rp) - 1 and int(out["nnz"]) == int(rp[-1])
    h = 0
    for x in rp.tolist():
        h = (h * 1000003 + x) % (1 << 64)
    assert int(out["row_ptr_hash"]) == h
    assert [int(x) for x in out["window0"].split()] == oracle.window(g, 0).tolist()
    assert out["status_string"].strip() != ""
    assert int(out["reuse_without_tau"]) == 1 and int(out["steady_without_kth"]) == 1   # NULL


def test_c_program_reports_errors(program):
    bad = dict(li.CONFIGS["first_768x1280"], grid_w=84)          # 84 is not tileable by 16 or 8
    rc, out = _run(program, bad)
    assert rc == 1 and out["error"].split()[0] == "3"             # LCSA_ERR_SHAPE


def test_header_compiles_as_cpp(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    src = tmp_path / "h.cpp"
    src.write_text('#include "lcsa.h"\nint main() { lcsa_desc d{}; (void)d; return lcsa_abi_version() > 0 ? 0 : 1; }\n')
    r = subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-fsyntax-only", "-I", INC, str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
