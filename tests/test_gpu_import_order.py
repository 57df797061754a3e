"""The binding works when it is imported before torch: it loads torch (and so
torch's HIP runtime) before liblcsa.so, so the process holds one HIP runtime.
Run in a fresh interpreter, where nothing else has loaded torch yet."""
import os
import subprocess
import sys

import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CODE = """
import sys
sys.path.insert(0, {root!r})
import block_sparse_attention_lcsa_amd as lcsa      # before torch, on purpose
import lcsa_inputs as li
import numpy as np
import torch
desc = li.CONFIGS["tiny"]
inp = li.generate(desc)
up = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
q, k, v = up(inp.q), up(inp.k), up(inp.v)
plan = lcsa.Plan.from_desc(desc)
rp, ci = lcsa.select(plan, q, k)
o = lcsa.attend(plan, q, k, v, rp, ci)
torch.cuda.synchronize()
assert torch.isfinite(o.float()).all()
print("ok", int(rp[-1]))
"""


def test_binding_imported_before_torch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("[gpu] start import-order check in a child interpreter")
    r = subprocess.run([sys.executable, "-c", CODE.format(root=ROOT)], capture_output=True,
                       text=True, timeout=180)
    say(f"[gpu] done  import-order check: rc {r.returncode}")
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.split()[0] == "ok"
