"""lcsa_select_noalloc through the C ABI: the workspace-free selection (its
pooled vectors in the library's per-device scratch array) must give
lcsa_select's CSR and scores bit for bit, on two calls in a row, the second
with a smaller input, so that the second call runs on a scratch array that
holds the first call's larger contents."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import device_qkv, say

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)

GUARD = 1024
SENTINEL = 0x3C3C3C3C


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    say(f"[gpu] done  {request.node.nodeid}")


def _noalloc(plan, q, k):
    """lcsa_select_noalloc into guard-padded buffers; returns the CSR and
    scores, after checking nothing past their ends was written."""
    inf, d = plan.info, plan.desc
    rows, nnz = int(inf["rows"]), int(inf["nnz"])
    n_sc = d["batch"] * d["heads"] * inf["nqb"] * inf["nkb"]
    rp = torch.full((rows + 1 + GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
    ci = torch.full((nnz + GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
    sc = torch.full((n_sc + GUARD,), 7.0, dtype=torch.float64, device="cuda")
    qv, kv = lcsa.tensor_view(q), lcsa.tensor_view(k)
    st = lcsa._lib.lcsa_select_noalloc(plan.handle, ctypes.byref(qv), ctypes.byref(kv),
                                       rp.data_ptr(), ci.data_ptr(), sc.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0, lcsa._lib.lcsa_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(rp[rows + 1:] == SENTINEL) and torch.all(ci[nnz:] == SENTINEL)
    assert torch.all(sc[n_sc:] == 7.0)
    return rp[:rows + 1], ci[:nnz], sc[:n_sc].view(d["batch"], d["heads"], inf["nqb"], inf["nkb"])


def test_noalloc_equals_select_on_two_calls_second_smaller():
    for name in ("first_768x1280", "small_edges"):
        desc, q, k, _ = device_qkv(name)
        plan = lcsa.Plan.from_desc(desc)
        assert plan.info["select_workspace_bytes"] <= lcsa.SELECT_NOALLOC_MAX_BYTES
        rp, ci, sc = _noalloc(plan, q, k)
        rp_w, ci_w, sc_w = lcsa.select(plan, q, k, return_scores=True)
        torch.cuda.synchronize()
        say(f"  {name}: {plan.info['select_workspace_bytes']} scratch bytes, "
            f"{plan.info['nnz']} selected blocks")
        assert torch.equal(rp, rp_w) and torch.equal(ci, ci_w)
        assert torch.equal(sc, sc_w)


def test_noalloc_binding_and_size_limit():
    desc, q, k, _ = device_qkv("tiny")
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select_noalloc(plan, q, k)
    rp_w, ci_w = lcsa.select(plan, q, k)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp_w) and torch.equal(ci, ci_w)
    big = lcsa.Plan.from_desc(dict(desc, batch=2, heads=12, grid_h=128, grid_w=240, q_frames=6,
                                   block_t=0, block_h=0, block_w=0, local_range=11, topk=45))
    assert big.info["select_workspace_bytes"] > lcsa.SELECT_NOALLOC_MAX_BYTES
    with pytest.raises(lcsa.LcsaError) as ei:
        lcsa._check(lcsa._lib.lcsa_select_noalloc(big.handle, None, None, None, None, None, None),
                    "lcsa_select_noalloc")
    assert ei.value.name == "LCSA_ERR_WORKSPACE"


def test_noalloc_select_in_a_graph():
    """The callers the call is for: a chunk captured in a HIP graph with
    lcsa_select_noalloc into static CSR buffers, then attention, replayed on
    new inputs with eager calls between replays; each replay must equal
    eager lcsa_select + lcsa_attend on the same inputs bit for bit."""
    desc, q0, k0, v0 = device_qkv("stream_768x1280", seed=0)
    plan = lcsa.Plan.from_desc(desc)
    inf = plan.info
    q, k, v = q0.clone(), k0.clone(), v0.clone()
    rp = torch.empty(inf["rows"] + 1, dtype=torch.int32, device="cuda")
    ci = torch.empty(inf["nnz"], dtype=torch.int32, device="cuda")
    att_ws = torch.empty(int(inf["attend_workspace_bytes"]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def chunk():
        lcsa.select_noalloc(plan, q, k, row_ptr=rp, col_idx=ci)
        lcsa.attend(plan, q, k, v, rp, ci, out=out, workspace=att_ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            chunk()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chunk()
    torch.cuda.synchronize()
    for seed in (1, 2, 0, 1):
        _, qs, ks, vs = device_qkv("stream_768x1280", seed=seed)
        q.copy_(qs)
        k.copy_(ks)
        v.copy_(vs)
        g.replay()
        torch.cuda.synchronize()
        got_ci, got_out = ci.clone(), out.clone()
        rp_e, ci_e = lcsa.select(plan, qs, ks)
        out_e = lcsa.attend(plan, qs, ks, vs, rp_e, ci_e)
        torch.cuda.synchronize()
        assert torch.equal(rp, rp_e) and torch.equal(got_ci, ci_e), f"seed {seed}: CSR differs"
        assert torch.equal(got_out, out_e), f"seed {seed}: attention output differs"
        say(f"  replay on seed {seed}: CSR and output equal to eager calls")
