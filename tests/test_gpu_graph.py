"""Select and attend captured in a HIP graph (torch.cuda.CUDAGraph on ROCm)
and replayed.

Every device operation of the path is a kernel launch whose arguments are
passed by value; the entry points make no host synchronisation, allocation
or memset.  A captured chunk therefore replays the same computation on
whatever its static buffers hold.  Each replay here is compared bitwise with
eager calls on the same inputs, with eager work and synchronisations between
the replays.  The frame-ring case captures one graph per ring phase (the
frame-to-slot table is part of the kernel arguments) and replays them over a
stream of chunks."""
import numpy as np
import pytest
import torch

import lcsa_inputs as li
from gpu_util import check_mask, device_qkv, oracle_select, say, to_device_bf16

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    say(f"[gpu] done  {request.node.nodeid}")


def _capture(fn):
    """Run fn twice eagerly on a side stream, then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


@pytest.mark.parametrize("name", ["small_edges", "stream_768x1280"])
def test_graph_replay_matches_eager(name):
    desc, q0, k0, v0 = device_qkv(name, seed=0)
    plan = lcsa.Plan.from_desc(desc)
    inf = plan.info
    q, k, v = q0.clone(), k0.clone(), v0.clone()
    sel_ws = torch.empty(max(int(inf["select_workspace_bytes"]), 256), dtype=torch.uint8,
                         device="cuda")
    att_ws = torch.empty(int(inf["attend_workspace_bytes"]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def chunk():
        rp, ci = lcsa.select(plan, q, k, workspace=sel_ws)
        _, lse = lcsa.attend(plan, q, k, v, rp, ci, out=out, return_lse=True, workspace=att_ws)
        return rp, ci, lse

    g, (rp_g, ci_g, lse_g) = _capture(chunk)
    say(f"  {name}: rows {inf['rows']}, nnz {inf['nnz']}, captured select + attend")

    for seed in (1, 2, 0):
        _, qs, ks, vs = device_qkv(name, seed=seed)
        q.copy_(qs)
        k.copy_(ks)
        v.copy_(vs)
        g.replay()
        torch.cuda.synchronize()
        got_ci, got_out, got_lse = ci_g.clone(), out.clone(), lse_g.clone()
        # eager on the same inputs, into fresh buffers
        rp_e, ci_e = lcsa.select(plan, qs, ks)
        out_e, lse_e = lcsa.attend(plan, qs, ks, vs, rp_e, ci_e, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(rp_g, rp_e), f"seed {seed}: row_ptr differs"
        assert torch.equal(got_ci, ci_e), f"seed {seed}: col_idx differs"
        assert torch.equal(got_out.view(torch.int16), out_e.view(torch.int16)), f"seed {seed}: O differs"
        assert torch.equal(got_lse, lse_e), f"seed {seed}: LSE differs"
        if seed == 0:
            gg, rp_ref, ci_ref, s_ref = oracle_select(name, 0)
            mism, ties = check_mask(gg, rp_ref, ci_ref, s_ref, rp_g.cpu().numpy(),
                                    got_ci.cpu().numpy())
            say(f"  replay on seed 0: {len(mism)} rows differ from the oracle, all near-ties")
        say(f"  replay on seed {seed}: bitwise equal to eager")


def test_graph_streaming_ring_phases():
    """A first chunk of 6 latent frames eagerly, then 2-frame chunks over a
    6-slot ring replayed from one graph per ring phase (3 phases, each used
    twice).  Each replay pools only its 2 new frames into the pooled-K cache."""
    base = dict(li.CONFIGS["small_edges"], cached_frames=0, kv_ratio=0.0, q_frames=18, topk=8)
    video = li.generate(base, seed=5)                  # latent frames 0..17
    ft = base["grid_h"] * base["grid_w"]
    qv, kv, vv = (to_device_bf16(x) for x in (video.q, video.k, video.v))
    B, _, H, D = qv.shape
    slots = 6
    k_ring = torch.zeros((B, slots * ft, H, D), dtype=qv.dtype, device="cuda")
    v_ring = torch.zeros_like(k_ring)

    first = lcsa.Plan.from_desc(dict(base, q_frames=6, cached_frames=0, kv_ratio=3.0))
    kcache = torch.full((lcsa.kcache_bytes(first, slots) // 8,), float("nan"),
                        dtype=torch.float64, device="cuda")
    k_ring[:, :6 * ft] = kv[:, :6 * ft]
    v_ring[:, :6 * ft] = vv[:, :6 * ft]
    ring0 = lcsa.kv_ring(slots, list(range(6)))
    lcsa.select_ring(first, qv[:, :6 * ft].contiguous(), k_ring, ring0, 6, kcache)

    plan = lcsa.Plan.from_desc(dict(base, q_frames=2, cached_frames=4, kv_ratio=3.0))
    assert plan.info["kv_frames"] == 6
    q = torch.empty((B, 2 * ft, H, D), dtype=qv.dtype, device="cuda")
    out = torch.empty_like(q)
    att_ws = torch.empty(int(plan.info["attend_workspace_bytes"]), dtype=torch.uint8,
                         device="cuda")
    sel_ws = torch.empty(max(int(plan.info["select_workspace_bytes"]), 256), dtype=torch.uint8,
                         device="cuda")

    # chunk c >= 1 has query frames 6+2(c-1) .. +1 and window 2c .. 2c+5, with
    # window frame t in slot (2c + t) % 6: phase (c - 1) % 3
    graphs = []
    for ph in range(3):
        c = ph + 1
        ring = lcsa.kv_ring(slots, [(2 * c + t) % slots for t in range(6)])
        # the captures run on the current ring contents; only the replays
        # below are checked, each after its chunk's frames are in place
        saved = kcache.clone()

        def chunk(ring=ring):
            rp, ci = lcsa.select_ring(plan, q, k_ring, ring, 2, kcache, workspace=sel_ws)
            lcsa.attend_ring(plan, q, k_ring, v_ring, ring, rp, ci, out=out, workspace=att_ws)
            return rp, ci

        graphs.append(_capture(chunk))
        kcache.copy_(saved)

    for c in range(1, 7):
        f0, w0 = 6 + 2 * (c - 1), 2 * c
        frame_slot = [(w0 + t) % slots for t in range(6)]
        # the producer writes the chunk's 2 new frames into their slots
        for t in (4, 5):
            s, f = frame_slot[t], w0 + t
            k_ring[:, s * ft:(s + 1) * ft] = kv[:, f * ft:(f + 1) * ft]
            v_ring[:, s * ft:(s + 1) * ft] = vv[:, f * ft:(f + 1) * ft]
        q.copy_(qv[:, f0 * ft:(f0 + 2) * ft])
        g, (rp_g, ci_g) = graphs[(c - 1) % 3]
        g.replay()
        torch.cuda.synchronize()
        got_ci, got_out = ci_g.clone(), out.clone()

        k_win = kv[:, w0 * ft:(w0 + 6) * ft].contiguous()
        v_win = vv[:, w0 * ft:(w0 + 6) * ft].contiguous()
        qc = q.clone()
        rp_e, ci_e = lcsa.select(plan, qc, k_win)
        out_e = lcsa.attend(plan, qc, k_win, v_win, rp_e, ci_e)
        torch.cuda.synchronize()
        assert torch.equal(rp_g, rp_e) and torch.equal(got_ci, ci_e), f"chunk {c}: mask differs"
        assert torch.equal(got_out.view(torch.int16), out_e.view(torch.int16)), f"chunk {c}: O differs"
        say(f"  chunk {c}: window frames {w0}..{w0 + 5}, slots {frame_slot}, phase graph "
            f"{(c - 1) % 3}: bitwise equal to the contiguous eager path")
