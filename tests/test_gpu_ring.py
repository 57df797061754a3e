"""Streaming KV storage through the C ABI: a frame ring for K/V and an
incremental pooled-K cache (lcsa_select_ring / lcsa_attend_ring).

The ring path computes the same function as the contiguous path on the KV
window, with the same kernels and the same arithmetic order, so its results
must be bitwise equal to the contiguous call; one chunk is also checked
against the float64 oracle.  A chunk sequence (first chunk of 6 latent
frames, then 2-frame chunks with kv_ratio 3) exercises the cache: later
chunks pool only their new frames and reuse the cached pooled K of the
older ones."""
import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle
from gpu_util import (bf16_to_np, check_mask, compare_output, device_qkv, say, to_device_bf16)

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


def _frame_tokens(desc):
    return desc["grid_h"] * desc["grid_w"]


def _to_ring(x, frames, slots, frame_slot, ft, ring=None):
    """Copy window frames of x [B, frames*ft, H, D] into ring slots."""
    B, _, H, D = x.shape
    if ring is None:
        ring = torch.zeros((B, slots * ft, H, D), dtype=x.dtype, device=x.device)
    for t in range(frames):
        s = frame_slot[t]
        ring[:, s * ft:(s + 1) * ft] = x[:, t * ft:(t + 1) * ft]
    return ring


def _nan_cache(plan, slots):
    return torch.full((lcsa.kcache_bytes(plan, slots) // 8,), float("nan"), dtype=torch.float64,
                      device="cuda")


@pytest.mark.parametrize("name", ["small_edges", "small_16x8", "tiny", "stream_768x1280"])
def test_ring_equals_contiguous(name):
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    kvf = plan.info["kv_frames"]
    ft = _frame_tokens(desc)
    slots = kvf + 3
    rng = np.random.default_rng(7)
    frame_slot = rng.permutation(slots)[:kvf].tolist()
    ring = lcsa.kv_ring(slots, frame_slot)
    k_ring = _to_ring(k, kvf, slots, frame_slot, ft)
    v_ring = _to_ring(v, kvf, slots, frame_slot, ft)
    kcache = _nan_cache(plan, slots)
    say(f"  {name}: kv_frames {kvf}, ring slots {slots}, frame_slot {frame_slot}")

    rp, ci, sc = lcsa.select(plan, q, k, return_scores=True)
    rp2, ci2, sc2 = lcsa.select_ring(plan, q, k_ring, ring, kvf, kcache, return_scores=True)
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    o2, lse2 = lcsa.attend_ring(plan, q, k_ring, v_ring, ring, rp2, ci2, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2)
    assert torch.equal(sc, sc2)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_ring_streaming_chunks():
    """First chunk of 6 frames, then two 2-frame chunks over a 6-slot ring; the
    later chunks pool only their 2 new frames."""
    base = dict(li.CONFIGS["small_edges"], cached_frames=0, kv_ratio=0.0, q_frames=10, topk=8)
    video = li.generate(base, seed=11)                 # Q, K, V of latent frames 0..9
    ft = _frame_tokens(base)
    qv, kv, vv = (to_device_bf16(x) for x in (video.q, video.k, video.v))
    slots = 6
    k_ring = v_ring = None
    kcache = None
    chunks = [(0, 6, 0), (6, 2, 4), (8, 2, 4)]         # (first query frame, q_frames, cached)
    for c, (f0, nq, cached) in enumerate(chunks):
        desc = dict(base, q_frames=nq, cached_frames=cached, kv_ratio=3.0)
        plan = lcsa.Plan.from_desc(desc)
        kvf = plan.info["kv_frames"]
        w0 = f0 + nq - kvf                             # first window frame (absolute)
        frame_slot = [(w0 + t) % slots for t in range(kvf)]
        ring = lcsa.kv_ring(slots, frame_slot)
        if kcache is None:
            kcache = _nan_cache(plan, slots)
        # the producer writes only this chunk's new frames into the ring
        new = nq if c > 0 else kvf
        k_new = kv[:, (f0 + nq - new) * ft:(f0 + nq) * ft]
        v_new = vv[:, (f0 + nq - new) * ft:(f0 + nq) * ft]
        k_ring = _to_ring(k_new, new, slots, frame_slot[kvf - new:], ft, k_ring)
        v_ring = _to_ring(v_new, new, slots, frame_slot[kvf - new:], ft, v_ring)
        q = qv[:, f0 * ft:(f0 + nq) * ft].contiguous()
        k_win = kv[:, w0 * ft:(w0 + kvf) * ft].contiguous()
        v_win = vv[:, w0 * ft:(w0 + kvf) * ft].contiguous()
        say(f"  chunk {c}: query frames {f0}..{f0 + nq - 1}, window {w0}..{w0 + kvf - 1}, "
            f"slots {frame_slot}, pooled new frames {new}")

        rp2, ci2, sc2 = lcsa.select_ring(plan, q, k_ring, ring, new, kcache, return_scores=True)
        o2 = lcsa.attend_ring(plan, q, k_ring, v_ring, ring, rp2, ci2)
        rp, ci, sc = lcsa.select(plan, q, k_win, return_scores=True)
        o = lcsa.attend(plan, q, k_win, v_win, rp, ci)
        torch.cuda.synchronize()
        assert torch.equal(rp, rp2) and torch.equal(ci, ci2) and torch.equal(sc, sc2)
        assert torch.equal(o, o2)
        if c == 1:
            g = oracle.geometry(desc)
            qf = li.bf16_bits_to_f64(video.q[:, f0 * ft:(f0 + nq) * ft])
            kf = li.bf16_bits_to_f64(video.k[:, w0 * ft:(w0 + kvf) * ft])
            vf = li.bf16_bits_to_f64(video.v[:, w0 * ft:(w0 + kvf) * ft])
            rp_ref, ci_ref, s_ref = oracle.select(g, qf, kf)
            check_mask(g, rp_ref, ci_ref, s_ref, rp2.cpu().numpy(), ci2.cpu().numpy())
            o_ref, _ = oracle.attend(g, qf, kf, vf, rp2.cpu().numpy().astype(np.int64),
                                     ci2.cpu().numpy().astype(np.int64))
            compare_output(bf16_to_np(o2), o_ref, "ring chunk 1 vs oracle")
