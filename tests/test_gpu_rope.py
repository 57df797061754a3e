"""Rotary embedding fused into selection (lcsa_select_rope,
lcsa_select_ring_rope) against the float64 oracle, through the C ABI.

The turned Q and K must equal the oracle's bit for bit (each value is the
exact product rounded once, on both sides).  The CSR selected on them must
match the oracle's selection on the turned tensors up to near-ties, and
lcsa_select on the turned tensors must give the same CSR and scores bitwise
(pooling sums exact values in both).  Attention on the turned tensors is
checked against the oracle on the whole tensor.  The ring variant is
checked against the contiguous one over a stream of chunks."""
import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle
from gpu_util import bf16_to_np, check_mask, compare_output, device_qkv, host_inputs, say, to_device_bf16
from oracle.parallel import OraclePool

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


def _tables(desc, frame_offset=0, pairs=(22, 21, 21)):
    t = li.rope_tables(desc, pairs=pairs, frame_offset=frame_offset)
    host = oracle.RopeTables(t=t["t"], h=t["h"], w=t["w"])
    dev = lcsa.rope(*(torch.from_numpy(t[a]).cuda() for a in ("t", "h", "w")))
    return host, dev


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def _f64_to_bits(x: np.ndarray) -> np.ndarray:
    return li.f32_to_bf16_bits(x.astype(np.float32))     # exact: the values are bf16


@pytest.mark.parametrize("name,pairs", [("tiny", (22, 21, 21)), ("small_edges", (22, 21, 21)),
                                        ("small_16x8", (0, 32, 32)), ("stream_768x1280", (22, 21, 21)),
                                        ("first_768x1280", (22, 21, 21))])
def test_select_rope_matches_oracle(name, pairs):
    desc, q, k, v = device_qkv(name)
    _, inp = host_inputs(name)
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    tab, dtab = _tables(desc, frame_offset=3, pairs=pairs)
    q_rot, k_rot, rp, ci, sc = lcsa.select_rope(plan, q, k, dtab, return_scores=True)
    o, lse = lcsa.attend(plan, q_rot, k_rot, v, rp, ci, return_lse=True)
    torch.cuda.synchronize()

    qr = oracle.rope_q(g, li.bf16_bits_to_f64(inp.q), tab)
    kr = oracle.rope_k(g, li.bf16_bits_to_f64(inp.k), tab)
    assert np.array_equal(_bits(q_rot), _f64_to_bits(qr)), "turned Q differs from the oracle"
    assert np.array_equal(_bits(k_rot), _f64_to_bits(kr)), "turned K differs from the oracle"
    say(f"  {name}: turned Q and K bitwise equal to the oracle")

    rp_ref, ci_ref, s_ref = oracle.select(g, qr, kr)
    mism, ties = check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    say(f"  mask: {len(mism)} rows differ from the oracle, {len(ties)} near-ties")
    fin = np.isfinite(s_ref)
    s_gpu = sc.cpu().numpy()
    assert np.array_equal(np.isfinite(s_gpu), fin)
    assert np.max(np.abs(s_gpu[fin] - s_ref[fin])) <= 1e-12 * max(1.0, np.abs(s_ref[fin]).max())

    # select on the turned tensors: same pooled values, so the same CSR and scores
    rp2, ci2, sc2 = lcsa.select(plan, q_rot, k_rot, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2) and torch.equal(sc, sc2)

    rp_h, ci_h = rp.cpu().numpy().astype(np.int64), ci.cpu().numpy().astype(np.int64)
    if g.q_tokens * g.heads <= 8192:
        o_ref, lse_ref = oracle.attend(g, qr, kr, li.bf16_bits_to_f64(inp.v), rp_h, ci_h)
    else:
        # the turned tensors hold bf16 values exactly, so their bit patterns
        # are the oracle pool's inputs; every row, spread over heads
        with OraclePool(desc, _f64_to_bits(qr), _f64_to_bits(kr), inp.v) as pool:
            o_ref, lse_ref, _ = pool.attend(rp_h, ci_h)
    compare_output(bf16_to_np(o), o_ref, f"{name} attend on turned Q, K (whole tensor)")
    assert float(np.abs(lse.cpu().numpy() - lse_ref).max()) <= 2e-3


def test_select_rope_streaming_pass_4k():
    """At the 184320-token chunk Q and K exceed the memory-side cache, so the
    pooling pass runs with non-temporal loads (its other form): the turned
    Q and K must still equal the oracle's bit for bit, and lcsa_select on
    them must give the rotary select's CSR and scores bitwise."""
    name = "first_2048x3840"
    desc, q, k, _ = device_qkv(name)
    _, inp = host_inputs(name)
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    tab, dtab = _tables(desc)
    q_rot, k_rot, rp, ci, sc = lcsa.select_rope(plan, q, k, dtab, return_scores=True)
    rp2, ci2, sc2 = lcsa.select(plan, q_rot, k_rot, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2) and torch.equal(sc, sc2)
    qr = oracle.rope_q(g, li.bf16_bits_to_f64(inp.q), tab)
    assert np.array_equal(_bits(q_rot), _f64_to_bits(qr)), "turned Q differs from the oracle"
    del qr
    kr = oracle.rope_k(g, li.bf16_bits_to_f64(inp.k), tab)
    assert np.array_equal(_bits(k_rot), _f64_to_bits(kr)), "turned K differs from the oracle"
    say(f"  {name}: turned Q and K bitwise equal to the oracle; select on them equals the rotary select")


def test_select_rope_in_place():
    name = "small_edges"
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    _, dtab = _tables(desc)
    q_rot, k_rot, rp, ci = lcsa.select_rope(plan, q, k, dtab)
    q2, k2 = q.clone(), k.clone()
    q3, k3, rp3, ci3 = lcsa.select_rope(plan, q2, k2, dtab, q_rot=q2, k_rot=k2)
    torch.cuda.synchronize()
    assert q3.data_ptr() == q2.data_ptr() and k3.data_ptr() == k2.data_ptr()
    assert torch.equal(q2.view(torch.int16), q_rot.view(torch.int16))
    assert torch.equal(k2.view(torch.int16), k_rot.view(torch.int16))
    assert torch.equal(rp, rp3) and torch.equal(ci, ci3)


def test_select_rope_strided_outputs():
    """Outputs with their own strides (heads-major storage viewed as
    [B, S, H, D]) hold the same values."""
    name = "small_edges"
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    _, dtab = _tables(desc)
    q_rot, k_rot, rp, ci = lcsa.select_rope(plan, q, k, dtab)
    B, Sq, H, D = q.shape
    qs = torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device).permute(0, 2, 1, 3)
    ks = torch.empty((B, H, k.shape[1], D), dtype=k.dtype, device=k.device).permute(0, 2, 1, 3)
    lcsa.select_rope(plan, q, k, dtab, q_rot=qs, k_rot=ks)
    torch.cuda.synchronize()
    assert torch.equal(qs.contiguous().view(torch.int16), q_rot.view(torch.int16))
    assert torch.equal(ks.contiguous().view(torch.int16), k_rot.view(torch.int16))


def test_select_ring_rope_stream_matches_contiguous():
    """A first chunk of 6 frames, then 2-frame chunks over a 6-slot ring: each
    chunk turns and pools only its new frames; CSR, turned Q and the turned
    K ring equal the contiguous rotary select on the window, bitwise."""
    base = dict(li.CONFIGS["small_edges"], cached_frames=0, kv_ratio=0.0, q_frames=10, topk=8)
    video = li.generate(base, seed=12)
    ft = base["grid_h"] * base["grid_w"]
    qv, kv = to_device_bf16(video.q), to_device_bf16(video.k)
    B, _, H, D = qv.shape
    slots = 6
    k_ring = torch.zeros((B, slots * ft, H, D), dtype=qv.dtype, device="cuda")
    kr_ring = torch.zeros_like(k_ring)
    kcache = None
    for c, (f0, nq, cached) in enumerate([(0, 6, 0), (6, 2, 4), (8, 2, 4)]):
        desc = dict(base, q_frames=nq, cached_frames=cached, kv_ratio=3.0)
        plan = lcsa.Plan.from_desc(desc)
        kvf = plan.info["kv_frames"]
        w0 = f0 + nq - kvf
        frame_slot = [(w0 + t) % slots for t in range(kvf)]
        ring = lcsa.kv_ring(slots, frame_slot)
        if kcache is None:
            kcache = torch.full((lcsa.kcache_bytes(plan, slots) // 8,), float("nan"),
                                dtype=torch.float64, device="cuda")
        new = nq if c > 0 else kvf
        for t in range(kvf - new, kvf):
            s = frame_slot[t]
            k_ring[:, s * ft:(s + 1) * ft] = kv[:, (w0 + t) * ft:(w0 + t + 1) * ft]
        q = qv[:, f0 * ft:(f0 + nq) * ft].contiguous()
        k_win = kv[:, w0 * ft:(w0 + kvf) * ft].contiguous()
        _, dtab = _tables(desc, frame_offset=w0)       # rows = window frames w0 ..
        q_rot, rp, ci = lcsa.select_ring_rope(plan, q, k_ring, ring, new, kcache, dtab, kr_ring)
        q_ref, k_ref, rp_ref, ci_ref = lcsa.select_rope(plan, q, k_win, dtab)
        torch.cuda.synchronize()
        assert torch.equal(rp, rp_ref) and torch.equal(ci, ci_ref), f"chunk {c}: CSR differs"
        assert torch.equal(q_rot.view(torch.int16), q_ref.view(torch.int16))
        for t in range(kvf - new, kvf):
            s = frame_slot[t]
            assert torch.equal(kr_ring[:, s * ft:(s + 1) * ft].view(torch.int16),
                               k_ref[:, t * ft:(t + 1) * ft].view(torch.int16)), f"chunk {c} frame {t}"
        say(f"  chunk {c}: window {w0}..{w0 + kvf - 1}, turned and pooled {new} new frames: "
            f"bitwise equal to the contiguous rotary select")


def _random_tables(rng, g, pairs):
    def tab(n, m):
        ang = rng.uniform(-np.pi, np.pi, size=(n, m))
        return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    return oracle.RopeTables(t=tab(g.kv_frames, pairs[0]), h=tab(g.grid_h, pairs[1]),
                             w=tab(g.grid_w, pairs[2]))


@pytest.mark.parametrize("case", range(8))
def test_select_rope_random_configs(case):
    """Random small configurations (as in test_gpu_random_configs) with a
    random split of the 64 pairs over the three axes and random angles."""
    from test_gpu_random_configs import random_desc
    rng = np.random.default_rng(2000 + case)
    desc = random_desc(rng)
    cuts = np.sort(rng.integers(0, 65, size=2))
    pairs = (int(cuts[0]), int(cuts[1] - cuts[0]), int(64 - cuts[1]))
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    tab = _random_tables(rng, g, pairs)
    dtab = lcsa.rope(*(torch.from_numpy(getattr(tab, a)).cuda() for a in ("t", "h", "w")))
    say(f"  case {case}: block {desc['block_h']}x{desc['block_w']}, grid {g.nbh}x{g.nbw}, "
        f"q {g.q_frames} kv {g.kv_frames}, pairs {pairs}")
    inp = li.generate(desc, seed=100 + case)
    q, k, v = (to_device_bf16(x) for x in (inp.q, inp.k, inp.v))
    q_rot, k_rot, rp, ci = lcsa.select_rope(plan, q, k, dtab)
    o = lcsa.attend(plan, q_rot, k_rot, v, rp, ci)
    torch.cuda.synchronize()
    qr = oracle.rope_q(g, li.bf16_bits_to_f64(inp.q), tab)
    kr = oracle.rope_k(g, li.bf16_bits_to_f64(inp.k), tab)
    assert np.array_equal(_bits(q_rot), _f64_to_bits(qr))
    assert np.array_equal(_bits(k_rot), _f64_to_bits(kr))
    rp_ref, ci_ref, s_ref = oracle.select(g, qr, kr)
    rp_g, ci_g = rp.cpu().numpy(), ci.cpu().numpy()
    check_mask(g, rp_ref, ci_ref, s_ref, rp_g, ci_g)
    o_ref, _ = oracle.attend(g, qr, kr, li.bf16_bits_to_f64(inp.v), rp_g.astype(np.int64),
                             ci_g.astype(np.int64))
    compare_output(bf16_to_np(o), o_ref, f"rope random case {case}")
