"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle on
the same seeded inputs.

Select: row_ptr bit-exact; pooled scores within 1e-12 of the row scale
(both sides sum in float64); selected blocks identical except at near-ties
(oracle k-th score gap <= 1e-4 relative), which are counted and reported.
Attend: bf16 output within max |err| <= 1e-2 and cosine >= 0.9999 of the
oracle run on the GPU's own mask; LSE within 2e-3.  Small grids, the stream
chunk and both 768-line first chunks are compared element by element on the
whole tensor (the oracle spread over heads on worker processes), and so is
the 184320-token 4K chunk (6.5 TFLOP of float64 oracle attention)."""
import math

import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle
from oracle.parallel import OraclePool
from gpu_util import (check_mask, compare_output, bf16_to_np, device_qkv, host_inputs,
                      oracle_select, say, to_device_bf16)

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)

SMALL = ["tiny", "tiny_window", "small_edges", "small_16x8"]
FULL = ["first_768x1280", "stream_768x1280", "first_768x1408", "first_2048x3840"]
LSE_TOL = 2e-3


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    say(f"[gpu] done  {request.node.nodeid}")


def _f32(bits):
    return li.bf16_bits_to_f32(bits)


@pytest.mark.parametrize("name", SMALL + FULL)
def test_select_parity(name):
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    say(f"  select {name}: rows {plan.info['rows']} nnz {plan.info['nnz']} "
        f"window {plan.info['min_window']}..{plan.info['max_window']} k {plan.info['k']}")
    rp, ci, sc = lcsa.select(plan, q, k, return_scores=True)
    rp2, ci2 = lcsa.select(plan, q, k)           # path without the score dump
    torch.cuda.synchronize()
    g, rp_ref, ci_ref, s_ref = oracle_select(name)
    s_gpu = sc.cpu().numpy()
    assert np.array_equal(np.isneginf(s_gpu), np.isneginf(s_ref))
    fin = np.isfinite(s_ref)
    scale = float(np.abs(s_ref[fin]).max())
    err = float(np.abs(s_gpu[fin] - s_ref[fin]).max())
    say(f"  score max|err| {err:.3e} (scale {scale:.3e})")
    assert err <= 1e-12 * scale
    mism, ties = check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    say(f"  rows {len(rp_ref) - 1}: mask mismatches {len(mism)}, all near-ties ({len(ties)})")
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2)


@pytest.mark.parametrize("name", SMALL + ["stream_768x1280"])
def test_attend_parity_full(name):
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    torch.cuda.synchronize()
    _, inp = host_inputs(name)
    g = oracle.geometry(desc)
    o_ref, lse_ref = oracle.attend(g, _f32(inp.q), _f32(inp.k), _f32(inp.v),
                                   rp.cpu().numpy().astype(np.int64),
                                   ci.cpu().numpy().astype(np.int64))
    compare_output(bf16_to_np(o), o_ref, name)
    lerr = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    say(f"  LSE max|err| {lerr:.3e}")
    assert lerr <= LSE_TOL


def split_tail_rows(plan):
    """CSR rows that lcsa_attend (with its workspace) splits over several
    workgroups on this GPU: the rows % slots last rows of the launch's
    visiting order (square tiles of block positions, all query frames of a
    tile together, head by head), when each gets at least two pieces."""
    inf, d = plan.info, plan.desc
    bt = inf["block_tokens"]
    slots = torch.cuda.get_device_properties(0).multi_processor_count * (8 // (bt // 32))
    rows = int(inf["rows"])
    tail = rows % slots
    if tail == 0 or min(slots // tail, min(inf["max_row_nnz"], 16)) < 2:
        return []
    nbh, nbw, nbf, nqb, qf = inf["nbh"], inf["nbw"], inf["blocks_per_frame"], inf["nqb"], d["q_frames"]
    tile = int(math.sqrt((slots // 8) / qf) + 0.5)
    tile = min(max(tile, 1), max(nbh, nbw))
    out = []
    for e in range(rows - tail, rows):
        bh, r = divmod(e, nqb)
        band = tile * nbw * qf
        ty, r = divmod(r, band)
        th = min(tile, nbh - ty * tile)
        tx, r = divmod(r, th * tile * qf)
        tw = min(tile, nbw - tx * tile)
        tq, pp = divmod(r, th * tw)
        py, px = divmod(pp, tw)
        out.append(bh * nqb + tq * nbf + (ty * tile + py) * nbw + tx * tile + px)
    return out


@pytest.mark.parametrize("name", ["first_768x1280", "first_768x1408", "first_2048x3840"])
def test_attend_parity_whole_tensor(name):
    """Every row of the first chunks against the oracle (run over the GPU's
    own mask), including the rows of the split tail."""
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    o1 = lcsa.attend(plan, q, k, v, rp, ci, split_tail=False)
    torch.cuda.synchronize()
    split = split_tail_rows(plan)
    g = oracle.geometry(desc)
    o_h, o1_h = bf16_to_np(o), bf16_to_np(o1)
    differ = set()
    for r in range(plan.info["rows"]):
        bb, rem = divmod(r, g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        tok = oracle.block_tokens(g, qb)
        if not np.array_equal(o_h[bb, tok, h], o1_h[bb, tok, h]):
            differ.add(r)
    say(f"  {name}: {len(split)} split-tail rows on this GPU, {len(differ)} rows differ from "
        f"the unsplit launch")
    assert differ <= set(split), "rows outside the computed split tail differ from unsplit"
    _, inp = host_inputs(name)
    with OraclePool(desc, inp.q, inp.k, inp.v) as pool:
        o_ref, lse_ref, wall = pool.attend(rp.cpu().numpy().astype(np.int64),
                                           ci.cpu().numpy().astype(np.int64))
    say(f"  oracle attention on every row: {wall:.1f} s on {pool.workers} processes")
    compare_output(o_h, o_ref, f"{name} whole tensor")
    if split:
        sel = np.zeros((g.batch, g.q_tokens, g.heads), dtype=bool)
        for r in split:
            bb, rem = divmod(r, g.heads * g.nqb)
            h, qb = divmod(rem, g.nqb)
            sel[bb, oracle.block_tokens(g, qb), h] = True
        compare_output(o_h[sel], o_ref[sel], f"{name} split-tail rows")
    lerr = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    say(f"  LSE max|err| {lerr:.3e}")
    assert lerr <= LSE_TOL


def test_one_gpu_head_share():
    """One GPU's share when the 12 heads of the first 768x1280 chunk are
    sharded over 4 GPUs: 3 heads at the full token shape.  Masks against the
    oracle, and attention on every row against it, split and unsplit.  On a
    256-CU GPU its 540 rows leave a last, partly filled round of 28 rows,
    each split into the largest number of pieces the entry point uses (16)."""
    name, heads = "first_768x1280", 3
    desc, q, k, v = device_qkv(name, heads=heads)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    o1 = lcsa.attend(plan, q, k, v, rp, ci, split_tail=False)
    torch.cuda.synchronize()
    g, rp_ref, ci_ref, s_ref = oracle_select(name, heads=heads)
    mism, ties = check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    split = split_tail_rows(plan)
    say(f"  {heads}-head share: rows {plan.info['rows']}, mask mismatches {len(mism)} "
        f"(near-ties {len(ties)}), {len(split)} split-tail rows")
    _, inp = host_inputs(name, heads=heads)
    with OraclePool(desc, inp.q, inp.k, inp.v) as pool:
        o_ref, lse_ref, _ = pool.attend(rp.cpu().numpy().astype(np.int64),
                                        ci.cpu().numpy().astype(np.int64))
    o_h = bf16_to_np(o)
    compare_output(o_h, o_ref, f"{heads}-head share whole tensor")
    compare_output(bf16_to_np(o1), o_ref, f"{heads}-head share, no split")
    if split:
        sel = np.zeros((g.batch, g.q_tokens, g.heads), dtype=bool)
        for r in split:
            bb, rem = divmod(r, g.heads * g.nqb)
            h, qb = divmod(rem, g.nqb)
            sel[bb, oracle.block_tokens(g, qb), h] = True
        compare_output(o_h[sel], o_ref[sel], f"{heads}-head share split-tail rows")
    lerr = float(np.abs(lse.cpu().numpy() - lse_ref).max())
    say(f"  LSE max|err| {lerr:.3e}")
    assert lerr <= LSE_TOL


@pytest.mark.parametrize("name", ["tiny_window", "small_edges", "stream_768x1280",
                                  "first_768x1280"])
def test_attend_split_tail_matches_unsplit(name):
    """With a workspace, the rows of the last partly filled round of
    workgroups are split over their block lists and merged (small_edges: 96
    rows in 5 pieces each, merged in two groups).  Each piece
    rounds its probabilities to bf16 against its own running max, so the two
    paths differ by rounding, not bitwise: both must meet the parity bar
    against each other and, on the small grid, against the oracle."""
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    o1, l1 = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True, split_tail=False)
    o2, l2 = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    torch.cuda.synchronize()
    a, b = bf16_to_np(o1), bf16_to_np(o2)
    frac = float(np.mean(a != b))
    say(f"  split vs unsplit: {100 * frac:.3f}% elements differ")
    compare_output(b, a, f"{name} split vs unsplit")
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2))
    assert float((l1[fin] - l2[fin]).abs().max()) <= LSE_TOL
    if name in ("tiny_window", "small_edges"):
        _, inp = host_inputs(name)
        g = oracle.geometry(desc)
        o_ref, lse_ref = oracle.attend(g, _f32(inp.q), _f32(inp.k), _f32(inp.v),
                                       rp.cpu().numpy().astype(np.int64),
                                       ci.cpu().numpy().astype(np.int64))
        compare_output(a, o_ref, f"{name} unsplit")
        compare_output(b, o_ref, f"{name} split")


@pytest.mark.parametrize("shape", [(4, 16), (16, 4), (2, 32), (32, 4), (4, 32)])
def test_explicit_block_shapes(shape):
    """Explicit block shapes other than the automatic 8x16 / 16x8: the tile
    loads and the window enumeration follow the block geometry."""
    bh, bw = shape
    desc = dict(li.CONFIGS["small_edges"], block_t=1, block_h=bh, block_w=bw, topk=6)
    inp = li.generate(desc, seed=5)
    q, k, v = (to_device_bf16(x) for x in (inp.q, inp.k, inp.v))
    plan = lcsa.Plan.from_desc(desc)
    rp, ci, sc = lcsa.select(plan, q, k, return_scores=True)
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    o1 = lcsa.attend(plan, q, k, v, rp, ci, split_tail=False)
    torch.cuda.synchronize()
    g = oracle.geometry(desc)
    rp_ref, ci_ref, s_ref = oracle.select(g, li.bf16_bits_to_f64(inp.q), li.bf16_bits_to_f64(inp.k))
    check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    o_ref, lse_ref = oracle.attend(g, _f32(inp.q), _f32(inp.k), _f32(inp.v),
                                   rp.cpu().numpy().astype(np.int64), ci.cpu().numpy().astype(np.int64))
    compare_output(bf16_to_np(o), o_ref, f"block {bh}x{bw}")
    compare_output(bf16_to_np(o1), o_ref, f"block {bh}x{bw} unsplit")
    assert float(np.abs(lse.cpu().numpy() - lse_ref).max()) <= LSE_TOL


def test_attend_dense_special_case():
    """k = all key blocks with a covering window: plain dense attention."""
    desc = dict(li.CONFIGS["tiny"], topk=8)
    inp = li.generate(desc, seed=3)
    q, k, v = (to_device_bf16(x) for x in (inp.q, inp.k, inp.v))
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    assert plan.info["nnz"] == plan.info["rows"] * plan.info["nkb"]
    o = lcsa.attend(plan, q, k, v, rp, ci)
    torch.cuda.synchronize()
    g = oracle.geometry(desc)
    rp_h, ci_h, _ = oracle.select(g, _f32(inp.q), _f32(inp.k))
    o_ref, _ = oracle.attend(g, _f32(inp.q), _f32(inp.k), _f32(inp.v), rp_h, ci_h)
    compare_output(bf16_to_np(o), o_ref, "dense")


def test_attend_caller_csr_edge_rows():
    """Empty rows, out-of-range block indices, a row over every key block and
    a final row end beyond nnz (clamped)."""
    name = "tiny_window"
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    _, rp_o, ci_o, _ = oracle_select(name)
    rows = plan.info["rows"]
    lists = [ci_o[rp_o[r]:rp_o[r + 1]].tolist() for r in range(rows)]
    lists[0] = []
    lists[1] = [-1, g.nkb + 3, 5, 2 ** 30]
    lists[2] = list(range(g.nkb))
    lists[3] = [-7]
    rp_h = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int64)
    ci_h = np.asarray([c for x in lists for c in x], dtype=np.int64)
    rp_dev_h = rp_h.copy()
    rp_dev_h[-1] += 10                      # end past nnz: the kernel clamps
    rp_d = torch.from_numpy(rp_dev_h.astype(np.int32)).cuda()
    ci_d = torch.from_numpy(ci_h.astype(np.int32)).cuda()
    o, lse = lcsa.attend(plan, q, k, v, rp_d, ci_d, return_lse=True)
    torch.cuda.synchronize()
    _, inp = host_inputs(name)
    o_ref, lse_ref = oracle.attend(g, _f32(inp.q), _f32(inp.k), _f32(inp.v), rp_h, ci_h)
    compare_output(bf16_to_np(o), o_ref, "edge rows")
    lse_h = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(lse_h), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert float(np.abs(lse_h[fin] - lse_ref[fin]).max()) <= LSE_TOL
    q_empty = oracle.block_tokens(g, 0)
    assert np.all(bf16_to_np(o)[0, q_empty, 0, :] == 0)


@pytest.mark.parametrize("order", ["rising", "falling", "random"])
def test_attend_softmax_reference_moves(order):
    """Key blocks scaled by factors 1 .. 256 so that block score maxima climb
    (rising), fall (falling) or jump about (random) along every row's block
    list, each row holding every key block in ascending order.  Rising and
    random scores move the softmax reference again and again inside a row
    (the branch that takes the block max, rescales O and the row sum, and
    recomputes P); falling scores leave later blocks near underflow.  A move
    happens only when the new block outweighs the earlier ones by about 2^10,
    so this guards the branch against gross failure (P left against the old
    reference, infinities, NaN), not the rescale factor's last bits."""
    name = "small_edges"
    desc, inp = host_inputs(name)
    g = oracle.geometry(desc)
    plan = lcsa.Plan.from_desc(desc)
    nkb = g.nkb
    if order == "rising":
        f = 2.0 ** (8.0 * np.arange(nkb) / (nkb - 1))
    elif order == "falling":
        f = 2.0 ** (8.0 * np.arange(nkb)[::-1] / (nkb - 1))
    else:
        f = 2.0 ** np.random.default_rng(5).uniform(0.0, 8.0, nkb)
    k32 = _f32(inp.k).copy()
    for kb in range(nkb):
        k32[:, oracle.block_tokens(g, kb)] *= np.float32(f[kb])
    k_bits = li.f32_to_bf16_bits(k32)
    rows = plan.info["rows"]
    rp_h = (np.arange(rows + 1) * nkb).astype(np.int64)
    ci_h = np.tile(np.arange(nkb), rows).astype(np.int64)
    q = to_device_bf16(inp.q)
    k = to_device_bf16(k_bits)
    v = to_device_bf16(inp.v)
    rp_d = torch.from_numpy(rp_h.astype(np.int32)).cuda()
    ci_d = torch.from_numpy(ci_h.astype(np.int32)).cuda()
    o, lse = lcsa.attend(plan, q, k, v, rp_d, ci_d, return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attend(g, _f32(inp.q), _f32(k_bits), _f32(inp.v), rp_h, ci_h)
    say(f"  {order}: LSE range {float(lse_ref.min()):.1f} .. {float(lse_ref.max()):.1f}")
    compare_output(bf16_to_np(o), o_ref, f"reference moves ({order})")
    lse_h = lse.cpu().numpy()
    assert np.all(np.abs(lse_h - lse_ref) <= LSE_TOL * np.maximum(1.0, np.abs(lse_ref)))


def test_strided_views_and_kv_cache_window():
    """Q/K/V as slices of a packed QKV tensor, O written into a strided view,
    and K/V of a streaming call as a window of a longer cache: bitwise equal
    to the contiguous call."""
    name = "small_16x8"
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    o_ref = lcsa.attend(plan, q, k, v, rp, ci)
    B, S, H, D = q.shape
    qkv = torch.empty((B, S, 3, H, D), dtype=torch.bfloat16, device="cuda")
    qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2] = q, k, v
    obuf = torch.zeros((B, S, H, 2 * D), dtype=torch.bfloat16, device="cuda")
    out = obuf[..., D:]
    rp2, ci2 = lcsa.select(plan, qkv[:, :, 0], qkv[:, :, 1])
    lcsa.attend(plan, qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], rp2, ci2, out=out)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2) and torch.equal(ci, ci2)
    assert torch.equal(out, o_ref) and torch.all(obuf[..., :D] == 0)

    name = "small_edges"       # 2 query frames, KV window of 3 frames
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci = lcsa.select(plan, q, k)
    o_ref = lcsa.attend(plan, q, k, v, rp, ci)
    fs = desc["grid_h"] * desc["grid_w"]
    cache_k = torch.zeros((B, k.shape[1] + 2 * fs, k.shape[2], D), dtype=torch.bfloat16, device="cuda")
    cache_v = torch.zeros_like(cache_k)
    cache_k[:, 2 * fs:], cache_v[:, 2 * fs:] = k, v
    kw, vw = cache_k[:, 2 * fs:], cache_v[:, 2 * fs:]
    rp2, ci2 = lcsa.select(plan, q, kw)
    o2 = lcsa.attend(plan, q, kw, vw, rp2, ci2)
    torch.cuda.synchronize()
    assert torch.equal(ci, ci2) and torch.equal(o_ref, o2)


def test_batch_two():
    name = "small_edges"
    desc, q, k, v = device_qkv(name, batch=2)
    plan = lcsa.Plan.from_desc(desc)
    rp, ci, sc = lcsa.select(plan, q, k, return_scores=True)
    o = lcsa.attend(plan, q, k, v, rp, ci)
    torch.cuda.synchronize()
    g, rp_ref, ci_ref, s_ref = oracle_select(name, batch=2)
    check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    _, inp = host_inputs(name, batch=2)
    o_ref, _ = oracle.attend(g, _f32(inp.q), _f32(inp.k), _f32(inp.v), rp_ref, ci_ref)
    compare_output(bf16_to_np(o), o_ref, "batch 2")


def test_deterministic_repeat():
    name = "first_768x1280"
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    outs = []
    for _ in range(2):
        rp, ci = lcsa.select(plan, q, k)
        o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
        outs.append((rp, ci, o, lse))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("ring", [False, True])
def test_longest_kv_window(ring):
    """The largest KV window the library takes: 64 latent frames (62 cached +
    2 query frames), every frame eligible, on a small grid; through the frame
    ring the 64 frames sit in scrambled slots."""
    desc = dict(li.CONFIGS["tiny"], heads=1, q_frames=2, cached_frames=62, kv_ratio=0.0, topk=24)
    plan = lcsa.Plan.from_desc(desc)
    assert plan.info["kv_frames"] == 64
    inp = li.generate(desc, seed=4)
    q, k, v = (to_device_bf16(x) for x in (inp.q, inp.k, inp.v))
    if ring:
        ft = desc["grid_h"] * desc["grid_w"]
        slots = 64
        frame_slot = np.random.default_rng(3).permutation(slots).tolist()
        rg = lcsa.kv_ring(slots, frame_slot)
        k_ring, v_ring = torch.empty_like(k), torch.empty_like(v)
        for t in range(64):
            s = frame_slot[t]
            k_ring[:, s * ft:(s + 1) * ft] = k[:, t * ft:(t + 1) * ft]
            v_ring[:, s * ft:(s + 1) * ft] = v[:, t * ft:(t + 1) * ft]
        kcache = torch.empty(lcsa.kcache_bytes(plan, slots) // 8, dtype=torch.float64, device="cuda")
        rp, ci = lcsa.select_ring(plan, q, k_ring, rg, 64, kcache)
        o = lcsa.attend_ring(plan, q, k_ring, v_ring, rg, rp, ci)
    else:
        rp, ci = lcsa.select(plan, q, k)
        o = lcsa.attend(plan, q, k, v, rp, ci)
    torch.cuda.synchronize()
    g = oracle.geometry(desc)
    qf, kf, vf = (li.bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    rp_ref, ci_ref, s_ref = oracle.select(g, qf, kf)
    check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    o_ref, _ = oracle.attend(g, qf, kf, vf, rp.cpu().numpy().astype(np.int64),
                             ci.cpu().numpy().astype(np.int64))
    compare_output(bf16_to_np(o), o_ref, f"64-frame KV window{' (ring)' if ring else ''}")
