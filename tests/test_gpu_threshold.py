"""Steady threshold reuse through the C ABI (lcsa_select_steady /
lcsa_select_reuse) against the float64 oracle (oracle/threshold_oracle.py).

Steady: the CSR is the top-k selection's, bit for bit; each row's threshold
is its keep-th largest window score (exactly the smallest kept GPU score,
and within 1e-12 of the row scale of the oracle's).  Reuse: the padded CSR
keeps exactly the oracle's blocks, except blocks whose oracle score lies
within 1e-9 of the score scale of the threshold (the two sides' float64
scores differ by ~1e-16 relative); thresholds of the same chunk give back
the top-k.  Attend on the padded CSR equals attend on the same blocks
compacted, bit for bit, and matches the oracle's attention on it."""
import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle
from gpu_util import bf16_to_np, compare_output, device_qkv, host_inputs, oracle_select, say

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)

SMALL = ["tiny", "tiny_window", "small_edges", "small_16x8"]
BAND = 1e-9


@pytest.fixture(autouse=True)
def _announce(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say(f"[gpu] start {request.node.nodeid}")
    yield
    torch.cuda.synchronize()
    say(f"[gpu] done  {request.node.nodeid}")


def _rows(g):
    for b in range(g.batch):
        for h in range(g.heads):
            for qb in range(g.nqb):
                yield (b * g.heads + h) * g.nqb + qb, b, h, qb


def _check_padded(g, rp, ci, pad):
    rows = g.batch * g.heads * g.nqb
    assert np.array_equal(rp, np.arange(rows + 1) * pad)
    out = []
    for r, b, h, qb in _rows(g):
        seg = ci[r * pad:(r + 1) * pad]
        n = int(np.sum(seg >= 0))
        assert np.all(seg[n:] == -1), f"row {r}: -1 padding not at the end"
        blocks = seg[:n]
        assert np.all(np.diff(blocks) > 0), f"row {r}: not ascending"
        assert set(blocks.tolist()) <= set(oracle.window(g, qb).tolist()), f"row {r}: off window"
        out.append(blocks)
    return out


def _compare_with_oracle(g, rows_gpu, s_ref, tau, label):
    rows_ref = oracle.select_threshold(g, s_ref, tau)
    scale = float(np.abs(s_ref[np.isfinite(s_ref)]).max())
    diff_rows = 0
    for (r, b, h, qb), a, e in zip(_rows(g), rows_gpu, rows_ref):
        if np.array_equal(a, e):
            continue
        diff_rows += 1
        for kb in set(a.tolist()) ^ set(e.tolist()):
            assert abs(s_ref[b, h, qb, kb] - tau[r]) <= BAND * scale, \
                f"{label} row {r} block {kb}: differs and is not at the threshold"
    kept = np.array([len(a) for a in rows_gpu])
    say(f"  {label}: kept per row mean {kept.mean():.2f} (min {kept.min()}, max {kept.max()}), "
        f"rows differing at the threshold {diff_rows}")
    return kept


@pytest.mark.parametrize("name", SMALL + ["stream_768x1280", "first_768x1280"])
def test_steady_is_top_k_with_thresholds(name):
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp0, ci0 = lcsa.select(plan, q, k)
    rp, ci, kth, sc = lcsa.select_steady(plan, q, k, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp0) and torch.equal(ci, ci0)
    g, _, _, s_ref = oracle_select(name)
    rp_h, ci_h, kth_h, sc_h = (x.cpu().numpy() for x in (rp, ci, kth, sc))
    for r, b, h, qb in _rows(g):
        kept = ci_h[rp_h[r]:rp_h[r + 1]]
        assert kth_h[r] == sc_h[b, h, qb, kept].min(), f"row {r}: kth is not the smallest kept"
    want = oracle.row_thresholds(g, s_ref)
    scale = float(np.abs(s_ref[np.isfinite(s_ref)]).max())
    err = float(np.abs(kth_h - want).max())
    say(f"  {name}: kth max|err| {err:.3e} (scale {scale:.3e})")
    assert err <= 1e-12 * scale


@pytest.mark.parametrize("name", SMALL + ["stream_768x1280"])
def test_reuse_parity(name):
    """Thresholds of another chunk (seed 1) applied to this chunk's scores."""
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    g, _, _, s_ref = oracle_select(name)
    _, inp1 = host_inputs(name, seed=1)
    _, _, s1 = oracle.select(g, li.bf16_bits_to_f64(inp1.q), li.bf16_bits_to_f64(inp1.k))
    tau = oracle.row_thresholds(g, s1)
    rp, ci = lcsa.select_reuse(plan, q, k, torch.from_numpy(tau).cuda())
    torch.cuda.synchronize()
    pad = plan.info["max_window"]
    rows_gpu = _check_padded(g, rp.cpu().numpy(), ci.cpu().numpy(), pad)
    _compare_with_oracle(g, rows_gpu, s_ref, tau, name)


@pytest.mark.parametrize("name", SMALL)
def test_reuse_with_own_thresholds_is_top_k(name):
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    rp0, ci0, kth, sc = lcsa.select_steady(plan, q, k, return_scores=True)
    rp, ci = lcsa.select_reuse(plan, q, k, kth)
    torch.cuda.synchronize()
    g = oracle.geometry(desc)
    pad = plan.info["max_window"]
    rows_gpu = _check_padded(g, rp.cpu().numpy(), ci.cpu().numpy(), pad)
    rp0_h, ci0_h, kth_h, sc_h = (x.cpu().numpy() for x in (rp0, ci0, kth, sc))
    for (r, b, h, qb), a in zip(_rows(g), rows_gpu):
        e = oracle.window(g, qb)
        ties = int(np.sum(sc_h[b, h, qb, e] == kth_h[r]))
        if ties == 1:
            assert np.array_equal(a, ci0_h[rp0_h[r]:rp0_h[r + 1]]), f"row {r}"


def test_reuse_extreme_thresholds():
    desc, q, k, v = device_qkv("small_edges")
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    rows, pad = plan.info["rows"], plan.info["max_window"]
    for label, val in (("-inf", -np.inf), ("+inf", np.inf), ("nan", np.nan)):
        tau = torch.full((rows,), val, dtype=torch.float64, device="cuda")
        rp, ci = lcsa.select_reuse(plan, q, k, tau)
        o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
        torch.cuda.synchronize()
        got = _check_padded(g, rp.cpu().numpy(), ci.cpu().numpy(), pad)
        for (r, b, h, qb), a in zip(_rows(g), got):
            want = oracle.window(g, qb) if val == -np.inf else np.empty(0, dtype=np.int64)
            assert np.array_equal(a, want), f"tau {label} row {r}"
        if val != -np.inf:   # nothing kept: O = 0, LSE = -inf
            assert not torch.any(o.float() != 0) and bool(torch.all(torch.isneginf(lse)))
        say(f"  tau {label}: ok")


@pytest.mark.parametrize("name", SMALL + ["stream_768x1280"])
def test_attend_on_padded_csr(name):
    """Padded rows give bitwise the result of the same blocks compacted
    (with and without the split tail), and match the oracle's attention."""
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    _, inp1 = host_inputs(name, seed=1)
    _, _, s1 = oracle.select(g, li.bf16_bits_to_f64(inp1.q), li.bf16_bits_to_f64(inp1.k))
    # a spread of row lengths: the other chunk's thresholds, raised on some rows
    tau = oracle.row_thresholds(g, s1)
    tau[::7] = np.inf
    rp, ci = lcsa.select_reuse(plan, q, k, torch.from_numpy(tau).cuda())
    ci_h = ci.cpu().numpy()
    pad = plan.info["max_window"]
    rows = _check_padded(g, rp.cpu().numpy(), ci_h, pad)
    rp_c = np.concatenate([[0], np.cumsum([len(a) for a in rows])]).astype(np.int32)
    ci_c = np.concatenate(rows + [np.empty(0, np.int32)]).astype(np.int32)
    rp_cd = torch.from_numpy(rp_c).cuda()
    ci_cd = torch.from_numpy(ci_c if len(ci_c) else np.zeros(1, np.int32)).cuda()[:len(ci_c)]
    res = {}
    for split in (True, False):
        o_p, lse_p = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True, split_tail=split)
        o_c, lse_c = lcsa.attend(plan, q, k, v, rp_cd, ci_cd, return_lse=True, split_tail=split)
        torch.cuda.synchronize()
        assert torch.equal(o_p, o_c) and torch.equal(lse_p, lse_c), f"split_tail={split}"
        res[split] = (o_p, lse_p)
    # with the workspace the rows of the last partly filled round run as
    # merged pieces: the same result to rounding
    d = float((res[True][0].float() - res[False][0].float()).abs().max())
    fin = torch.isfinite(res[False][1])
    assert torch.equal(fin, torch.isfinite(res[True][1]))
    dl = float((res[True][1][fin] - res[False][1][fin]).abs().max()) if bool(fin.any()) else 0.0
    say(f"  {name}: split tail vs whole rows: O max|d| {d:.3e}, LSE max|d| {dl:.3e}")
    assert d <= 1e-2 and dl <= 2e-3   # P is rounded to bf16 against each piece's own reference
    o_p, lse_p = res[True]
    if name in SMALL:
        _, inp = host_inputs(name)
        o_ref, lse_ref = oracle.attend(g, li.bf16_bits_to_f32(inp.q), li.bf16_bits_to_f32(inp.k),
                                       li.bf16_bits_to_f32(inp.v), rp.cpu().numpy().astype(np.int64),
                                       ci_h.astype(np.int64))
        compare_output(bf16_to_np(o_p), o_ref, f"{name} padded CSR vs oracle")
        lse_h = lse_p.cpu().numpy()
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(lse_h), np.isneginf(lse_ref))
        assert float(np.abs(lse_h[fin] - lse_ref[fin]).max(initial=0.0)) <= 2e-3


def test_ring_and_rope_forms_match():
    """The ring and rotary forms of both calls give the plain forms' results."""
    name = "small_edges"
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    kvf = plan.info["kv_frames"]
    ft = desc["grid_h"] * desc["grid_w"]
    slots = kvf + 1
    frame_slot = [(t + 2) % slots for t in range(kvf)]
    ring = lcsa.kv_ring(slots, frame_slot)
    k_ring = torch.zeros((k.shape[0], slots * ft, k.shape[2], k.shape[3]), dtype=k.dtype,
                         device=k.device)
    for t, s in enumerate(frame_slot):
        k_ring[:, s * ft:(s + 1) * ft] = k[:, t * ft:(t + 1) * ft]
    kcache = torch.empty(lcsa.kcache_bytes(plan, slots) // 8, dtype=torch.float64, device="cuda")
    rp0, ci0, kth0 = lcsa.select_steady(plan, q, k)
    rp1, ci1, kth1 = lcsa.select_steady(plan, q, k_ring, ring=ring, new_frames=kvf, kcache=kcache)
    tau = kth0 * 1.0001 - 1e-3
    rq0, cq0 = lcsa.select_reuse(plan, q, k, tau)
    rq1, cq1 = lcsa.select_reuse(plan, q, k_ring, tau, ring=ring, new_frames=0, kcache=kcache)
    torch.cuda.synchronize()
    assert torch.equal(rp0, rp1) and torch.equal(ci0, ci1) and torch.equal(kth0, kth1)
    assert torch.equal(rq0, rq1) and torch.equal(cq0, cq1)

    tabs = li.rope_tables(desc)
    tt, th, tw = (torch.from_numpy(tabs[a]).cuda() for a in "thw")
    tables = lcsa.rope(tt, th, tw)
    q_rot0, k_rot0, rp2, ci2 = lcsa.select_rope(plan, q, k, tables)
    q_rot, k_rot = torch.empty_like(q), torch.empty_like(k)
    rp3, ci3, kth3 = lcsa.select_steady(plan, q, k, tables=tables, q_rot=q_rot, k_rot=k_rot)
    rq3, cq3 = lcsa.select_reuse(plan, q, k, kth3, tables=tables, q_rot=q_rot, k_rot=k_rot)
    rq4, cq4 = lcsa.select_reuse(plan, q_rot0, k_rot0, kth3)
    torch.cuda.synchronize()
    assert torch.equal(q_rot, q_rot0) and torch.equal(k_rot, k_rot0)
    assert torch.equal(rp3, rp2) and torch.equal(ci3, ci2)
    assert torch.equal(rq3, rq4) and torch.equal(cq3, cq4)


@pytest.mark.parametrize("varlen", [False, True])
def test_threshold_chain_in_graph(varlen):
    """Steady select on one chunk, reuse on the next and attention on the
    padded CSR (lcsa_attend, or lcsa_attend_varlen with its row-order
    kernels), captured once in a HIP graph and replayed on new inputs:
    bitwise equal to eager calls every time."""
    name = "small_edges"
    desc, _, _, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    inf = plan.info
    bufs = [torch.empty_like(x) for x in device_qkv(name)[1:]]
    qa, ka = torch.empty_like(bufs[0]), torch.empty_like(bufs[1])
    qb, kb, vb = bufs
    sel_ws = torch.empty(max(int(inf["select_workspace_bytes"]), 256), dtype=torch.uint8,
                         device="cuda")
    att_ws = torch.empty(int(inf["attend_workspace_bytes"]), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qb)

    def chain():
        _, _, kth = lcsa.select_steady(plan, qa, ka, workspace=sel_ws)
        rp, ci = lcsa.select_reuse(plan, qb, kb, kth, workspace=sel_ws)
        if varlen:
            lcsa.attend_varlen(plan, qb, kb, vb, rp, ci, out=out, workspace=att_ws)
        else:
            lcsa.attend(plan, qb, kb, vb, rp, ci, out=out, workspace=att_ws)
        return kth, rp, ci

    def load(seed):
        _, q1, k1, _ = device_qkv(name, seed=seed)
        _, q2, k2, v2 = device_qkv(name, seed=seed + 1)
        for dst, src in ((qa, q1), (ka, k1), (qb, q2), (kb, k2), (vb, v2)):
            dst.copy_(src)

    load(10)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        g_kth, g_rp, g_ci = chain()
    torch.cuda.synchronize()
    for rep, seed in enumerate((20, 30, 40)):
        load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (g_kth, g_rp, g_ci, out)]
        e_kth, e_rp, e_ci = chain()
        torch.cuda.synchronize()
        for a, b, what in zip(got, (e_kth, e_rp, e_ci, out), ("kth", "row_ptr", "col_idx", "out")):
            assert torch.equal(a, b), f"replay {rep}: {what} differs from eager"
        say(f"  replay {rep} (seed {seed}): bitwise equal to eager")
    del g


def test_ring_rope_steady_matches_ring_rope_select():
    """Ring and rotary tables together: lcsa_select_steady gives the CSR and
    turned tensors of lcsa_select_ring_rope bit for bit."""
    name = "small_edges"
    desc, q, k, _ = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    kvf = plan.info["kv_frames"]
    ft = desc["grid_h"] * desc["grid_w"]
    slots = kvf + 2
    frame_slot = [(t + 3) % slots for t in range(kvf)]
    ring = lcsa.kv_ring(slots, frame_slot)
    k_ring = torch.zeros((k.shape[0], slots * ft, k.shape[2], k.shape[3]), dtype=k.dtype,
                         device=k.device)
    for t, s in enumerate(frame_slot):
        k_ring[:, s * ft:(s + 1) * ft] = k[:, t * ft:(t + 1) * ft]
    tabs = li.rope_tables(desc)
    tables = lcsa.rope(*(torch.from_numpy(tabs[a]).cuda() for a in "thw"))
    kc1 = torch.empty(lcsa.kcache_bytes(plan, slots) // 8, dtype=torch.float64, device="cuda")
    kc2 = torch.empty_like(kc1)
    kr1, kr2 = torch.zeros_like(k_ring), torch.zeros_like(k_ring)
    q_rot1, rp1, ci1 = lcsa.select_ring_rope(plan, q, k_ring, ring, kvf, kc1, tables, kr1)
    q_rot2 = torch.empty_like(q)
    rp2, ci2, kth2 = lcsa.select_steady(plan, q, k_ring, ring=ring, new_frames=kvf, kcache=kc2,
                                        tables=tables, q_rot=q_rot2, k_rot=kr2)
    rq, cq = lcsa.select_reuse(plan, q, k_ring, kth2, ring=ring, new_frames=kvf, kcache=kc2,
                               tables=tables, q_rot=q_rot2, k_rot=kr2)
    torch.cuda.synchronize()
    assert torch.equal(q_rot1, q_rot2) and torch.equal(kr1, kr2)
    assert torch.equal(rp1, rp2) and torch.equal(ci1, ci2)
    used = torch.tensor(frame_slot, device="cuda")   # the other slots hold no frame
    assert torch.equal(kc1.view(slots, -1)[used], kc2.view(slots, -1)[used])
    g = oracle.geometry(desc)
    rows = _check_padded(g, rq.cpu().numpy(), cq.cpu().numpy(), plan.info["max_window"])
    say(f"  ring + rope: steady equals ring rotary select; reuse kept {sum(len(r) for r in rows)} "
        f"blocks against {int(rp1[-1])} top-k")


@pytest.mark.parametrize("name", SMALL + ["stream_768x1280"])
def test_attend_varlen(name):
    """lcsa_attend_varlen on a reused-threshold CSR (rows of many lengths,
    some empty): every row written (the output starts as NaN), the same bits
    on a second run, the oracle's attention on the small grids, and the
    whole-row attention's result to rounding: bit for bit on every row that
    is not split (at most rows % workgroup slots rows are)."""
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    _, inp1 = host_inputs(name, seed=1)
    _, _, s1 = oracle.select(g, li.bf16_bits_to_f64(inp1.q), li.bf16_bits_to_f64(inp1.k))
    tau = oracle.row_thresholds(g, s1)
    tau[::7] = np.inf
    rp, ci = lcsa.select_reuse(plan, q, k, torch.from_numpy(tau).cuda())
    lens = (ci.view(-1, plan.info["max_window"]) >= 0).sum(dim=1)
    say(f"  {name}: row lengths {int(lens.min())}..{int(lens.max())}, "
        f"{int((lens == 0).sum())} empty rows")
    runs = []
    for _ in range(2):
        out = torch.full_like(q, float("nan"))
        o, lse = lcsa.attend_varlen(plan, q, k, v, rp, ci, out=out, return_lse=True)
        torch.cuda.synchronize()
        assert not bool(torch.isnan(o.float()).any()), "a row was not written"
        runs.append((o, lse))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    o_v, lse_v = runs[0]
    o_w, lse_w = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True, split_tail=False)
    torch.cuda.synchronize()
    d = float((o_v.float() - o_w.float()).abs().max())
    fin = torch.isfinite(lse_w)
    assert torch.equal(fin, torch.isfinite(lse_v))
    dl = float((lse_v[fin] - lse_w[fin]).abs().max()) if bool(fin.any()) else 0.0
    assert d <= 1e-2 and dl <= 2e-3
    rows, bt = plan.info["rows"], plan.info["block_tokens"]
    props = torch.cuda.get_device_properties(0)
    slots = props.multi_processor_count * (8 // (bt // 32))
    # rows whose output differs at all from the whole-row run
    pd = plan.desc
    ov = o_v.view(pd["batch"], -1, pd["heads"], 128)
    ow = o_w.view(pd["batch"], -1, pd["heads"], 128)
    differ = 0
    for r, b, h, qb in _rows(g):
        tok = oracle.block_tokens(g, qb)
        differ += int(not torch.equal(ov[b, tok, h], ow[b, tok, h]))
    say(f"  {name}: vs whole rows O max|d| {d:.3e}, LSE max|d| {dl:.3e}; "
        f"{differ} of {rows} rows differ (at most {rows % slots} split)")
    assert differ <= rows % slots
    if name in SMALL:
        _, inp = host_inputs(name)
        o_ref, lse_ref = oracle.attend(g, li.bf16_bits_to_f32(inp.q), li.bf16_bits_to_f32(inp.k),
                                       li.bf16_bits_to_f32(inp.v), rp.cpu().numpy().astype(np.int64),
                                       ci.cpu().numpy().astype(np.int64))
        compare_output(bf16_to_np(o_v), o_ref, f"{name} varlen vs oracle")
        lse_h = lse_v.cpu().numpy()
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(lse_h), np.isneginf(lse_ref))
        assert float(np.abs(lse_h[fin] - lse_ref[fin]).max(initial=0.0)) <= 2e-3


def test_attend_varlen_ring_and_top_k():
    """The ring form of lcsa_attend_varlen gives the contiguous form's bits;
    on a top-k CSR (equal rows) it gives attend's result to rounding."""
    name = "small_edges"
    desc, q, k, v = device_qkv(name)
    plan = lcsa.Plan.from_desc(desc)
    g = oracle.geometry(desc)
    _, inp1 = host_inputs(name, seed=1)
    _, _, s1 = oracle.select(g, li.bf16_bits_to_f64(inp1.q), li.bf16_bits_to_f64(inp1.k))
    rp, ci = lcsa.select_reuse(plan, q, k, torch.from_numpy(oracle.row_thresholds(g, s1)).cuda())
    kvf = plan.info["kv_frames"]
    ft = desc["grid_h"] * desc["grid_w"]
    slots = kvf + 2
    fs = [int(x) for x in np.random.default_rng(11).permutation(slots)[:kvf]]
    ring = lcsa.kv_ring(slots, fs)
    kr = torch.zeros((desc["batch"], slots * ft, desc["heads"], 128), dtype=q.dtype, device="cuda")
    vr = torch.zeros_like(kr)
    for t in range(kvf):
        kr[:, fs[t] * ft:(fs[t] + 1) * ft] = k[:, t * ft:(t + 1) * ft]
        vr[:, fs[t] * ft:(fs[t] + 1) * ft] = v[:, t * ft:(t + 1) * ft]
    o_c = lcsa.attend_varlen(plan, q, k, v, rp, ci)
    o_r = lcsa.attend_varlen(plan, q, kr, vr, rp, ci, ring=ring)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_r)
    rp_t, ci_t = lcsa.select(plan, q, k)
    o_t = lcsa.attend(plan, q, k, v, rp_t, ci_t)
    o_tv = lcsa.attend_varlen(plan, q, k, v, rp_t, ci_t)
    torch.cuda.synchronize()
    assert float((o_t.float() - o_tv.float()).abs().max()) <= 1e-2
