"""Pins of the CPU oracle to things other than itself: hand-derived geometry
of the page workloads, closed forms, brute force on tiny grids, a library
attention routine (torch SDPA in float64 on the CPU), scipy's logsumexp, and
invariants / metamorphic relations of the method.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import lcsa_inputs as li
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "geometry.json")


def _desc(name, **over):
    d = dict(li.CONFIGS[name])
    d.update(over)
    return d


def _rand_inputs(desc, seed):
    inp = li.generate(desc, seed=seed)
    return (li.bf16_bits_to_f64(inp.q), li.bf16_bits_to_f64(inp.k),
            li.bf16_bits_to_f64(inp.v))


def _token_block_ids(g, n_frames):
    """Block index of every raster token, from token coordinates."""
    s = np.arange(n_frames * g.grid_h * g.grid_w)
    t = s // (g.grid_h * g.grid_w)
    y = (s // g.grid_w) % g.grid_h
    x = s % g.grid_w
    return t * g.nbf + (y // g.block_h) * g.nbw + (x // g.block_w)


# ------------------------------------------------------------- geometry
@pytest.mark.parametrize("name", li.PAGE_WORKLOADS)
def test_geometry_matches_hand_derivation(name):
    gold = json.load(open(GOLDEN))["workloads"][name]
    g = oracle.geometry(li.CONFIGS[name])
    assert g.q_tokens == gold["q_tokens"] and g.kv_tokens == gold["kv_tokens"]
    assert [g.block_h, g.block_w] == gold["block"]
    assert (g.nbh, g.nbw, g.nqb, g.nkb, g.half, g.k) == (
        gold["nbh"], gold["nbw"], gold["nqb"], gold["nkb"], gold["half"], gold["k"])
    sizes = [len(oracle.window(g, qb)) for qb in range(g.nqb)]
    assert min(sizes) == gold["eligible_min"] and max(sizes) == gold["eligible_max"]
    pairs = g.batch * g.heads * sum(min(g.k, n) for n in sizes)
    assert pairs == gold["pairs"]
    row_ptr = np.concatenate([[0], np.cumsum([min(g.k, n) for n in sizes] * g.heads)])
    assert oracle.useful_flops(g, row_ptr) == gold["useful_flop"]


def test_page_token_counts():
    facts = json.load(open(GOLDEN))["_page_facts"]
    g = oracle.geometry(li.CONFIGS["first_768x1280"])
    assert g.q_tokens == facts["first_chunk_tokens_768x1280"]["value"]
    shp = facts["first_chunk_latent_shape"]["value"]
    assert (g.q_frames, g.grid_h * 2, g.grid_w * 2) == tuple(shp[2:])


@pytest.mark.parametrize("name", list(li.CONFIGS))
def test_window_closed_form(name):
    g = oracle.geometry(li.CONFIGS[name])
    for qb in range(g.nqb):
        t, by, bx = oracle.block_coords(g, qb)
        rows = min(by + g.half, g.nbh - 1) - max(by - g.half, 0) + 1
        cols = min(bx + g.half, g.nbw - 1) - max(bx - g.half, 0) + 1
        e = oracle.window(g, qb)
        assert len(e) == g.kv_frames * rows * cols
        assert np.all(np.diff(e) > 0)
        for kb in e[:50]:
            _, ky, kx = oracle.block_coords(g, int(kb))
            assert abs(ky - by) <= g.half and abs(kx - bx) <= g.half


def test_budget_rounding_rules():
    # 1.5 * 768*1280/(768*1408) * 33 lands a hair off 45 in float64: must snap.
    g = oracle.geometry(li.CONFIGS["first_768x1408"])
    assert g.k == 45
    assert oracle.geometry(_desc("first_768x1280", topk_ratio=0.05)).k == 2   # 1.5 -> 2
    assert oracle.geometry(_desc("first_768x1280", topk_ratio=0.04)).k == 1   # 1.2 -> 1
    assert oracle.geometry(_desc("first_768x1280", topk_ratio=0.001)).k == 1  # clamp >= 1
    assert oracle.geometry(_desc("stream_768x1280", cached_frames=10)).kv_frames == 6
    assert oracle.geometry(_desc("stream_768x1280", cached_frames=1)).kv_frames == 3
    assert oracle.geometry(_desc("stream_768x1280", kv_ratio=0.0, cached_frames=3)).kv_frames == 5


def test_block_tokens_partition_grid():
    for name in ("tiny", "small_16x8", "small_edges"):
        g = oracle.geometry(li.CONFIGS[name])
        ids = _token_block_ids(g, g.kv_frames)
        seen = np.zeros(g.kv_tokens, dtype=int)
        for kb in range(g.nkb):
            tok = oracle.block_tokens(g, kb)
            assert len(tok) == g.block_tokens
            assert np.all(ids[tok] == kb)
            seen[tok] += 1
        assert np.all(seen == 1)


# ------------------------------------------------------ pooling + scoring
@pytest.mark.parametrize("name", ["tiny", "small_16x8", "small_edges"])
def test_block_score_is_block_mean_of_token_scores(name):
    """pooled q . pooled k = mean over (i in qb, j in kb) of q_i . k_j."""
    desc = li.CONFIGS[name]
    g = oracle.geometry(desc)
    q, k, _ = _rand_inputs(desc, 3)
    s = oracle.block_scores(g, q, k)
    qid = _token_block_ids(g, g.q_frames)
    kid = _token_block_ids(g, g.kv_frames)
    mq = np.zeros((g.nqb, g.q_tokens)); mq[qid, np.arange(g.q_tokens)] = 1.0 / g.block_tokens
    mk = np.zeros((g.nkb, g.kv_tokens)); mk[kid, np.arange(g.kv_tokens)] = 1.0 / g.block_tokens
    for b in range(g.batch):
        for h in range(g.heads):
            tok = q[b, :, h, :] @ k[b, :, h, :].T
            blk = mq @ tok @ mk.T
            finite = np.isfinite(s[b, h])
            np.testing.assert_allclose(s[b, h][finite], blk[finite], rtol=1e-10, atol=1e-10)
            # finite exactly on the window
            for qb in range(g.nqb):
                assert set(np.nonzero(finite[qb])[0]) == set(oracle.window(g, qb).tolist())


# -------------------------------------------------------------- selection
def _brute_force_topk(scores_row, elig, k):
    """Best k-subset by total score; among equal totals the smallest sorted
    index tuple (which is what 'ties go to the lower index' means)."""
    best = None
    for sub in itertools.combinations(sorted(elig), min(k, len(elig))):
        key = (-sum(scores_row[i] for i in sub), sub)
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("name", ["tiny", "tiny_window", "small_16x8"])
def test_select_matches_brute_force(name):
    desc = li.CONFIGS[name]
    g = oracle.geometry(desc)
    q, k, _ = _rand_inputs(desc, 5)
    row_ptr, col_idx, s = oracle.select(g, q, k)
    for b in range(g.batch):
        for h in range(g.heads):
            for qb in range(g.nqb):
                r = (b * g.heads + h) * g.nqb + qb
                got = col_idx[row_ptr[r]:row_ptr[r + 1]].tolist()
                e = oracle.window(g, qb).tolist()
                if len(e) > 12:
                    continue
                assert got == _brute_force_topk(s[b, h, qb], e, g.k)


def test_select_ties_go_to_lower_index():
    desc = li.CONFIGS["tiny"]
    g = oracle.geometry(desc)
    q, k, _ = _rand_inputs(desc, 7)
    # make every key block a copy of block 0: all scores in a row tie exactly
    tok0 = oracle.block_tokens(g, 0)
    for kb in range(1, g.nkb):
        k[:, oracle.block_tokens(g, kb)] = k[:, tok0]
    row_ptr, col_idx, s = oracle.select(g, q, k)
    for r in range(len(row_ptr) - 1):
        assert col_idx[row_ptr[r]:row_ptr[r + 1]].tolist() == list(range(g.k))
    for b in range(g.batch):
        for h in range(g.heads):
            for qb in range(g.nqb):
                e = oracle.window(g, qb).tolist()
                assert _brute_force_topk(s[b, h, qb], e, g.k) == list(range(g.k))


@pytest.mark.parametrize("name", ["tiny", "tiny_window", "small_edges", "small_16x8"])
def test_select_invariants(name):
    desc = li.CONFIGS[name]
    g = oracle.geometry(desc)
    q, k, _ = _rand_inputs(desc, 11)
    row_ptr, col_idx, s = oracle.select(g, q, k)
    assert row_ptr[0] == 0 and np.all(np.diff(row_ptr) >= 1) and row_ptr[-1] == len(col_idx)
    for r in range(len(row_ptr) - 1):
        qb = r % g.nqb
        sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
        e = oracle.window(g, qb)
        assert len(sel) == min(g.k, len(e))
        assert np.all(np.diff(sel) > 0)
        assert set(sel.tolist()) <= set(e.tolist())
        # every kept score >= every dropped score of the window
        b, h = divmod(r // g.nqb, g.heads)
        dropped = np.setdiff1d(e, sel)
        if len(dropped):
            assert s[b, h, qb, sel].min() >= s[b, h, qb, dropped].max()


def test_select_metamorphic():
    desc = li.CONFIGS["small_edges"]
    g = oracle.geometry(desc)
    q, k, _ = _rand_inputs(desc, 13)
    rp, ci, _ = oracle.select(g, q, k)
    # a constant vector added to every key shifts each row by one constant
    shift = np.linspace(-0.5, 0.5, g.head_dim)
    rp2, ci2, _ = oracle.select(g, q, k + shift)
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
    # positive scaling of the queries
    rp3, ci3, _ = oracle.select(g, q * 4.0, k)
    assert np.array_equal(ci, ci3)
    # permuting tokens inside each block
    rng = np.random.default_rng(0)
    qp, kp = q.copy(), k.copy()
    for blk in range(g.nkb):
        tok = oracle.block_tokens(g, blk)
        kp[:, tok] = k[:, rng.permutation(tok)]
    for blk in range(g.nqb):
        tok = oracle.block_tokens(g, blk)
        qp[:, tok] = q[:, rng.permutation(tok)]
    rp4, ci4, _ = oracle.select(g, qp, kp)
    assert np.array_equal(ci, ci4)


# ---------------------------------------------------------------- attend
def _sdpa(q, k, v, mask=None, scale=None):
    """torch SDPA in float64 on the CPU; q/k/v [S, D] per (b, h)."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, scale=scale)[0, 0].numpy()


def test_attend_dense_special_case_equals_sdpa():
    desc = _desc("tiny", topk=8)     # k = NKB and the window covers the frame
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 17)
    rp, ci, _ = oracle.select(g, q, k)
    assert np.all(np.diff(rp) == g.nkb)
    o, lse = oracle.attend(g, q, k, v, rp, ci)
    for b in range(g.batch):
        for h in range(g.heads):
            ref = _sdpa(q[b, :, h], k[b, :, h], v[b, :, h])
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-12, atol=1e-12)
            z = (q[b, :, h] @ k[b, :, h].T) / math.sqrt(g.head_dim)
            np.testing.assert_allclose(lse[b, h], logsumexp(z, axis=1), rtol=1e-12)


@pytest.mark.parametrize("name,batch", [("tiny", 1), ("tiny_window", 1), ("small_edges", 1),
                                        ("small_16x8", 1), ("small_edges", 2)])
def test_attend_equals_token_masked_sdpa(name, batch):
    """Rows of the CSR follow select's (batch, head, query block) order; with
    two batch entries a wrong row order changes the result."""
    desc = _desc(name, batch=batch)
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 19)
    rp, ci, _ = oracle.select(g, q, k)
    o, lse = oracle.attend(g, q, k, v, rp, ci)
    qid = _token_block_ids(g, g.q_frames)
    kid = _token_block_ids(g, g.kv_frames)
    for b in range(g.batch):
        for h in range(g.heads):
            allowed = np.zeros((g.nqb, g.nkb), dtype=bool)
            for qb in range(g.nqb):
                r = (b * g.heads + h) * g.nqb + qb
                allowed[qb, ci[rp[r]:rp[r + 1]]] = True
            mask = allowed[qid][:, kid]
            ref = _sdpa(q[b, :, h], k[b, :, h], v[b, :, h], mask=mask)
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-11, atol=1e-12)
            z = (q[b, :, h] @ k[b, :, h].T) / math.sqrt(g.head_dim)
            z[~mask] = -np.inf
            np.testing.assert_allclose(lse[b, h], logsumexp(z, axis=1), rtol=1e-12)


@pytest.mark.parametrize("name", ["tiny_window", "small_edges"])
def test_attend_rows_equals_attend_on_every_row(name):
    """attend_rows decodes each CSR row r into (batch, head, query block) on
    its own; on batch-2, multi-head grids (where any other decode order
    names different tokens) it must give attend's O and LSE bit for bit on
    every row, asked for in a shuffled order with repeats, and a sample of
    its rows must equal the token-masked SDPA of that row."""
    desc = _desc(name, batch=2, heads=3)
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 41)
    rp, ci, _ = oracle.select(g, q, k)
    o, lse = oracle.attend(g, q, k, v, rp, ci)
    rows = g.batch * g.heads * g.nqb
    order = np.random.default_rng(2).permutation(rows).tolist() + [0, rows - 1, rows // 2]
    got = oracle.attend_rows(g, q, k, v, rp, ci, order)
    assert len(got) == len(order)
    seen = set()
    for r, (b, h, qtok, orow, lrow) in zip(order, got):
        qb = r % g.nqb
        assert (b, h) == divmod(r // g.nqb, g.heads)
        assert np.array_equal(qtok, oracle.block_tokens(g, qb))
        assert np.array_equal(orow, o[b, qtok, h]) and np.array_equal(lrow, lse[b, h, qtok])
        seen.add(r)
    assert seen == set(range(rows))
    qid = _token_block_ids(g, g.q_frames)
    kid = _token_block_ids(g, g.kv_frames)
    for r in [1, rows // 3, rows - 2]:
        b, h, qtok, orow, _ = oracle.attend_rows(g, q, k, v, rp, ci, [r])[0]
        allowed = np.zeros(g.nkb, dtype=bool)
        allowed[ci[rp[r]:rp[r + 1]]] = True
        qsel = qid == r % g.nqb
        ref = _sdpa(q[b, :, h], k[b, :, h], v[b, :, h], mask=np.broadcast_to(
            allowed[kid], (g.q_tokens, g.kv_tokens)).copy())[qsel]
        np.testing.assert_allclose(orow, ref, rtol=1e-11, atol=1e-12)


def test_attend_row_stochastic_and_bounded():
    desc = li.CONFIGS["small_edges"]
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 23)
    rp, ci, _ = oracle.select(g, q, k)
    ones = np.ones_like(v)
    o1, _ = oracle.attend(g, q, k, ones, rp, ci)
    np.testing.assert_allclose(o1, 1.0, rtol=0, atol=1e-13)
    o, _ = oracle.attend(g, q, k, v, rp, ci)
    for r in range(len(rp) - 1):
        b, rem = divmod(r, g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        ktok = np.concatenate([oracle.block_tokens(g, kb) for kb in ci[rp[r]:rp[r + 1]]])
        lo = v[b, ktok, h].min(axis=0)
        hi = v[b, ktok, h].max(axis=0)
        orow = o[b, oracle.block_tokens(g, qb), h]
        assert np.all(orow >= lo - 1e-12) and np.all(orow <= hi + 1e-12)


def test_attend_constant_keys_give_mean_of_values():
    desc = li.CONFIGS["tiny"]
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 29)
    k[:] = 0.25
    rp, ci, _ = oracle.select(g, q, k)
    o, _ = oracle.attend(g, q, k, v, rp, ci)
    for r in range(len(rp) - 1):
        b, rem = divmod(r, g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        ktok = np.concatenate([oracle.block_tokens(g, kb) for kb in ci[rp[r]:rp[r + 1]]])
        np.testing.assert_allclose(o[b, oracle.block_tokens(g, qb), h],
                                   np.broadcast_to(v[b, ktok, h].mean(axis=0), (g.block_tokens, g.head_dim)),
                                   rtol=1e-12, atol=1e-13)


def test_attend_empty_and_out_of_range_rows():
    desc = li.CONFIGS["tiny"]
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 31)
    rows = g.batch * g.heads * g.nqb
    rp = np.zeros(rows + 1, dtype=np.int64)
    rp[2:] = 1                       # row 1 holds one out-of-range block
    ci = np.asarray([g.nkb + 3])
    o, lse = oracle.attend(g, q, k, v, rp, ci)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_attend_permutation_inside_blocks():
    desc = li.CONFIGS["small_16x8"]
    g = oracle.geometry(desc)
    q, k, v = _rand_inputs(desc, 37)
    rp, ci, _ = oracle.select(g, q, k)
    o, _ = oracle.attend(g, q, k, v, rp, ci)
    rng = np.random.default_rng(1)
    kp, vp = k.copy(), v.copy()
    for blk in range(g.nkb):
        tok = oracle.block_tokens(g, blk)
        perm = rng.permutation(tok)
        kp[:, tok] = k[:, perm]
        vp[:, tok] = v[:, perm]
    o2, _ = oracle.attend(g, q, kp, vp, rp, ci)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------- generator
def test_generator_deterministic_and_rne():
    desc = li.CONFIGS["tiny"]
    a = li.generate(desc, seed=0)
    b = li.generate(desc, seed=0)
    c = li.generate(desc, seed=1)
    assert a.sha256 == b.sha256 and a.sha256 != c.sha256
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(li.f32_to_bf16_bits(x), ref)
    qf = li.bf16_bits_to_f32(a.q)
    assert np.all(np.abs(qf) < 4.5) and abs(float(qf.std()) - 0.87) < 0.1
