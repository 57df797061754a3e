"""Pins of the threshold-reuse oracle (oracle/threshold_oracle.py): with the
thresholds of the same chunk and no ties it reproduces the exact top-k; it is
monotone in the thresholds; -inf keeps every window block and +inf none; the
thresholds are the keep-th largest window scores (brute force over the
sorted window on a tiny grid); the padded layout holds each row's blocks
first.  CPU only."""
import numpy as np
import pytest

import lcsa_inputs as li
import oracle


def _scores(name, seed=0, batch=None):
    desc = dict(li.CONFIGS[name])
    if batch is not None:
        desc["batch"] = batch
    g = oracle.geometry(desc)
    inp = li.generate(desc, seed=seed)
    q, k = li.bf16_bits_to_f64(inp.q), li.bf16_bits_to_f64(inp.k)
    rp, ci, s = oracle.select(g, q, k)
    return g, rp, ci, s


def test_own_thresholds_reproduce_top_k():
    for name, batch in (("tiny", None), ("tiny_window", None), ("small_edges", None),
                        ("small_16x8", None), ("tiny", 2)):
        g, rp, ci, s = _scores(name, batch=batch)
        tau = oracle.row_thresholds(g, s)
        rows = oracle.select_threshold(g, s, tau)
        for r, blocks in enumerate(rows):
            assert np.array_equal(blocks, ci[rp[r]:rp[r + 1]]), f"{name} row {r}"


@pytest.mark.parametrize("name,batch", [("tiny_window", None), ("tiny", 2)])
def test_thresholds_are_kth_scores_by_brute_force(name, batch):
    # thresholds are indexed by CSR row (b, h, query block); batch 2 tells
    # that order from (h, b, query block)
    g, rp, ci, s = _scores(name, batch=batch)
    tau = oracle.row_thresholds(g, s)
    for r in range(len(rp) - 1):
        b, rem = divmod(r, g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        e = oracle.window(g, qb)
        vals = s[b, h, qb, e]
        keep = min(g.k, len(e))
        # exactly `keep` window scores are >= tau (no ties in these inputs) and
        # tau is one of them
        assert np.sum(vals >= tau[r]) == keep and tau[r] in vals
        if keep < len(e):
            assert np.sum(vals > tau[r]) == keep - 1


def test_extreme_and_monotone_thresholds():
    g, rp, ci, s = _scores("small_edges")
    n = len(rp) - 1
    every = oracle.select_threshold(g, s, np.full(n, -np.inf))
    none = oracle.select_threshold(g, s, np.full(n, np.inf))
    for r in range(n):
        qb = r % g.nqb
        assert np.array_equal(every[r], oracle.window(g, qb)) and len(none[r]) == 0
    tau = oracle.row_thresholds(g, s)
    lo = oracle.select_threshold(g, s, tau - 0.5)
    hi = oracle.select_threshold(g, s, tau + 0.5)
    for r in range(n):
        assert set(hi[r].tolist()) <= set(ci[rp[r]:rp[r + 1]].tolist()) <= set(lo[r].tolist())
        assert np.all(np.diff(lo[r]) > 0)


def test_ties_at_the_threshold_are_all_kept():
    g, rp, ci, s = _scores("tiny")
    s = s.copy()
    e = oracle.window(g, 0)
    s[0, 0, 0, e] = 1.0                      # every block of row 0 ties
    tau = oracle.row_thresholds(g, s)
    rows = oracle.select_threshold(g, s, tau)
    assert np.array_equal(rows[0], e)        # top-k would keep k of them, by index


def test_padded_layout():
    g, rp, ci, s = _scores("tiny_window")
    tau = oracle.row_thresholds(g, s) + 0.25
    rows = oracle.select_threshold(g, s, tau)
    rpp, cip = oracle.padded_csr(g, rows)
    w = max(len(oracle.window(g, qb)) for qb in range(g.nqb))
    assert np.array_equal(rpp, np.arange(len(rows) + 1) * w)
    for r, blocks in enumerate(rows):
        seg = cip[rpp[r]:rpp[r + 1]]
        assert np.array_equal(seg[:len(blocks)], blocks) and np.all(seg[len(blocks):] == -1)
