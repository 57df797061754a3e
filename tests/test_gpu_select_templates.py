"""Select parity on small grids chosen to reach every compiled width of the
select kernel: window candidates per lane M in {1, 2, 3, 4, 6, 8, 12, 16}
and query frames per workgroup R in {1, 2, 4, 6, 8}, including a partly
filled last frame group, more rows than waves and the largest window the
kernel takes (1024 candidates, with k = 300 and k = 1023).  Scores must match the
float64 oracle to 1e-12 of the row scale and masks must be identical except
at near-ties, as in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle
from gpu_util import check_mask, say, to_device_bf16

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)


def _desc(q_frames, cached, kv_ratio, nb, local_range, topk):
    """2 heads, 8x8-token blocks, an nb x nb block grid per frame."""
    return dict(batch=1, heads=2, head_dim=128, grid_h=8 * nb, grid_w=8 * nb, q_frames=q_frames,
                cached_frames=cached, kv_ratio=kv_ratio, block_t=1, block_h=8, block_w=8,
                local_range=local_range, topk_ratio=0.0, topk=topk, scale=0.0)


# (label, desc, expected M, expected R)
CASES = [
    ("m16_r8", _desc(8, 0, 1.0, 11, 11, 50), 16, 8),     # 8 KV frames x 11x11 = 968 candidates
    # the largest window the select kernel takes: 16 KV frames x 8x8 = 1024
    ("m16_full_window", _desc(8, 8, 2.0, 8, 15, 300), 16, 8),
    ("m16_full_window_all_but_one", _desc(8, 8, 2.0, 8, 15, 1023), 16, 8),
    ("m12_r4", _desc(4, 2, 1.5, 11, 11, 60), 12, 4),     # 6 x 121 = 726
    ("m8_r2", _desc(2, 2, 2.0, 11, 11, 40), 8, 2),       # 4 x 121 = 484
    ("m6_r1", _desc(1, 2, 3.0, 11, 11, 30), 6, 1),       # 3 x 121 = 363
    ("m4_r6", _desc(6, 0, 1.0, 6, 11, 20), 4, 6),        # 6 x 36 = 216
    ("m3_r8_two_groups", _desc(10, 0, 1.0, 4, 11, 12), 3, 8),   # 10 x 16 = 160; groups of 8 and 2
    ("m2_r8", _desc(8, 0, 1.0, 4, 11, 9), 2, 8),         # 8 x 16 = 128
    ("m1_r4_partial", _desc(3, 1, 4.0 / 3.0, 4, 3, 5), 1, 4),   # 4 x (3x3 at most) <= 64; 3 of 4 rows
]


def _expected_mr(info, q_frames):
    m = (info["max_window"] + 63) // 64
    m = next(w for w in (1, 2, 3, 4, 6, 8, 12, 16) if w >= m)
    r = 1 if q_frames <= 1 else 2 if q_frames <= 2 else 4 if q_frames <= 4 else 6 if q_frames <= 6 else 8
    return m, r


@pytest.mark.parametrize("label,desc,m_want,r_want", CASES, ids=[c[0] for c in CASES])
def test_select_template_parity(label, desc, m_want, r_want):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    plan = lcsa.Plan.from_desc(desc)
    info = plan.info
    assert _expected_mr(info, desc["q_frames"]) == (m_want, r_want), (label, info["max_window"])
    say(f"[gpu] select template {label}: window {info['min_window']}..{info['max_window']}, "
        f"k {info['k']}, rows {info['rows']}")
    inp = li.generate(desc, seed=3)
    q, k = to_device_bf16(inp.q), to_device_bf16(inp.k)
    rp, ci, sc = lcsa.select(plan, q, k, return_scores=True)
    torch.cuda.synchronize()
    g = oracle.geometry(desc)
    rp_ref, ci_ref, s_ref = oracle.select(g, li.bf16_bits_to_f64(inp.q), li.bf16_bits_to_f64(inp.k))
    s_gpu = sc.cpu().numpy()
    assert np.array_equal(np.isneginf(s_gpu), np.isneginf(s_ref))
    fin = np.isfinite(s_ref)
    assert float(np.abs(s_gpu[fin] - s_ref[fin]).max()) <= 1e-12 * float(np.abs(s_ref[fin]).max())
    mism, ties = check_mask(g, rp_ref, ci_ref, s_ref, rp.cpu().numpy(), ci.cpu().numpy())
    say(f"  mask mismatches {len(mism)}, all near-ties ({len(ties)})")


@pytest.mark.parametrize("label,desc,m_want,r_want", CASES, ids=[c[0] for c in CASES])
def test_threshold_modes_every_template(label, desc, m_want, r_want):
    """The k-th score output and the threshold selection in every compiled
    width: steady thresholds equal the oracle's (1e-12 of the score scale),
    and thresholds of another chunk (seed 4) select exactly the oracle's
    blocks except within 1e-9 of the scale of a threshold, padded with -1."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    plan = lcsa.Plan.from_desc(desc)
    info = plan.info
    say(f"[gpu] threshold modes {label}: window {info['min_window']}..{info['max_window']}")
    g = oracle.geometry(desc)
    inp = li.generate(desc, seed=3)
    q, k = to_device_bf16(inp.q), to_device_bf16(inp.k)
    _, _, s_ref = oracle.select(g, li.bf16_bits_to_f64(inp.q), li.bf16_bits_to_f64(inp.k))
    inp1 = li.generate(desc, seed=4)
    _, _, s1 = oracle.select(g, li.bf16_bits_to_f64(inp1.q), li.bf16_bits_to_f64(inp1.k))
    _, _, kth = lcsa.select_steady(plan, q, k)
    tau = oracle.row_thresholds(g, s1)
    rp, ci = lcsa.select_reuse(plan, q, k, torch.from_numpy(tau).cuda())
    torch.cuda.synchronize()
    scale = float(np.abs(s_ref[np.isfinite(s_ref)]).max())
    assert float(np.abs(kth.cpu().numpy() - oracle.row_thresholds(g, s_ref)).max()) <= 1e-12 * scale
    pad = info["max_window"]
    rows_ref = oracle.select_threshold(g, s_ref, tau)
    rp_ref, ci_ref = oracle.padded_csr(g, rows_ref)
    assert np.array_equal(rp.cpu().numpy(), rp_ref)
    ci_h = ci.cpu().numpy().astype(np.int64)
    for r, want in enumerate(rows_ref):
        seg = ci_h[r * pad:(r + 1) * pad]
        got = seg[seg >= 0]
        assert np.all(seg[len(got):] == -1)
        if not np.array_equal(got, want):
            b, rem = divmod(r, g.heads * g.nqb)
            h, qb = divmod(rem, g.nqb)
            for kb in set(got.tolist()) ^ set(want.tolist()):
                assert abs(s_ref[b, h, qb, kb] - tau[r]) <= 1e-9 * scale, f"{label} row {r}"
