"""Select and attend parity on seeded random small configurations: batch
1-2, 1-3 heads, 64- and 128-token block shapes, 1-6 x 1-6 block grids, 1-4
query frames with 0-3 cached frames, self-attention or kv_ratio 1-3, window
widths 1-7 blocks and budgets from 1 to beyond the window size.  Each case
is checked against the float64 oracle: masks identical except at
near-ties, attention within the parity bar on the GPU's mask."""
import numpy as np
import pytest
import torch

import lcsa_inputs as li
import oracle
from gpu_util import bf16_to_np, check_mask, compare_output, say, to_device_bf16

pytestmark = pytest.mark.gpu

import block_sparse_attention_lcsa_amd as lcsa  # noqa: E402  (fails loudly if not built)

SHAPES = [(8, 8), (8, 16), (16, 8), (4, 16), (16, 4), (2, 32), (32, 4)]


def random_desc(rng):
    bh, bw = SHAPES[rng.integers(len(SHAPES))]
    nbh, nbw = int(rng.integers(1, 7)), int(rng.integers(1, 7))
    q_frames = int(rng.integers(1, 5))
    cached = int(rng.integers(0, 4))
    kv_ratio = float(rng.choice([0.0, 1.0, 1.5, 2.0, 3.0]))
    local_range = int(rng.choice([1, 3, 5, 7]))
    nbf = nbh * nbw
    topk = int(rng.integers(1, nbf * (q_frames + cached) + 4))
    return dict(batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 4)), head_dim=128,
                grid_h=bh * nbh, grid_w=bw * nbw, q_frames=q_frames, cached_frames=cached,
                kv_ratio=kv_ratio, block_t=1, block_h=bh, block_w=bw, local_range=local_range,
                topk_ratio=0.0, topk=topk, scale=0.0)


CASES = [random_desc(np.random.default_rng(1000 + i)) for i in range(16)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_config_parity(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    desc = CASES[case]
    plan = lcsa.Plan.from_desc(desc)
    info = plan.info
    say(f"[gpu] random case {case}: {desc['batch']}x{desc['heads']} heads, block "
        f"{desc['block_h']}x{desc['block_w']}, grid {info['nbh']}x{info['nbw']}, "
        f"q {desc['q_frames']} kv {info['kv_frames']}, local_range {desc['local_range']}, "
        f"topk {desc['topk']}, window {info['min_window']}..{info['max_window']}")
    inp = li.generate(desc, seed=case)
    q, k, v = (to_device_bf16(x) for x in (inp.q, inp.k, inp.v))
    rp, ci = lcsa.select(plan, q, k)
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    torch.cuda.synchronize()
    g = oracle.geometry(desc)
    qf, kf, vf = (li.bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    rp_ref, ci_ref, s_ref = oracle.select(g, qf, kf)
    rp_g, ci_g = rp.cpu().numpy(), ci.cpu().numpy()
    check_mask(g, rp_ref, ci_ref, s_ref, rp_g, ci_g)
    o_ref, lse_ref = oracle.attend(g, qf, kf, vf, rp_g.astype(np.int64), ci_g.astype(np.int64))
    compare_output(bf16_to_np(o), o_ref, f"random case {case}")
    lse_h = lse.cpu().numpy()
    assert np.all(np.abs(lse_h - lse_ref) <= 2e-3 * np.maximum(1.0, np.abs(lse_ref)))


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_config_threshold_reuse(case):
    """Threshold reuse on the same random configurations: the oracle's
    thresholds of another chunk (seed + 100) select exactly the oracle's
    blocks (up to 1e-9 of the score scale of a threshold), and attention on
    the padded CSR meets the parity bar against the oracle on that mask."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    desc = CASES[case]
    plan = lcsa.Plan.from_desc(desc)
    info = plan.info
    say(f"[gpu] random reuse case {case}: window {info['min_window']}..{info['max_window']}, "
        f"rows {info['rows']}")
    g = oracle.geometry(desc)
    inp = li.generate(desc, seed=case)
    inp1 = li.generate(desc, seed=case + 100)
    qf, kf, vf = (li.bf16_bits_to_f64(x) for x in (inp.q, inp.k, inp.v))
    _, _, s_ref = oracle.select(g, qf, kf)
    _, _, s1 = oracle.select(g, li.bf16_bits_to_f64(inp1.q), li.bf16_bits_to_f64(inp1.k))
    tau = oracle.row_thresholds(g, s1)
    q, k, v = (to_device_bf16(x) for x in (inp.q, inp.k, inp.v))
    rp, ci = lcsa.select_reuse(plan, q, k, torch.from_numpy(tau).cuda())
    o, lse = lcsa.attend(plan, q, k, v, rp, ci, return_lse=True)
    torch.cuda.synchronize()
    pad = info["max_window"]
    rows_ref = oracle.select_threshold(g, s_ref, tau)
    rp_h, ci_h = rp.cpu().numpy().astype(np.int64), ci.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp_h, np.arange(info["rows"] + 1) * pad)
    scale = float(np.abs(s_ref[np.isfinite(s_ref)]).max())
    for r, want in enumerate(rows_ref):
        seg = ci_h[r * pad:(r + 1) * pad]
        got = seg[seg >= 0]
        assert np.all(seg[len(got):] == -1) and np.all(np.diff(got) > 0)
        if not np.array_equal(got, want):
            b, rem = divmod(r, g.heads * g.nqb)
            h, qb = divmod(rem, g.nqb)
            for kb in set(got.tolist()) ^ set(want.tolist()):
                assert abs(s_ref[b, h, qb, kb] - tau[r]) <= 1e-9 * scale, f"case {case} row {r}"
    o_ref, lse_ref = oracle.attend(g, qf, kf, vf, rp_h, ci_h)
    compare_output(bf16_to_np(o), o_ref, f"random reuse case {case}")
    lse_h = lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse_h), np.isneginf(lse_ref))
    assert np.all(np.abs(lse_h[fin] - lse_ref[fin]) <= 2e-3 * np.maximum(1.0, np.abs(lse_ref[fin])))
