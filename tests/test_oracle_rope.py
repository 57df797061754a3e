"""Pins of the RoPE oracle (oracle/rope_oracle.py) against what the
mathematics fixes: the bf16 rounding against an independent float32 routine
and a double-rounding case, the pair rotation against numpy's complex
multiplication, special angles, norm preservation, and which axis position
and channel pairs each token uses (tables that turn one axis position only).
CPU only."""
import numpy as np
import pytest

import lcsa_inputs as li
import oracle


def _bf16_values(rng, shape):
    return li.bf16_bits_to_f64(li.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)))


def _identity_tables(desc, pairs=(22, 21, 21)):
    g = oracle.geometry(desc)

    def ident(n, m):
        t = np.zeros((n, m, 2), dtype=np.float32)
        t[..., 0] = 1.0
        return t
    return oracle.RopeTables(t=ident(g.kv_frames, pairs[0]), h=ident(g.grid_h, pairs[1]),
                             w=ident(g.grid_w, pairs[2]))


def test_round_bf16_matches_float32_rounding():
    """On float32 values the one-step rounding must agree bit for bit with
    the float32 -> bf16 round-to-nearest-even of the input generator."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-3,
                        rng.standard_normal(2000) * 1e3]).astype(np.float32)
    # exact ties and their neighbours
    base = li.bf16_bits_to_f32(np.arange(0x3F80, 0x3F90, dtype=np.uint16))
    x = np.concatenate([x, base + np.float32(2.0 ** -8), base - np.float32(2.0 ** -8)])
    want = li.bf16_bits_to_f64(li.f32_to_bf16_bits(x))
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_rounds_once_from_float64():
    # 1 + 2^-8 + 2^-30 lies just above the tie between 1 and 1 + 2^-7: one
    # rounding gives 1 + 2^-7, rounding through float32 first would give 1.
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8,
                  -(1 + 2.0 ** -8 + 2.0 ** -40), 3.0])
    assert oracle.round_bf16(x).tolist() == [1 + 2.0 ** -7, 1.0, 1 + 2.0 ** -6, -(1 + 2.0 ** -7), 3.0]


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(5)
    x = _bf16_values(rng, (7, 128))
    ang = rng.uniform(-np.pi, np.pi, size=(7, 64))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    r = oracle.rotate_pairs(x, c, s)
    # bf16 x float32 products are exact in float64, so both round once per sum
    assert np.array_equal(r[:, 0::2], z.real) and np.array_equal(r[:, 1::2], z.imag)


def test_special_angles():
    rng = np.random.default_rng(6)
    x = _bf16_values(rng, (5, 128))
    one, zero = np.ones((5, 64), np.float32), np.zeros((5, 64), np.float32)
    assert np.array_equal(oracle.rotate_pairs(x, one, zero), x)
    quarter = oracle.rotate_pairs(x, zero, one)                 # 90 degrees
    assert np.array_equal(quarter[:, 0::2], -x[:, 1::2]) and np.array_equal(quarter[:, 1::2], x[:, 0::2])
    half = oracle.rotate_pairs(x, -one, zero)                   # 180 degrees
    assert np.array_equal(half, -x)


def test_rotation_preserves_pair_norms():
    desc = dict(li.CONFIGS["small_edges"])
    g = oracle.geometry(desc)
    inp = li.generate(desc)
    t = li.rope_tables(desc)
    tab = oracle.RopeTables(t=t["t"], h=t["h"], w=t["w"])
    k = li.bf16_bits_to_f64(inp.k)
    for rnd, tol in ((False, 1e-6), (True, 2.0 ** -7)):
        r = oracle.rope_k(g, k, tab, round_out=rnd)
        n0 = np.hypot(k[..., 0::2], k[..., 1::2])
        n1 = np.hypot(r[..., 0::2], r[..., 1::2])
        big = n0 > 1e-3
        assert np.max(np.abs(n1[big] - n0[big]) / n0[big]) <= tol


@pytest.mark.parametrize("axis", ["t", "h", "w"])
def test_each_axis_turns_its_own_pairs_at_its_own_positions(axis):
    """Tables that turn one position of one axis by 90 degrees and leave the
    rest alone: exactly the tokens at that position change, and only in that
    axis's channel pairs."""
    desc = dict(li.CONFIGS["small_edges"])          # 3 KV frames, 32 x 64 tokens
    g = oracle.geometry(desc)
    tab = _identity_tables(desc)
    pos = {"t": 1, "h": 5, "w": 9}[axis]
    getattr(tab, axis)[pos, :, 0] = 0.0
    getattr(tab, axis)[pos, :, 1] = 1.0
    pt, ph, pw = tab.pairs
    pair_range = {"t": (0, pt), "h": (pt, pt + ph), "w": (pt + ph, 64)}[axis]
    rng = np.random.default_rng(8)
    k = _bf16_values(rng, (1, g.kv_tokens, 2, 128))
    r = oracle.rope_k(g, k, tab)
    s = np.arange(g.kv_tokens)
    coord = {"t": s // (g.grid_h * g.grid_w), "h": (s // g.grid_w) % g.grid_h, "w": s % g.grid_w}[axis]
    hit = coord == pos
    j0, j1 = pair_range
    want = k.copy()
    want[:, hit, :, 2 * j0:2 * j1:2] = -k[:, hit, :, 2 * j0 + 1:2 * j1:2]
    want[:, hit, :, 2 * j0 + 1:2 * j1:2] = k[:, hit, :, 2 * j0:2 * j1:2]
    assert np.array_equal(r, want)


def test_queries_use_their_kv_window_frame():
    """Stream chunk: 2 query frames at the end of a 6-frame window, so query
    frame 0 is window frame 4."""
    desc = dict(li.CONFIGS["small_edges"], q_frames=2, cached_frames=4, kv_ratio=3.0)
    g = oracle.geometry(desc)
    assert g.kv_frames == 6
    tab = _identity_tables(desc)
    tab.t[4, :, 0] = -1.0                              # 180 degrees at window frame 4
    rng = np.random.default_rng(9)
    q = _bf16_values(rng, (1, g.q_tokens, 1, 128))
    r = oracle.rope_q(g, q, tab)
    fs = g.grid_h * g.grid_w
    pt = tab.pairs[0]
    assert np.array_equal(r[:, :fs, :, :2 * pt], -q[:, :fs, :, :2 * pt])
    assert np.array_equal(r[:, :fs, :, 2 * pt:], q[:, :fs, :, 2 * pt:])
    assert np.array_equal(r[:, fs:], q[:, fs:])


def test_relative_positions_on_one_axis():
    """Unrounded rotation by angles pos * w: the score of a rotated query and
    key depends only on their position difference."""
    desc = dict(li.CONFIGS["small_edges"])
    g = oracle.geometry(desc)
    t = li.rope_tables(desc)
    tab = oracle.RopeTables(t=t["t"], h=t["h"], w=t["w"])
    rng = np.random.default_rng(10)
    q = _bf16_values(rng, (1, 1, 1, 128))
    k = _bf16_values(rng, (1, 1, 1, 128))

    def at(x, frame, y, xx):
        c, s = oracle.rope_oracle._angles(tab, np.array([frame]), np.array([y]), np.array([xx]))
        return oracle.rotate_pairs(x, c[None, :, None, :], s[None, :, None, :]).ravel()
    # angles are float32-rounded cos/sin of pos * w, hence the tolerance
    a = at(q, 0, 3, 5) @ at(k, 1, 7, 6)
    b = at(q, 1, 10, 20) @ at(k, 2, 14, 21)
    assert abs(a - b) <= 1e-5 * (np.abs(q).sum() * np.abs(k).max())
