"""Plain CPU oracle of the factored 3D rotary position embedding (RoPE) of Q
and K that precedes LCSA select, in float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests, the smoke check and the bench's CPU-baseline leg
do.  It shares no code with the HIP library.

What the pages state:

* The DiT applies a factored 3D RoPE to its queries and keys (NxDI FlashVSR
  contrib page, "Model Information").
* Applying RoPE is part of the attention glue that moves data around the
  sparse kernel on every chunk (FlashVSR Hopper PR page, "What Was Actually
  Slow"), and that page's fix list names a coalesced RoPE kernel ("How I
  Fixed It").

The pages do not write the rotation out.  Reading taken here (R10, listed
with the others in the design notes):

  R10 Channel pairs (2j, 2j + 1), j < head_dim / 2, are complex numbers.
      Pairs [0, pt) turn by an angle set by the token's KV-window frame,
      pairs [pt, pt + ph) by one set by its token row and pairs
      [pt + ph, head_dim / 2) by one set by its token column ("factored 3D").
      The angles enter as cos/sin tables per axis position (float32, given
      by the caller), so the frequencies and the split are the caller's.
      A query of query frame tq sits in KV-window frame
      kv_frames - q_frames + tq (reading R6).  Each rotated value is rounded
      to bf16 (nearest, ties to even) once, from its float64 value: the DiT's
      rotated Q and K are bf16 tensors, and pooling, scoring and attention
      all see exactly those values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["RopeTables", "round_bf16", "rotate_pairs", "rope_q", "rope_k", "token_positions"]


@dataclass(frozen=True)
class RopeTables:
    """cos/sin per axis position and channel pair, float32 [positions, pairs, 2]."""
    t: np.ndarray     # [kv_frames, pt, 2]
    h: np.ndarray     # [grid_h, ph, 2]
    w: np.ndarray     # [grid_w, pw, 2]

    @property
    def pairs(self) -> tuple[int, int, int]:
        return self.t.shape[1], self.h.shape[1], self.w.shape[1]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even, in
    one step from the float64 value (no intermediate float32 rounding).
    bf16 keeps 7 of float64's 52 fraction bits, so the low 45 bits go."""
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    drop = np.uint64(45)
    lsb = (b >> drop) & np.uint64(1)
    half_minus_one = np.uint64((1 << 44) - 1)
    mask = np.uint64(0xFFFFFFFFFFFFFFFF ^ ((1 << 45) - 1))
    return ((b + half_minus_one + lsb) & mask).view(np.float64).reshape(np.shape(x))


def rotate_pairs(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Turn each channel pair (x[2j], x[2j+1]) by the angle with the given
    cosine and sine: (x0 cos - x1 sin, x0 sin + x1 cos), in float64.
    x: [..., D]; cos, sin: broadcastable to [..., D/2]."""
    x0 = x[..., 0::2].astype(np.float64)
    x1 = x[..., 1::2].astype(np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def token_positions(n_tokens: int, grid_h: int, grid_w: int, frame0: int):
    """(KV-window frame, token row, token column) of raster tokens 0..n-1
    whose first frame is window frame frame0."""
    s = np.arange(n_tokens)
    per = grid_h * grid_w
    return frame0 + s // per, (s // grid_w) % grid_h, s % grid_w


def _angles(tab: RopeTables, pos_t, pos_h, pos_w):
    """cos and sin [S, D/2] of every token and channel pair (reading R10)."""
    pt, ph, pw = tab.pairs
    cs = np.concatenate([tab.t[pos_t], tab.h[pos_h], tab.w[pos_w]], axis=1)   # [S, D/2, 2]
    assert cs.shape[1] == pt + ph + pw
    return cs[..., 0], cs[..., 1]


def _rope(x: np.ndarray, tab: RopeTables, grid_h: int, grid_w: int, frame0: int, round_out: bool):
    B, S, H, D = x.shape
    if sum(tab.pairs) * 2 != D:
        raise ValueError("channel pairs of the three axes must cover head_dim")
    pos_t, pos_h, pos_w = token_positions(S, grid_h, grid_w, frame0)
    c, s = _angles(tab, pos_t, pos_h, pos_w)
    r = rotate_pairs(x, c[None, :, None, :], s[None, :, None, :])
    return round_bf16(r) if round_out else r


def rope_q(g, q: np.ndarray, tab: RopeTables, round_out: bool = True) -> np.ndarray:
    """Rotated queries [B, Sq, H, D]: query frame tq is KV-window frame
    kv_frames - q_frames + tq."""
    return _rope(q, tab, g.grid_h, g.grid_w, g.kv_frames - g.q_frames, round_out)


def rope_k(g, k: np.ndarray, tab: RopeTables, round_out: bool = True) -> np.ndarray:
    """Rotated keys [B, Skv, H, D] of the KV window."""
    return _rope(k, tab, g.grid_h, g.grid_w, 0, round_out)
