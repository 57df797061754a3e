"""Seeded synthetic inputs and workload shapes for LCSA select + attend.

This module is shared by the oracle, the tests and the bench.  It holds no
step of the attention method itself: only workload descriptors, the seeded
generator of Q/K/V, synthetic rotary-embedding tables (inputs a caller
supplies) and bf16 bit conversions.

Workloads (token grids are the latent grid after the DiT's 2x2 patching, so
a H x W output video gives a (H/16) x (W/16) token grid):

* the first chunk of the streaming pipeline is 6 latent frames and a stream
  chunk is 2 latent frames (NxDI FlashVSR contrib page, "Description");
  23040 tokens = 6 x 48 x 80 at 768x1280;
* ``topk_ratio = sparse_ratio * 768 * 1280 / (H * W)`` with sparse_ratio 1.5
  or 2.0, ``local_range`` 11 or 9 and ``kv_ratio = 3`` (FlashVSR Inference
  skill page, "Non-Negotiable Streaming Contract");
* 768x1408 is the resolution of the published end-to-end throughput figures
  (FlashVSR Hopper PR page, title and "Measured Results"; agentlens FlashVSR
  summary, "Why it matters");
* 2048x3840 is the untiled 4K example (FlashVSR+ README, "Overview" and
  "Command-Line Inference", Turbo).

Generator (identical for every workload, seed 0 by default):
  rng = numpy.random.default_rng(seed) (PCG64); draw in this order
  wt ~ U[0, pi/4), wy ~ U[0, pi/16), wx ~ U[0, pi/16), phi ~ U[0, 2 pi), each
  [H, D]; then Nq [B,Sq,H,D], Nk [B,Skv,H,D], Nv [B,Skv,H,D] standard normal
  in float32.  The shared field F(t,y,x)[h,c] = sin(wt t + wy y + wx x + phi)
  is evaluated in float64 at the absolute KV-frame index t (queries sit in the
  last q_frames KV frames).  Q = bf16(f32(0.5 Nq + F_q)), K and V likewise
  with F_kv; both roundings are round-to-nearest-even.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

SPARSE_RES = 768 * 1280


def _topk_ratio(sparse_ratio: float, h_px: int, w_px: int) -> float:
    return sparse_ratio * SPARSE_RES / (h_px * w_px)


def _desc(**kw):
    d = dict(batch=1, heads=12, head_dim=128, grid_h=48, grid_w=80, q_frames=6,
             cached_frames=0, kv_ratio=3.0, block_t=0, block_h=0, block_w=0,
             local_range=11, topk_ratio=0.0, topk=0, scale=0.0)
    d.update(kw)
    return d


# The five workloads of the method at their real shapes plus small grids that
# exercise window edges, short rows and the 16x8 block shape.
CONFIGS = {
    # 2 latent frames of 16x16 tokens, 8x8-token blocks, window 3, keep 4.
    "tiny": _desc(heads=2, grid_h=16, grid_w=16, q_frames=2, block_t=1,
                  block_h=8, block_w=8, local_range=3, topk=4),
    # First chunk at 768x1280: 6 x 48 x 80 = 23040 tokens, sparse_ratio 2.0.
    "first_768x1280": _desc(grid_h=48, grid_w=80, q_frames=6,
                            topk_ratio=_topk_ratio(2.0, 768, 1280)),
    # Stream chunk at 768x1280: 2 query frames, 4 cached, kv_ratio 3 -> 6.
    "stream_768x1280": _desc(grid_h=48, grid_w=80, q_frames=2, cached_frames=4,
                             topk_ratio=_topk_ratio(1.5, 768, 1280)),
    # First chunk at 768x1408: 6 x 48 x 88 = 25344 tokens, local_range 9.
    "first_768x1408": _desc(grid_h=48, grid_w=88, q_frames=6, local_range=9,
                            topk_ratio=_topk_ratio(1.5, 768, 1408)),
    # Untiled 4K-class first chunk: 6 x 128 x 240 = 184320 tokens.
    "first_2048x3840": _desc(grid_h=128, grid_w=240, q_frames=6,
                             topk_ratio=_topk_ratio(1.5, 2048, 3840)),
    # Small grids (not page workloads): window edges and rows shorter than k.
    "tiny_window": _desc(heads=2, grid_h=64, grid_w=64, q_frames=1, block_t=1,
                         block_h=8, block_w=8, local_range=3, topk=6),
    "small_edges": _desc(heads=3, grid_h=32, grid_w=64, q_frames=2,
                         cached_frames=1, kv_ratio=1.5, local_range=3, topk=10),
    "small_16x8": _desc(heads=2, grid_h=32, grid_w=24, q_frames=2,
                        local_range=3, topk=5),
}

# The five workloads named by the method's deployment, in order.
PAGE_WORKLOADS = ["tiny", "first_768x1280", "stream_768x1280",
                  "first_768x1408", "first_2048x3840"]


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# --------------------------------------------------------------- generator
@dataclass
class Inputs:
    q: np.ndarray  # uint16 bf16 bits [B, Sq, H, D]
    k: np.ndarray  # uint16 bf16 bits [B, Skv, H, D]
    v: np.ndarray  # uint16 bf16 bits [B, Skv, H, D]
    kv_frames: int
    sha256: str


def kv_frames_of(desc: dict) -> int:
    """Number of latent frames in the KV window (the streaming contract keeps
    at most ceil(kv_ratio * q_frames) frames; no cache means q_frames)."""
    q, c, r = desc["q_frames"], desc["cached_frames"], desc["kv_ratio"]
    if r <= 0:
        return q + c
    x = r * q
    n = round(x)
    cap = int(n) if abs(x - n) < 1e-9 else int(math.ceil(x))
    return min(q + c, cap)


def _field_frame(t: int, grid_h: int, grid_w: int, wt, wy, wx, phi) -> np.ndarray:
    y = np.arange(grid_h, dtype=np.float64)[:, None, None, None]
    x = np.arange(grid_w, dtype=np.float64)[None, :, None, None]
    ph = wt * float(t) + phi
    return np.sin(ph[None, None] + wy[None, None] * y + wx[None, None] * x)


def generate(desc: dict, seed: int = 0) -> Inputs:
    """Seeded bf16 Q/K/V of the workload's shape in raster [B, S, H, D]."""
    B, H, D = desc["batch"], desc["heads"], desc["head_dim"]
    gh, gw, qf = desc["grid_h"], desc["grid_w"], desc["q_frames"]
    kvf = kv_frames_of(desc)
    fs = gh * gw
    sq, skv = qf * fs, kvf * fs
    rng = np.random.default_rng(seed)
    wt = rng.uniform(0.0, math.pi / 4, size=(H, D))
    wy = rng.uniform(0.0, math.pi / 16, size=(H, D))
    wx = rng.uniform(0.0, math.pi / 16, size=(H, D))
    phi = rng.uniform(0.0, 2 * math.pi, size=(H, D))
    noise = {name: rng.standard_normal(size=(B, n, H, D), dtype=np.float32)
             for name, n in (("q", sq), ("k", skv), ("v", skv))}
    out = {name: np.empty(noise[name].shape, dtype=np.uint16) for name in noise}
    q0 = kvf - qf                      # first query frame inside the KV window
    rows_per_piece = max(1, (1 << 21) // (H * D))

    def one_frame(t):
        fld = _field_frame(t, gh, gw, wt, wy, wx, phi).reshape(fs, H, D)
        targets = [("k", t), ("v", t)] + ([("q", t - q0)] if t >= q0 else [])
        for r0 in range(0, fs, rows_per_piece):
            r1 = min(fs, r0 + rows_per_piece)
            for name, f in targets:
                sl = slice(f * fs + r0, f * fs + r1)
                for b in range(B):
                    val = 0.5 * noise[name][b, sl].astype(np.float64) + fld[r0:r1]
                    out[name][b, sl] = f32_to_bf16_bits(val.astype(np.float32))

    workers = max(1, min(kvf, len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one_frame, range(kvf)))
    del noise
    h = hashlib.sha256()
    for name in ("q", "k", "v"):
        h.update(out[name].tobytes())
    return Inputs(q=out["q"], k=out["k"], v=out["v"], kv_frames=kvf, sha256=h.hexdigest())


# ------------------------------------------------------------ RoPE tables
def rope_tables(desc: dict, pairs=(22, 21, 21), base: float = 10000.0, frame_offset: int = 0):
    """Synthetic cos/sin tables of a factored 3D rotary embedding, as a caller
    would supply them: for axis a with n pairs, pair j turns by
    pos * base**(-j / n) radians at axis position pos (the frame index is
    frame_offset + window frame).  Returns float32 arrays t [kv_frames, pt, 2],
    h [grid_h, ph, 2], w [grid_w, pw, 2] of (cos, sin).  The 22/21/21 split
    of head_dim 128 gives the spare pair to the time axis."""
    kvf = kv_frames_of(desc)

    def table(positions, n):
        ang = np.asarray(positions, dtype=np.float64)[:, None] * base ** (-np.arange(n) / n)[None, :]
        return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)

    pt, ph, pw = pairs
    return {"t": table(frame_offset + np.arange(kvf), pt),
            "h": table(np.arange(desc["grid_h"]), ph),
            "w": table(np.arange(desc["grid_w"]), pw)}
