"""Plain CPU oracle of LCSA (locality-constrained sparse attention): block
selection and block-sparse attention, in float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests, the smoke check and the bench's CPU-baseline leg
do.  It shares no code with the HIP library: the only common dependency is
the seeded input generator in ``lcsa_inputs`` (shapes and random numbers, no
step of the method).

What the method computes, and where it is stated:

* LCSA restricts each query's attention to spatially local patches of the
  latent token grid and keeps only the most relevant key blocks (agentlens
  FlashVSR summary, "How it works", item 2; "Why it matters", Scalability).
* The attention glue around the block-sparse kernel is pooling, mask
  selection and KV concatenation, and the mask is built as a CSR structure
  (FlashVSR Hopper PR page, "What Was Actually Slow" and "Rebuild sparse
  attention for Hopper").
* The controls are ``topk_ratio = sparse_ratio * 768 * 1280 / (H * W)``,
  ``local_range`` (11 or 9) and ``kv_ratio = 3`` (FlashVSR Inference skill
  page, "Non-Negotiable Streaming Contract").
* The first chunk is 6 latent frames, stream chunks are 2 (NxDI FlashVSR
  contrib page, "Description"); DiT heads are 12 x 128 ("Model Information").

The pages never write the selection out step by step.  Readings taken where
they are silent (each is also listed with its reason in the design notes):

  R1 block = 1 latent frame x bh x bw tokens; auto shape 8x16, else 16x8.
  R2 k = round-half-up(topk_ratio * blocks_per_frame), values within 1e-9 of
     an integer snap to it; an explicit ``topk`` overrides; each row keeps
     min(k, |window|) blocks.
  R3 the window of query block (t, by, bx) is every KV frame and the
     block rows/columns within local_range // 2 of (by, bx).
  R4 pooling is the arithmetic mean of the block's tokens; score = dot of the
     pooled query and pooled key (no softmax, no scale: neither moves top-k).
  R5 ties go to the lower key-block index; selected blocks are emitted in
     ascending index order.
  R6 no causal mask; queries are the last q_frames KV frames and see all
     selected blocks.
  R7 kv_frames = min(cached + q_frames, ceil(kv_ratio * q_frames)).
  R8 attention: z = scale * q.k with scale = 1/sqrt(head_dim); natural-base
     softmax over the tokens of the selected blocks; LSE = m + ln(sum).
  R9 a row with no valid key block gives O = 0 and LSE = -inf.

All arithmetic is float64: block sums (exact for bf16 inputs), scores and the
whole attention.  Pins that tie this code to the mathematics live in
``tests/test_oracle.py``.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Geometry", "geometry", "block_coords", "window", "block_tokens",
    "pool", "block_scores", "select", "attend", "attend_rows", "useful_flops",
]


@dataclass(frozen=True)
class Geometry:
    batch: int
    heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    q_frames: int
    kv_frames: int
    block_h: int
    block_w: int
    nbh: int            # block rows per frame
    nbw: int            # block columns per frame
    nbf: int            # blocks per frame
    nqb: int            # query blocks
    nkb: int            # key blocks
    half: int           # window half-width in blocks (local_range // 2)
    k: int              # kept-block budget before clamping to the window
    scale: float

    @property
    def block_tokens(self) -> int:
        return self.block_h * self.block_w

    @property
    def q_tokens(self) -> int:
        return self.q_frames * self.grid_h * self.grid_w

    @property
    def kv_tokens(self) -> int:
        return self.kv_frames * self.grid_h * self.grid_w


def _snap_round_half_up(x: float) -> int:
    n = round(x)
    if abs(x - n) < 1e-9:
        return int(n)
    return int(math.floor(x + 0.5))


def _snap_ceil(x: float) -> int:
    n = round(x)
    if abs(x - n) < 1e-9:
        return int(n)
    return int(math.ceil(x))


def geometry(desc: dict) -> Geometry:
    """Block layout, KV window length and budget (readings R1, R2, R7)."""
    gh, gw = desc["grid_h"], desc["grid_w"]
    qf, cf = desc["q_frames"], desc["cached_frames"]
    ratio = desc["kv_ratio"]
    kvf = qf + cf if ratio <= 0 else min(qf + cf, _snap_ceil(ratio * qf))
    bh, bw = desc.get("block_h", 0), desc.get("block_w", 0)
    if bh == 0 and bw == 0:
        if gw % 16 == 0 and gh % 8 == 0:
            bh, bw = 8, 16
        elif gh % 16 == 0 and gw % 8 == 0:
            bh, bw = 16, 8
        else:
            raise ValueError("token grid not tileable by 8x16 or 16x8 blocks")
    if gh % bh or gw % bw:
        raise ValueError("block shape does not tile the token grid")
    nbh, nbw = gh // bh, gw // bw
    nbf = nbh * nbw
    if desc.get("topk", 0) > 0:
        k = int(desc["topk"])
    else:
        k = _snap_round_half_up(float(desc["topk_ratio"]) * nbf)
    k = max(k, 1)
    scale = desc.get("scale", 0.0) or 1.0 / math.sqrt(desc["head_dim"])
    return Geometry(batch=desc["batch"], heads=desc["heads"], head_dim=desc["head_dim"],
                    grid_h=gh, grid_w=gw, q_frames=qf, kv_frames=kvf,
                    block_h=bh, block_w=bw, nbh=nbh, nbw=nbw, nbf=nbf,
                    nqb=qf * nbf, nkb=kvf * nbf, half=desc["local_range"] // 2,
                    k=k, scale=float(scale))


def block_coords(g: Geometry, blk: int) -> tuple[int, int, int]:
    """Block index -> (frame, block row, block column); raster over blocks."""
    t, rem = divmod(blk, g.nbf)
    by, bx = divmod(rem, g.nbw)
    return t, by, bx


@functools.lru_cache(maxsize=None)
def _window_at(g: Geometry, by: int, bx: int) -> np.ndarray:
    kb = np.arange(g.nkb)
    rem = kb % g.nbf
    ky, kx = rem // g.nbw, rem % g.nbw
    inside = (np.abs(ky - by) <= g.half) & (np.abs(kx - bx) <= g.half)
    out = kb[inside]
    out.setflags(write=False)
    return out


def window(g: Geometry, qb: int) -> np.ndarray:
    """Key blocks eligible for query block qb, ascending (reading R3): every
    KV frame, block rows and columns within ``half`` of the query block's."""
    _, by, bx = block_coords(g, qb)
    return _window_at(g, by, bx)


def block_tokens(g: Geometry, blk: int) -> np.ndarray:
    """Raster token indices (t, y, x) -> (t*Hg + y)*Wg + x of one block."""
    t, by, bx = block_coords(g, blk)
    ys = by * g.block_h + np.arange(g.block_h)
    xs = bx * g.block_w + np.arange(g.block_w)
    return ((t * g.grid_h + ys[:, None]) * g.grid_w + xs[None, :]).reshape(-1)


def pool(g: Geometry, x: np.ndarray, n_blocks: int) -> np.ndarray:
    """Mean of each block's tokens (reading R4): [B,S,H,D] -> [B,H,NB,D]."""
    B, _, H, D = x.shape
    out = np.zeros((B, H, n_blocks, D), dtype=np.float64)
    for blk in range(n_blocks):
        tok = block_tokens(g, blk)
        out[:, :, blk, :] = x[:, tok, :, :].astype(np.float64).sum(axis=1) / len(tok)
    return out


def block_scores(g: Geometry, q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Pooled score of every (query block, key block) pair inside the window
    and -inf outside it: [B, H, NQB, NKB] float64."""
    qbar = pool(g, q, g.nqb)
    kbar = pool(g, k, g.nkb)
    s = np.full((g.batch, g.heads, g.nqb, g.nkb), -np.inf)
    for qb in range(g.nqb):
        e = window(g, qb)
        # scores[b, h, kb] = sum_d qbar[b,h,qb,d] * kbar[b,h,kb,d]
        s[:, :, qb, e] = np.einsum("bhd,bhkd->bhk", qbar[:, :, qb, :], kbar[:, :, e, :])
    return s


def select(g: Geometry, q: np.ndarray, k: np.ndarray):
    """Top-k key blocks per query block inside the window (readings R2-R5).

    Returns (row_ptr int64 [B*H*NQB+1], col_idx int64 [nnz], scores
    float64 [B,H,NQB,NKB]).  Row r = (b*H + h)*NQB + qb.
    """
    s = block_scores(g, q, k)
    rows = []
    for b in range(g.batch):
        for h in range(g.heads):
            for qb in range(g.nqb):
                e = window(g, qb)
                keep = min(g.k, len(e))
                # sort by descending score, ties by ascending block index
                order = e[np.lexsort((e, -s[b, h, qb, e]))]
                rows.append(np.sort(order[:keep]))
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in rows])
    col_idx = np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)
    return row_ptr, col_idx, s


def _attend_row(g: Geometry, q, k, v, b, h, qb, blocks):
    qtok = block_tokens(g, qb)
    kblocks = [kb for kb in blocks if 0 <= kb < g.nkb]
    if not kblocks:
        return qtok, np.zeros((len(qtok), g.head_dim)), np.full(len(qtok), -np.inf)
    ktok = np.concatenate([block_tokens(g, kb) for kb in kblocks])
    qi = q[b, qtok, h, :].astype(np.float64)
    kj = k[b, ktok, h, :].astype(np.float64)
    vj = v[b, ktok, h, :].astype(np.float64)
    z = (qi @ kj.T) * g.scale                 # R8: scaled dot products
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    den = p.sum(axis=1, keepdims=True)
    o = (p @ vj) / den
    lse = m[:, 0] + np.log(den[:, 0])
    return qtok, o, lse


def attend(g: Geometry, q, k, v, row_ptr, col_idx):
    """Softmax attention of each query block over the tokens of its selected
    key blocks.  q: [B,Sq,H,D], k/v: [B,Skv,H,D] (any float dtype, values are
    taken exactly).  Returns (O float64 [B,Sq,H,D], LSE float64 [B,H,Sq])."""
    o = np.zeros((g.batch, g.q_tokens, g.heads, g.head_dim))
    lse = np.full((g.batch, g.heads, g.q_tokens), -np.inf)
    for b in range(g.batch):
        for h in range(g.heads):
            for qb in range(g.nqb):
                r = (b * g.heads + h) * g.nqb + qb
                blocks = col_idx[row_ptr[r]:row_ptr[r + 1]].tolist()
                qtok, orow, lrow = _attend_row(g, q, k, v, b, h, qb, blocks)
                o[b, qtok, h, :] = orow
                lse[b, h, qtok] = lrow
    return o, lse


def attend_rows(g: Geometry, q, k, v, row_ptr, col_idx, rows):
    """Attention of a sample of CSR rows only.  Returns a list of
    (b, h, query token indices, O rows [BT, D], LSE [BT])."""
    out = []
    for r in rows:
        b, rem = divmod(int(r), g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        blocks = col_idx[row_ptr[r]:row_ptr[r + 1]].tolist()
        qtok, orow, lrow = _attend_row(g, q, k, v, b, h, qb, blocks)
        out.append((b, h, qtok, orow, lrow))
    return out


def useful_flops(g: Geometry, row_ptr) -> float:
    """Multiply-adds x 2 of QK^T and PV on the selected block pairs."""
    nnz = int(row_ptr[-1])
    return 4.0 * g.head_dim * g.block_tokens * g.block_tokens * nnz
