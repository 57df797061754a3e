"""Plain CPU oracle of steady threshold reuse for LCSA block selection, in
float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module; only the tests, the smoke check and the bench's CPU-baseline leg
do.  It shares no code with the HIP library.

What the pages state: among the last GH200 optimisations is a cache of mask
thresholds (FlashVSR Hopper PR page, "Remove the remaining control-plane
tax"): each DiT block keeps the threshold found on a steady chunk and uses it
again on the next one, a switch that is accepted only on quality
("Recommended GH200 Controls").

The pages do not define the threshold or its use.  Reading taken here (R11,
listed with the others in the design notes):

  R11 A steady chunk's exact selection gives every CSR row a threshold: the
      keep-th largest pooled score among the row's window blocks (keep =
      min(k, |window|)).  Keeping the window blocks scored at or above it is
      the exact top-k whenever no other block ties that score.  A later
      chunk of the same layer keeps, in each row, every window block whose
      pooled score is at or above the row's stored threshold, in ascending
      block order, and skips the top-k.  The number kept varies by row, from
      none to the whole window; an empty row attends to nothing (R9).  The
      result follows the scores of the new chunk, not its top-k: it is an
      approximation, gated on quality rather than on equality with top-k.
"""
from __future__ import annotations

import numpy as np

from .lcsa_oracle import window

__all__ = ["row_thresholds", "select_threshold", "padded_csr"]


def _rows(g):
    for b in range(g.batch):
        for h in range(g.heads):
            for qb in range(g.nqb):
                yield (b * g.heads + h) * g.nqb + qb, b, h, qb


def row_thresholds(g, s: np.ndarray) -> np.ndarray:
    """keep-th largest window score of every row: float64 [rows]
    (s: pooled scores [B, H, NQB, NKB], -inf outside windows)."""
    out = np.empty(g.batch * g.heads * g.nqb)
    for r, b, h, qb in _rows(g):
        e = window(g, qb)
        keep = min(g.k, len(e))
        out[r] = np.sort(s[b, h, qb, e])[::-1][keep - 1]
    return out


def select_threshold(g, s: np.ndarray, tau: np.ndarray) -> list:
    """Per row, the window blocks with score >= tau[row], ascending."""
    out = []
    for r, b, h, qb in _rows(g):
        e = window(g, qb)
        out.append(e[s[b, h, qb, e] >= tau[r]])
    return out


def padded_csr(g, rows: list):
    """The library's layout for variable rows: row r occupies entries
    [r * W, (r + 1) * W) with W the largest window, its blocks first in
    ascending order, then -1 (an index attention skips)."""
    w = max(len(window(g, qb)) for qb in range(g.nqb))
    row_ptr = np.arange(len(rows) + 1, dtype=np.int64) * w
    col_idx = np.full(len(rows) * w, -1, dtype=np.int64)
    for r, blocks in enumerate(rows):
        col_idx[r * w:r * w + len(blocks)] = blocks
    return row_ptr, col_idx
