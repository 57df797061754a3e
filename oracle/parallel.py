"""The oracle over (batch, head) slices on a pool of worker processes.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests and the
bench's CPU-baseline leg use it; the library never does.

Nothing here computes any step of the method.  Selection and attention are
independent per (batch, head) (every score, top-k and softmax of a row stays
inside its head), so each task takes one (batch, head) slice of the inputs,
builds the one-head geometry and calls the oracle's own functions on it as
they stand (``select``, ``attend``, ``attend_rows``); the results are put
back in the CSR row order r = (b * heads + h) * nqb + qb.

Workers are spawned processes (no state inherited from a parent that may
hold a GPU context) that read the inputs from memory-mapped files, each
with one BLAS thread.
"""
from __future__ import annotations

import os
import shutil
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import get_context

import numpy as np

import lcsa_inputs as li

from . import lcsa_oracle as o

__all__ = ["OraclePool"]

_ARRAYS: dict = {}


def _init_worker(paths: dict):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001  (BLAS threads stay as they are)
        pass
    for name, path in paths.items():
        _ARRAYS[name] = np.load(path, mmap_mode="r")


def _head(name: str, b: int, h: int) -> np.ndarray:
    """[1, tokens, 1, D] float64 slice of a bf16-bits input."""
    return li.bf16_bits_to_f64(np.ascontiguousarray(_ARRAYS[name][b:b + 1, :, h:h + 1, :]))


def _select_task(args):
    desc1, b, h = args
    g1 = o.geometry(desc1)
    t0 = time.perf_counter()
    rp, ci, s = o.select(g1, _head("q", b, h), _head("k", b, h))
    return b, h, rp, ci, s[0, 0], time.perf_counter() - t0


def _attend_task(args):
    desc1, b, h, rp, ci, rows = args
    g1 = o.geometry(desc1)
    q, k, v = _head("q", b, h), _head("k", b, h), _head("v", b, h)
    t0 = time.perf_counter()
    if rows is None:
        out, lse = o.attend(g1, q, k, v, rp, ci)
        res = (out[0, :, 0, :], lse[0, 0])
    else:
        res = [(qtok, orow, lrow) for _, _, qtok, orow, lrow in o.attend_rows(g1, q, k, v, rp, ci, rows)]
    return b, h, res, time.perf_counter() - t0


class OraclePool:
    """Oracle select and attention of one workload, split over (batch,
    head).  q, k, v are the bf16 bit arrays [B, S, H, D] (uint16)."""

    def __init__(self, desc: dict, q, k, v, workers: int | None = None):
        self.desc = dict(desc)
        self.g = o.geometry(self.desc)
        self.desc1 = dict(self.desc, batch=1, heads=1)
        self.heads = [(b, h) for b in range(self.g.batch) for h in range(self.g.heads)]
        cores = len(os.sched_getaffinity(0))
        self.workers = max(1, min(workers or cores, cores, len(self.heads), 15))
        self._dir = tempfile.mkdtemp(prefix="lcsa_oracle_")
        paths = {}
        for name, arr in (("q", q), ("k", k), ("v", v)):
            paths[name] = os.path.join(self._dir, f"{name}.npy")
            np.save(paths[name], np.ascontiguousarray(arr, dtype=np.uint16))
        self._pool = ProcessPoolExecutor(max_workers=self.workers, mp_context=get_context("spawn"),
                                         initializer=_init_worker, initargs=(paths,))

    def close(self):
        self._pool.shutdown(wait=True)
        shutil.rmtree(self._dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def select(self):
        """Oracle top-k CSR of every row (int64), pooled scores [B, H, NQB,
        NKB] and the wall time of the pass."""
        g = self.g
        t0 = time.perf_counter()
        res = list(self._pool.map(_select_task, [(self.desc1, b, h) for b, h in self.heads]))
        wall = time.perf_counter() - t0
        rows = g.batch * g.heads * g.nqb
        counts = np.zeros(rows, dtype=np.int64)
        lists = [None] * (g.batch * g.heads)
        scores = np.empty((g.batch, g.heads, g.nqb, g.nkb))
        for b, h, rp, ci, s, _ in res:
            i = b * g.heads + h
            counts[i * g.nqb:(i + 1) * g.nqb] = np.diff(rp)
            lists[i] = ci
            scores[b, h] = s
        row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        col_idx = np.concatenate(lists).astype(np.int64) if lists else np.zeros(0, np.int64)
        return row_ptr, col_idx, scores, wall

    def _head_csr(self, row_ptr, col_idx, b, h):
        g = self.g
        r0 = (b * g.heads + h) * g.nqb
        seg = np.asarray(row_ptr[r0:r0 + g.nqb + 1], dtype=np.int64)
        return seg - seg[0], np.asarray(col_idx[seg[0]:seg[-1]], dtype=np.int64)

    def attend(self, row_ptr, col_idx):
        """Oracle attention of every row over the given CSR: O float64
        [B, Sq, H, D], LSE [B, H, Sq] and the wall time of the pass."""
        g = self.g
        tasks = [(self.desc1, b, h, *self._head_csr(row_ptr, col_idx, b, h), None)
                 for b, h in self.heads]
        t0 = time.perf_counter()
        res = list(self._pool.map(_attend_task, tasks))
        wall = time.perf_counter() - t0
        out = np.zeros((g.batch, g.q_tokens, g.heads, g.head_dim))
        lse = np.full((g.batch, g.heads, g.q_tokens), -np.inf)
        for b, h, (oh, lh), _ in res:
            out[b, :, h, :] = oh
            lse[b, h] = lh
        return out, lse, wall

    def attend_rows(self, row_ptr, col_idx, rows):
        """Oracle attention of the listed CSR rows only: a list of (b, h,
        query token indices, O rows, LSE) in the order of ``rows``."""
        g = self.g
        by_head: dict = {}
        for r in rows:
            b, rem = divmod(int(r), g.heads * g.nqb)
            h, qb = divmod(rem, g.nqb)
            by_head.setdefault((b, h), []).append(qb)
        tasks = [(self.desc1, b, h, *self._head_csr(row_ptr, col_idx, b, h), qbs)
                 for (b, h), qbs in by_head.items()]
        got = {}
        for b, h, res, _ in self._pool.map(_attend_task, tasks):
            for qb, (qtok, orow, lrow) in zip(by_head[(b, h)], res):
                got[(b * g.heads + h) * g.nqb + qb] = (b, h, qtok, orow, lrow)
        return [got[int(r)] for r in rows]
