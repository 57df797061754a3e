"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
oracle's results for the same inputs (cached per process), and the mask
parity rule with near-tie accounting."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import lcsa_inputs as li
import oracle

# Selected-mask parity: a row may differ from the oracle only where the
# oracle's k-th and (k+1)-th window scores are a near-tie.
NEAR_TIE_REL = 1e-4
NEAR_TIE_FLOOR = 1e-6
# Attention output parity against the float64 oracle.
MAX_ABS_ERR = 1e-2
MIN_COSINE = 0.9999


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


@functools.lru_cache(maxsize=2)
def host_inputs(name: str, seed: int = 0, batch: int | None = None, heads: int | None = None):
    desc = dict(li.CONFIGS[name])
    if batch is not None:
        desc["batch"] = batch
    if heads is not None:
        desc["heads"] = heads
    inp = li.generate(desc, seed=seed)
    return desc, inp


@functools.lru_cache(maxsize=2)
def oracle_select(name: str, seed: int = 0, batch: int | None = None, heads: int | None = None):
    desc, inp = host_inputs(name, seed, batch, heads)
    g = oracle.geometry(desc)
    q = li.bf16_bits_to_f64(inp.q)
    k = li.bf16_bits_to_f64(inp.k)
    rp, ci, s = oracle.select(g, q, k)
    return g, rp, ci, s


def device_qkv(name: str, seed: int = 0, batch: int | None = None, heads: int | None = None):
    desc, inp = host_inputs(name, seed, batch, heads)
    return desc, to_device_bf16(inp.q), to_device_bf16(inp.k), to_device_bf16(inp.v)


def check_mask(g, rp_ref, ci_ref, s_ref, rp_gpu, ci_gpu):
    """Compare a GPU CSR with the oracle's.  Returns (mismatched rows,
    near-tie rows among them).  Asserts CSR well-formedness, identical
    row_ptr, and that every mismatch is an acceptable near-tie."""
    rp_gpu = np.asarray(rp_gpu, dtype=np.int64)
    ci_gpu = np.asarray(ci_gpu, dtype=np.int64)
    assert np.array_equal(rp_gpu, rp_ref), "row_ptr differs from the plan/oracle"
    mism, ties = [], []
    for r in range(len(rp_ref) - 1):
        a = ci_gpu[rp_ref[r]:rp_ref[r + 1]]
        b = ci_ref[rp_ref[r]:rp_ref[r + 1]]
        if np.array_equal(a, b):
            continue
        mism.append(r)
        bb, rem = divmod(r, g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        e = oracle.window(g, qb)
        assert np.all(np.diff(a) > 0) and set(a.tolist()) <= set(e.tolist()), f"row {r} malformed"
        srt = np.sort(s_ref[bb, h, qb, e])[::-1]
        kk = len(b)
        sk, sk1 = srt[kk - 1], srt[kk]
        band = max(NEAR_TIE_REL * max(abs(sk), abs(sk1)), NEAR_TIE_FLOOR * np.abs(srt).max())
        assert sk - sk1 <= band, f"row {r}: mask differs and is not a near-tie (gap {sk - sk1:.3e})"
        assert s_ref[bb, h, qb, a].min() >= sk1 - band, f"row {r}: GPU kept a block below the band"
        ties.append(r)
    return mism, ties


def compare_output(o_gpu: np.ndarray, o_ref: np.ndarray, label: str):
    o_gpu = o_gpu.astype(np.float64).ravel()
    o_ref = o_ref.astype(np.float64).ravel()
    err = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    na, nb = np.linalg.norm(o_gpu), np.linalg.norm(o_ref)
    cos = 1.0 if na == 0 and nb == 0 else float(o_gpu @ o_ref / (na * nb + 1e-300))
    say(f"  {label}: max|err| {err:.3e}  cosine {cos:.7f}")
    assert err <= MAX_ABS_ERR, f"{label}: max |err| {err} > {MAX_ABS_ERR}"
    assert cos >= MIN_COSINE, f"{label}: cosine {cos} < {MIN_COSINE}"
    return err, cos


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()
