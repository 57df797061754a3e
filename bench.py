"""Benchmark of one LCSA layer call (select + attend) on one MI355X.

A step is one pass of the whole hot path on one chunk: host plan, pooled
block scores + top-k CSR mask (lcsa_select), block-sparse attention
(lcsa_attend).  Default workload: the first chunk at 768x1280 output
(6 latent frames x 48x80 tokens = 23040 tokens, 12 heads x 128, 128-token
blocks, local_range 11, sparse_ratio 2.0 -> 60 kept blocks per query block),
seeded synthetic bf16 inputs resident in HBM before timing starts.

Prints ONE JSON line.  value = useful attention TFLOP/s of the whole step
(useful FLOP = 4 * 128 * 128 * 128 per selected block pair; skipped blocks do
not count), ms_per_step = select+attend ms per chunk, from --steps steps run
back to back with no event between kernels.  roofline = the attend kernel
(MFMA-bound) timed with HIP events on its stream over a second pass of as
many steps, each with events around select and attend.  Before the --warmup
steps, steps run back to back for SPIN_UP_S seconds (spin_up_steps) so that
the GPU's clocks leave the idle of input generation; select_roofline =
the select entry point (pool + select kernels) against HBM bandwidth;
cpu_baseline = the float64 CPU oracle on the same step, its heads spread
over worker processes (1 warm-up and 3 timed runs, medians); parity = the
GPU's CSR, O and LSE of that step against the oracle's, on every row and
element; workloads = select and attend medians of the other named workloads
in the same run, each with the oracle's host timing and a parity record of
its own.  Means, medians and p10/p90 come from the warm steps; cold_cache
repeats --cold-steps steps after a 512 MiB read that evicts L2 and the
memory-side cache before each one (and, under after_write_flush, after a
512 MiB fill instead, whose dirty lines are written back during the step);
graph times --graph-steps replays of select + attend captured once in a HIP
graph.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--no-workloads] [--cold-steps N] [--graph-steps N]
  python bench.py --workload stream_768x1280 --ring   # streaming steady state
  python bench.py --rope                               # rotary embedding fused into select
  python bench.py --workload stream_768x1280 --reuse [--ring]   # steady threshold reuse
  python bench.py --heads 3            # one GPU's share of 12 heads sharded over 4 GPUs
  python bench.py --copy-calibration   # plain copy of known size (counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
SPIN_UP_S = 0.25                 # back-to-back steps before the warm-up steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_traffic.json")
ATTEND_SRC = os.path.join(ROOT, "block_sparse_attention_lcsa_amd", "csrc", "attend.hip")


def _src_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def _traffic(workload):
    """HBM bytes per attend launch from the committed rocprofv3 counter runs,
    if they were taken on the current attend kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("attend_src_sha256") != _src_sha(ATTEND_SRC):
        return None
    return entry.get("bytes_per_launch")


NEAR_TIE_REL, NEAR_TIE_FLOOR = 1e-4, 1e-6     # k-th score gap that counts as a near-tie
MAX_ABS_ERR, MIN_COSINE = 1e-2, 0.9999          # attention parity bar


def _mask_parity(g, window, rp_ref, ci_ref, s_ref, rp_gpu, ci_gpu):
    """Rows whose GPU blocks differ from the oracle's, and how many of them
    are near-ties (k-th and (k+1)-th oracle window scores within 1e-4
    relative, or 1e-6 of the row's largest |score|, with every GPU-kept
    block scored inside that band)."""
    import numpy as np
    mism, ties = [], 0
    if not np.array_equal(np.asarray(rp_gpu, np.int64), rp_ref):
        return list(range(len(rp_ref) - 1)), 0
    for r in range(len(rp_ref) - 1):
        a = ci_gpu[rp_ref[r]:rp_ref[r + 1]]
        b = ci_ref[rp_ref[r]:rp_ref[r + 1]]
        if np.array_equal(a, b):
            continue
        mism.append(r)
        bb, rem = divmod(r, g.heads * g.nqb)
        h, qb = divmod(rem, g.nqb)
        e = window(g, qb)
        srt = np.sort(s_ref[bb, h, qb, e])[::-1]
        kk = len(b)
        if kk >= len(e):
            continue
        sk, sk1 = srt[kk - 1], srt[kk]
        band = max(NEAR_TIE_REL * max(abs(sk), abs(sk1)), NEAR_TIE_FLOOR * np.abs(srt).max())
        if sk - sk1 <= band and s_ref[bb, h, qb, a].min() >= sk1 - band:
            ties += 1
    return mism, ties


def cpu_baseline(name, desc, inp, useful_flops, gpu, runs=3):
    """The oracle as it stands, timed on the host cores on the whole step of
    the workload: select and attention, each head on one of a pool of
    worker processes (one BLAS thread each); 1 warm-up run and `runs` timed
    runs, medians.  The warm-up run's results are also the reference of the
    parity record: the GPU's CSR against the oracle's (mismatches, near-
    ties) and the GPU's O and LSE against the oracle's attention over the
    GPU's own mask, on every element."""
    import numpy as np
    import oracle
    from oracle.parallel import OraclePool
    g = oracle.geometry(desc)
    rp_g, ci_g, o_g, lse_g = gpu
    with OraclePool(desc, inp.q, inp.k, inp.v) as pool:
        rp, ci, s, _ = pool.select()                       # warm-up, and the reference
        o_ref, lse_ref, _ = pool.attend(rp, ci)
        t_sel, t_att = [], []
        for _ in range(runs):
            t_sel.append(pool.select()[3])
            t_att.append(pool.attend(rp, ci)[2])
        mism, ties = _mask_parity(g, oracle.window, rp, ci, s, rp_g, ci_g)
        if mism:  # attention is compared on the GPU's own mask
            for b, h, qtok, orow, lrow in pool.attend_rows(rp_g, ci_g, mism):
                o_ref[b, qtok, h] = orow
                lse_ref[b, h, qtok] = lrow
        workers = pool.workers
    a, bref = o_g.astype(np.float64).ravel(), o_ref.ravel()
    cos = float(a @ bref / (np.linalg.norm(a) * np.linalg.norm(bref)))
    head_cos = []
    for b in range(g.batch):
        for h in range(g.heads):
            x, y = o_g[b, :, h].astype(np.float64).ravel(), o_ref[b, :, h].ravel()
            head_cos.append(float(x @ y / (np.linalg.norm(x) * np.linalg.norm(y))))
    fin = np.isfinite(lse_ref)
    parity = {
        "reference": "float64 oracle: its own top-k CSR; attention over the GPU's CSR",
        "rows": int(len(rp) - 1),
        "mask_rows_differing": len(mism),
        "mask_near_ties": int(ties),
        "mask_mismatches_not_near_tie": len(mism) - int(ties),
        "attend_elements": int(o_g.size),
        "attend_max_abs_err": float(np.abs(o_g.astype(np.float64) - o_ref).max()),
        "attend_cosine": cos,
        "attend_worst_head_cosine": min(head_cos),
        "lse_max_abs_err": float(np.abs(lse_g[fin] - lse_ref[fin]).max()),
        "bar": {"max_abs_err": MAX_ABS_ERR, "cosine": MIN_COSINE},
    }
    parity["pass"] = bool(parity["mask_mismatches_not_near_tie"] == 0
                          and parity["attend_max_abs_err"] <= MAX_ABS_ERR
                          and cos >= MIN_COSINE)
    sel_s, att_s = float(np.median(t_sel)), float(np.median(t_att))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    base = {
        "value": useful_flops / (sel_s + att_s) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "ms_per_step": (sel_s + att_s) * 1e3,
        "select_s_median": sel_s,
        "attend_s_median": att_s,
        "select_s_runs": t_sel,
        "attend_s_runs": t_att,
        "processes": int(workers),
        "blas_threads_per_process": 1,
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "parent_blas_threads": blas,
        "sample": (f"{name}: the whole step, oracle select and attention on all "
                   f"{len(rp) - 1} CSR rows, one (batch, head) per task on {workers} worker "
                   f"processes x 1 BLAS thread; 1 warm-up + {runs} timed runs, medians; "
                   f"float64 numpy"),
    }
    return base, parity


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="first_768x1280")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle's CPU timing and the parity record built from it")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only the chosen workload, not the other named ones")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps timed after a 512 MiB cache flush each (0: none)")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="extra steps replayed from a HIP graph of select + attend (0: none)")
    ap.add_argument("--rope", action="store_true",
                    help="factored 3D rotary embedding fused into select (lcsa_select_rope): "
                         "the step turns Q and K, pools the turned values and attends on them")
    ap.add_argument("--ring", action="store_true",
                    help="K/V in a frame ring with the pooled-K cache: each step pools only "
                         "the chunk's q_frames new frames (streaming steady state)")
    ap.add_argument("--heads", type=int, default=0,
                    help="heads of the timed workload (0: its own, 12 for the named chunks); "
                         "e.g. 3 = one GPU's share when the 12 heads are sharded over 4 GPUs")
    ap.add_argument("--reuse", action="store_true",
                    help="steady threshold reuse (lcsa_select_reuse): each step selects by the "
                         "previous chunk's per-row thresholds (from lcsa_select_steady) instead "
                         "of top-k; streaming workloads only")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the LCSA path runs per (batch, head) with no "
              "cross-GPU exchange, and the library has no multi-GPU code. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    import block_sparse_attention_lcsa_amd as lcsa
    import lcsa_inputs as li

    name = args.workload
    desc = dict(li.CONFIGS[name])
    if args.heads < 0:
        print("bench.py: --heads must be positive", file=sys.stderr)
        sys.exit(2)
    if args.heads:
        desc["heads"] = args.heads
    inp = li.generate(desc, seed=args.seed)
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    plan = lcsa.Plan.from_desc(desc)
    info = plan.info
    flops = float(info["useful_flops"])
    ws = torch.empty(max(int(info["select_workspace_bytes"]), 256), dtype=torch.uint8, device=dev)
    inputs_sha = inp.sha256
    if args.reuse:
        # Two consecutive chunks of one synthetic video: the previous chunk
        # (window frames 0 .. kv_frames-1) gives the thresholds, the current
        # one (shifted by q_frames) is timed.
        if desc["cached_frames"] <= 0 or args.rope:
            print("bench.py: --reuse needs a streaming workload (cached frames) and no --rope",
                  file=sys.stderr)
            sys.exit(2)
        kvf, qf = info["kv_frames"], desc["q_frames"]
        ft = desc["grid_h"] * desc["grid_w"]
        video = li.generate(dict(desc, q_frames=kvf + qf, cached_frames=0, kv_ratio=0.0),
                            seed=args.seed)
        vk, vv = up(video.k), up(video.v)

        def chunk(c):
            w0 = c * qf
            qs = up(video.q[:, (w0 + kvf - qf) * ft:(w0 + kvf) * ft])
            return (qs, vk[:, w0 * ft:(w0 + kvf) * ft].contiguous(),
                    vv[:, w0 * ft:(w0 + kvf) * ft].contiguous())
        q_prev, k_prev, _ = chunk(0)
        _, _, tau = lcsa.select_steady(plan, q_prev, k_prev, workspace=ws)
        q, k, v = chunk(1)
        del vk, vv, q_prev, k_prev, video
        inputs_sha = None
    att_ws = torch.empty(int(info["attend_workspace_bytes"]), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    new_frames = info["kv_frames"]
    if args.rope and args.ring:
        print("bench.py: --rope and --ring together are not timed here", file=sys.stderr)
        sys.exit(2)
    if args.rope:
        tabs = li.rope_tables(desc)
        rtab = lcsa.rope(*(torch.from_numpy(tabs[a]).to(dev) for a in ("t", "h", "w")))
        q_rot, k_rot = torch.empty_like(q), torch.empty_like(k)
    if args.ring:
        # ring of kv_frames slots, window frame t in slot (t + 1) % slots;
        # the cache is filled once, then each step pools the newest q_frames
        kvf, ft = info["kv_frames"], desc["grid_h"] * desc["grid_w"]
        slots = kvf
        frame_slot = [(t + 1) % slots for t in range(kvf)]
        ring = lcsa.kv_ring(slots, frame_slot)
        k_ring, v_ring = torch.empty_like(k), torch.empty_like(v)
        for t in range(kvf):
            sl = frame_slot[t]
            k_ring[:, sl * ft:(sl + 1) * ft] = k[:, t * ft:(t + 1) * ft]
            v_ring[:, sl * ft:(sl + 1) * ft] = v[:, t * ft:(t + 1) * ft]
        kcache = torch.empty(lcsa.kcache_bytes(plan, slots) // 8, dtype=torch.float64, device=dev)
        lcsa.select_ring(plan, q, k_ring, ring, kvf, kcache, workspace=ws)
        new_frames = min(desc["q_frames"], kvf)

    def do_select(p):
        if args.reuse and args.ring:
            return lcsa.select_reuse(p, q, k_ring, tau, ring=ring, new_frames=new_frames,
                                     kcache=kcache, workspace=ws)
        if args.reuse:
            return lcsa.select_reuse(p, q, k, tau, workspace=ws)
        if args.ring:
            return lcsa.select_ring(p, q, k_ring, ring, new_frames, kcache, workspace=ws)
        if args.rope:
            return lcsa.select_rope(p, q, k, rtab, q_rot=q_rot, k_rot=k_rot, workspace=ws)[2:]
        return lcsa.select(p, q, k, workspace=ws)

    def do_attend(p, rp, ci):
        # a reused-threshold CSR has rows of many lengths: longest first
        if args.reuse:
            return lcsa.attend_varlen(p, q, k_ring if args.ring else k, v_ring if args.ring else v,
                                      rp, ci, out=out, workspace=att_ws,
                                      ring=ring if args.ring else None)
        if args.ring:
            return lcsa.attend_ring(p, q, k_ring, v_ring, ring, rp, ci, out=out, workspace=att_ws)
        if args.rope:
            return lcsa.attend(p, q_rot, k_rot, v, rp, ci, out=out, workspace=att_ws)
        return lcsa.attend(p, q, k, v, rp, ci, out=out, workspace=att_ws)

    def step(ev=None):
        p = lcsa.Plan.from_desc(desc)                      # host plan (per shape)
        if ev:
            ev[0].record(stream)
        rp, ci = do_select(p)
        if ev:
            ev[1].record(stream)
        do_attend(p, rp, ci)
        if ev:
            ev[2].record(stream)

    # Spin-up: the GPU has idled through input generation, and the first few
    # tens of back-to-back steps after that run a few per cent slow and
    # unevenly (up to 9 % in A/B passes of 20 steps) before its clocks settle.
    # Steps are run until SPIN_UP_S of wall time has passed, then the W
    # warm-up steps, then the timed ones.
    spin_steps = 0
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < SPIN_UP_S:
        for _ in range(10):
            step()
        spin_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed steps: nothing between the kernels of one step or between
    # steps.  A timing event recorded on the stream costs the GPU an idle
    # gap of about 6-10 us before the next kernel (seen in kernel traces),
    # so the per-kernel events are recorded in a second pass of as many
    # steps, right after this one.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    gpu_ms = t_start.elapsed_time(t_end) / args.steps

    # Per-kernel breakdown: events before select, between select and attend
    # and after attend, on the stream the kernels run on.  The attend window
    # holds the event gap before attend, so it reads slightly high.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    sel_ms = [e[0].elapsed_time(e[1]) for e in evs]
    att_ms = [e[1].elapsed_time(e[2]) for e in evs]
    both_ms = [e[0].elapsed_time(e[2]) for e in evs]

    # Cold caches: before each of these steps a 512 MiB buffer is read (a
    # reduction), which evicts every XCD's L2 and the memory-side cache and
    # leaves them holding clean lines; the flush is outside the timed event
    # pairs.  A second pass flushes by writing the 512 MiB instead (a fill
    # kernel), which leaves the caches full of dirty lines that are written
    # back while the step runs.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        flush.fill_(1)
        sink = torch.empty((), dtype=torch.int64, device=dev)

        def cold_pass(write):
            cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.cold_steps)]
            for i in range(args.cold_steps):
                if write:
                    flush.fill_(i & 0xFF)
                else:
                    torch.sum(flush, dim=0, dtype=torch.int64, out=sink)
                step(cevs[i])
            torch.cuda.synchronize()
            return {
                "select_ms_median": float(np.median([e[0].elapsed_time(e[1]) for e in cevs])),
                "attend_ms_median": float(np.median([e[1].elapsed_time(e[2]) for e in cevs])),
                "select_attend_ms_median": float(np.median([e[0].elapsed_time(e[2]) for e in cevs])),
            }
        cold = {"steps": args.cold_steps, "flush_bytes": 512 << 20, "flush": "read"}
        cold.update(cold_pass(False))
        cold["after_write_flush"] = cold_pass(True)
        del flush, sink
    # The same select + attend captured once in a HIP graph and replayed:
    # the step a serving loop would launch, without per-kernel launch calls.
    graph = None
    if args.graph_steps > 0:
        gplan = lcsa.Plan.from_desc(desc)

        def graph_body():
            rp, ci = do_select(gplan)
            do_attend(gplan, rp, ci)
            return rp, ci

        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            graph_body()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            g_out = graph_body()
        # the first replays of a new graph run slower, and the cold-cache
        # steps before left the GPU idle between flushes: spin up as above
        t_spin = time.perf_counter()
        while time.perf_counter() - t_spin < SPIN_UP_S:
            for _ in range(10):
                g.replay()
            torch.cuda.synchronize()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        gev[0].record(stream)
        for _ in range(args.graph_steps):
            g.replay()
        gev[1].record(stream)
        torch.cuda.synchronize()
        graph = {"steps": args.graph_steps,
                 "select_attend_ms": gev[0].elapsed_time(gev[1]) / args.graph_steps}
        del g, g_out

    # Rotary embedding: the fused select against plain select on the same
    # inputs plus a device copy of Q and K, the least a separate rotary pass
    # (read Q and K, write the turned tensors) would cost.
    def tmed(fn, n=20):
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts]))

    rope_cmp = None
    if args.rope:
        rope_plan = lcsa.Plan.from_desc(desc)
        for _ in range(3):
            lcsa.select(rope_plan, q, k, workspace=ws)
        plain_ms = tmed(lambda: lcsa.select(rope_plan, q, k, workspace=ws))
        fused_ms = tmed(lambda: lcsa.select_rope(rope_plan, q, k, rtab, q_rot=q_rot, k_rot=k_rot,
                                                 workspace=ws))

        def copy_qk():
            q_rot.copy_(q)
            k_rot.copy_(k)
        copy_ms = tmed(copy_qk)
        rope_cmp = {"select_rope_ms_median": fused_ms, "select_ms_median_without_rope": plain_ms,
                    "qk_copy_ms_median": copy_ms,
                    "separate_pass_lower_bound_ms": plain_ms + copy_ms}

    # Threshold reuse against top-k on the same (current) chunk: times of
    # both selections and of attention on both masks, and how far the reused
    # mask and its output are from top-k's.
    reuse_cmp = None
    n_idx = int(info["nnz"])
    if args.reuse:
        rplan = lcsa.Plan.from_desc(desc)
        rows, nkb, pad = int(info["rows"]), int(info["nkb"]), int(info["max_window"])
        rp_r, ci_r = do_select(rplan)
        rp_t, ci_t = lcsa.select(rplan, q, k, workspace=ws)
        o_t, o_r = torch.empty_like(q), torch.empty_like(q)
        lcsa.attend(rplan, q, k, v, rp_t, ci_t, out=o_t, workspace=att_ws)
        lcsa.attend(rplan, q, k, v, rp_r, ci_r, out=o_r, workspace=att_ws)
        torch.cuda.synchronize()
        n_idx = ci_r.numel()
        cr = ci_r.view(rows, pad).long()
        kept = (cr >= 0).sum(dim=1)
        m_r = torch.zeros(rows, nkb + 1, dtype=torch.bool, device=dev)
        m_r.scatter_(1, torch.where(cr >= 0, cr, nkb), True)
        rl = (rp_t[1:] - rp_t[:-1]).long()
        m_t = torch.zeros(rows, nkb, dtype=torch.bool, device=dev)
        m_t[torch.repeat_interleave(torch.arange(rows, device=dev), rl), ci_t.long()] = True
        both = int((m_t & m_r[:, :nkb]).sum())
        kept_pairs = int(kept.sum())
        flops = float(info["useful_flops"]) * kept_pairs / max(int(info["nnz"]), 1)
        of_t, of_r = o_t.float(), o_r.float()
        reuse_cmp = {
            "thresholds": "previous chunk's per-row k-th window score (lcsa_select_steady)",
            "kept_pairs": kept_pairs, "top_k_pairs": int(info["nnz"]),
            "kept_per_row_mean": float(kept.float().mean()),
            "kept_per_row_min": int(kept.min()), "kept_per_row_max": int(kept.max()),
            "rows_keeping_none": int((kept == 0).sum()),
            "recall_of_top_k": both / max(int(info["nnz"]), 1),
            "precision_vs_top_k": both / max(kept_pairs, 1),
            "output_rel_l2_vs_top_k": float((of_r - of_t).norm() / of_t.norm()),
            "output_max_abs_vs_top_k": float((of_r - of_t).abs().max()),
            "select_reuse_ms_median": tmed(lambda: do_select(rplan)),
            "select_top_k_ms_median": tmed(lambda: lcsa.select(rplan, q, k, workspace=ws)),
            "attend_reused_mask_ms_median": tmed(
                lambda: lcsa.attend(rplan, q, k, v, rp_r, ci_r, out=o_r, workspace=att_ws)),
            "attend_varlen_reused_mask_ms_median": tmed(
                lambda: lcsa.attend_varlen(rplan, q, k, v, rp_r, ci_r, out=o_r, workspace=att_ws)),
            "attend_top_k_mask_ms_median": tmed(
                lambda: lcsa.attend(rplan, q, k, v, rp_t, ci_t, out=o_t, workspace=att_ws)),
        }
        del m_r, m_t, o_t, o_r

    att_avg = float(np.mean(att_ms))
    sel_avg = float(np.mean(sel_ms))
    step_ms = max(wall_ms, gpu_ms)
    achieved = flops / (att_avg * 1e-3) / 1e12
    # select: algorithmic HBM bytes = Q and K read once (bf16) + the CSR
    # written (row_ptr and col_idx, int32)
    pooled_kv_tokens = info["kv_tokens"] * new_frames // info["kv_frames"]
    qk_bytes = 2 * desc["batch"] * desc["heads"] * 128 * (info["q_tokens"] + pooled_kv_tokens)
    # with the rotary embedding the turned Q and K are written as well
    sel_bytes = qk_bytes * (2 if args.rope else 1) + 4 * (info["rows"] + 1 + n_idx)
    sel_gbs = sel_bytes / (sel_avg * 1e-3) / 1e9

    res = {
        "metric": "LCSA attend useful TFLOP/s + fraction of bf16 MFMA peak; select+attend ms/chunk",
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spin_up_steps": spin_steps,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name,
            "batch": desc["batch"], "heads": desc["heads"], "head_dim": desc["head_dim"],
            "q_tokens": info["q_tokens"], "kv_tokens": info["kv_tokens"],
            "block": [info["block_h"], info["block_w"]], "local_range": desc["local_range"],
            "k": info["k"],
            "selected_pairs": reuse_cmp["kept_pairs"] if args.reuse else info["nnz"],
            "useful_tflop": flops / 1e12,
            "seed": args.seed, "inputs_sha256": inputs_sha,
            "selection": "threshold reuse" if args.reuse else "top-k",
            "kv_storage": "frame ring + pooled-K cache" if args.ring else "contiguous window",
            "rope": "factored 3D, fused into select (22/21/21 pairs)" if args.rope else None,
            "pooled_kv_frames": new_frames,
        },
        "select_ms": sel_avg,
        "attend_ms": att_avg,
        "select_ms_p10_p90": [float(np.percentile(sel_ms, 10)), float(np.percentile(sel_ms, 90))],
        "attend_ms_p10_p90": [float(np.percentile(att_ms, 10)), float(np.percentile(att_ms, 90))],
        "select_ms_median": float(np.median(sel_ms)),
        "attend_ms_median": float(np.median(att_ms)),
        "select_attend_ms_median": float(np.median(both_ms)),
        "select_attend_ms_p10_p90": [float(np.percentile(both_ms, 10)), float(np.percentile(both_ms, 90))],
        "cold_cache": cold,
        "graph": graph,
        "rope_fusion": rope_cmp,
        "threshold_reuse": reuse_cmp,
        "attend_tflops": achieved,
        "attend_frac_of_bf16_peak": achieved / PEAK_BF16_TFLOPS,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": _traffic(name) if desc["heads"] == li.CONFIGS[name]["heads"] else None,
        },
        "select_roofline": {
            "bound": "hbm",
            "achieved": sel_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": sel_gbs / PEAK_HBM_GBS,
            "bytes": sel_bytes,
        },
        "device": torch.cuda.get_device_name(0),
    }
    plain = not (args.reuse or args.rope or args.ring)
    if not args.no_cpu_baseline and plain:
        # the GPU's CSR, O and LSE of one more step, for the parity record
        pplan = lcsa.Plan.from_desc(desc)
        rp_g, ci_g = lcsa.select(pplan, q, k, workspace=ws)
        o_g, lse_g = lcsa.attend(pplan, q, k, v, rp_g, ci_g, return_lse=True, workspace=att_ws)
        torch.cuda.synchronize()
        gpu = (rp_g.cpu().numpy().astype(np.int64), ci_g.cpu().numpy().astype(np.int64),
               o_g.float().cpu().numpy(), lse_g.cpu().numpy())
        res["cpu_baseline"], res["parity"] = cpu_baseline(name, desc, inp, flops, gpu)
    if not args.no_workloads and plain:
        del q, k, v, out, att_ws, ws
        torch.cuda.empty_cache()
        res["workloads"] = time_workloads([n for n in li.PAGE_WORKLOADS if n != name],
                                          args.seed, dev, stream, cpu=not args.no_cpu_baseline)
    print(json.dumps(res), flush=True)


def time_workloads(names, seed, dev, stream, cpu=True):
    """Step time and select / attend medians of the other named workloads,
    timed with HIP events on the launch stream in this same run: a spin-up
    of SPIN_UP_S seconds and 10 warm-up steps, then 50 steps back to back (20
    at the 184320-token chunk) for the step time, then as many with events
    around select and attend (medians, p10 and p90).  With `cpu`, each
    workload also gets the oracle timed on the host cores (as cpu_baseline:
    1 warm-up and 3 timed runs, 1 at the 184320-token chunk) and a parity
    record of one more GPU step against it on every row and element."""
    import numpy as np
    import torch
    import block_sparse_attention_lcsa_amd as lcsa
    import lcsa_inputs as li

    out = {}
    for name in names:
        desc = dict(li.CONFIGS[name])
        inp = li.generate(desc, seed=seed)

        def up(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = up(inp.q), up(inp.k), up(inp.v)
        plan = lcsa.Plan.from_desc(desc)
        info = plan.info
        ws = torch.empty(max(int(info["select_workspace_bytes"]), 256), dtype=torch.uint8, device=dev)
        att_ws = torch.empty(int(info["attend_workspace_bytes"]), dtype=torch.uint8, device=dev)
        o = torch.empty_like(q)
        n = 20 if info["q_tokens"] > 100000 else 50

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            rp, ci = lcsa.select(plan, q, k, workspace=ws)
            if ev:
                ev[1].record(stream)
            lcsa.attend(plan, q, k, v, rp, ci, out=o, workspace=att_ws)
            if ev:
                ev[2].record(stream)
        # spin-up after the idle of input generation, as for the main workload
        t_spin = time.perf_counter()
        while time.perf_counter() - t_spin < SPIN_UP_S:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
        for _ in range(10):
            step()
        # n steps back to back (the step time), then n with per-kernel events
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(n):
            step()
        t1.record(stream)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        step_ms = t0.elapsed_time(t1) / n
        sel_t = [e[0].elapsed_time(e[1]) for e in evs]
        att_t = [e[1].elapsed_time(e[2]) for e in evs]
        both_t = [e[0].elapsed_time(e[2]) for e in evs]
        sel, att, both = (float(np.median(x)) for x in (sel_t, att_t, both_t))

        def p10_p90(x):
            return [float(np.percentile(x, 10)), float(np.percentile(x, 90))]
        flops = float(info["useful_flops"])
        sel_bytes = (2 * desc["batch"] * desc["heads"] * 128 * (info["q_tokens"] + info["kv_tokens"])
                     + 4 * (info["rows"] + 1 + info["nnz"]))
        out[name] = {
            "steps": n, "q_tokens": info["q_tokens"], "kv_tokens": info["kv_tokens"],
            "block": [info["block_h"], info["block_w"]], "k": info["k"],
            "selected_pairs": info["nnz"], "useful_tflop": flops / 1e12,
            "inputs_sha256": inp.sha256,
            "select_ms_median": sel, "attend_ms_median": att, "select_attend_ms_median": both,
            "select_ms_p10_p90": p10_p90(sel_t), "attend_ms_p10_p90": p10_p90(att_t),
            "select_attend_ms_p10_p90": p10_p90(both_t),
            "attend_tflops": flops / (att * 1e-3) / 1e12,
            "attend_frac_of_bf16_peak": flops / (att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "select_gbs": sel_bytes / (sel * 1e-3) / 1e9,
            "select_frac_of_hbm": sel_bytes / (sel * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "step_ms": step_ms,
            "step_tflops": flops / (step_ms * 1e-3) / 1e12,
        }
        print(f"bench: {name} select {sel:.4f} ms, attend {att:.4f} ms", file=sys.stderr, flush=True)
        if cpu:
            # the oracle on the host cores, and the parity of one more GPU step
            rp_g, ci_g = lcsa.select(plan, q, k, workspace=ws)
            o_g, lse_g = lcsa.attend(plan, q, k, v, rp_g, ci_g, return_lse=True, workspace=att_ws)
            torch.cuda.synchronize()
            gpu = (rp_g.cpu().numpy().astype(np.int64), ci_g.cpu().numpy().astype(np.int64),
                   o_g.float().cpu().numpy(), lse_g.cpu().numpy())
            del rp_g, ci_g, o_g, lse_g
            base, par = cpu_baseline(name, desc, inp, flops, gpu,
                                     runs=1 if info["q_tokens"] > 100000 else 3)
            del gpu
            out[name]["cpu_oracle"] = {key: base[key] for key in (
                "value", "unit", "ms_per_step", "select_s_median", "attend_s_median",
                "processes", "sample")}
            out[name]["parity"] = {key: par[key] for key in (
                "rows", "mask_rows_differing", "mask_near_ties", "mask_mismatches_not_near_tie",
                "attend_elements", "attend_max_abs_err", "attend_cosine",
                "attend_worst_head_cosine", "lse_max_abs_err", "pass")}
            print(f"bench: {name} oracle {base['ms_per_step'] / 1e3:.2f} s per step, parity "
                  f"{'pass' if par['pass'] else 'FAIL'}", file=sys.stderr, flush=True)
        del q, k, v, o, ws, att_ws, inp
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
