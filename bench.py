"""Benchmark of one LCSA layer call (select + attend) on one MI355X.

A step is one pass of the whole hot path on one chunk: host plan, pooled
block scores + top-k CSR mask (lcsa_select), block-sparse attention
(lcsa_attend).  Default workload: the first chunk at 768x1280 output
(6 latent frames x 48x80 tokens = 23040 tokens, 12 heads x 128, 128-token
blocks, local_range 11, sparse_ratio 2.0 -> 60 kept blocks per query block),
seeded synthetic bf16 inputs resident in HBM before timing starts.

Prints ONE JSON line.  value = useful attention TFLOP/s of the whole step
(useful FLOP = 4 * 128 * 128 * 128 per selected block pair; skipped blocks do
not count), ms_per_step = select+attend ms per chunk.  roofline = the attend
kernel (MFMA-bound) timed with HIP events on its stream; select_roofline =
the select entry point (pool + select kernels) against HBM bandwidth;
cpu_baseline = the float64 CPU oracle on a bounded sample of the same
workload.  Means, medians and p10/p90 come from the warm steps; cold_cache
repeats --cold-steps steps after a 512 MiB fill that evicts L2 and the
memory-side cache before each one; graph times --graph-steps replays of
select + attend captured once in a HIP graph.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                  [--cold-steps N] [--graph-steps N]
  python bench.py --workload stream_768x1280 --ring   # streaming steady state
  python bench.py --rope                               # rotary embedding fused into select
  python bench.py --workload stream_768x1280 --reuse [--ring]   # steady threshold reuse
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


def cpu_baseline(name, desc, inp, useful_flops, rope_tables=None):
    """Time the oracle as it stands on a bounded sample and scale to a step
    (with rope_tables, the oracle's rotary embedding of Q and K first)."""
    import numpy as np
    import lcsa_inputs as li
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    g = oracle.geometry(desc)
    qf, kf, vf = (li.bf16_bits_to_f32(x) for x in (inp.q, inp.k, inp.v))
    t0 = time.perf_counter()
    if rope_tables is not None:
        tab = oracle.RopeTables(t=rope_tables["t"], h=rope_tables["h"], w=rope_tables["w"])
        qf, kf = oracle.rope_q(g, qf, tab), oracle.rope_k(g, kf, tab)
    rp, ci, _ = oracle.select(g, qf, kf)
    t_sel = time.perf_counter() - t0
    rows = len(rp) - 1
    # rows sampled evenly; grow the sample until ~10 s of attention work
    n = max(8, rows // 64)
    t_att, done = 0.0, 0
    while True:
        sample = np.linspace(0, rows - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.attend_rows(g, qf, kf, vf, rp, ci, sample)
        t_att = time.perf_counter() - t0
        done = n
        if t_att >= 8.0 or n >= rows:
            break
        n = min(rows, int(n * max(2.0, 10.0 / max(t_att, 1e-3))))
    step_s = t_sel + t_att * rows / done
    return {
        "value": useful_flops / step_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "ms_per_step": step_s * 1e3,
        "sample": (f"{name}: oracle {'rotary embedding + ' if rope_tables is not None else ''}"
                   f"select on all {rows} CSR rows ({t_sel:.2f} s) + oracle "
                   f"attention on {done} of {rows} rows ({t_att:.2f} s), scaled to the full "
                   f"step; float64 numpy, {blas_threads} BLAS threads, "
                   f"{len(os.sched_getaffinity(0))} host cores visible"),
    }


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
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    def step(ev=None):
        p = lcsa.Plan.from_desc(desc)                      # host plan (per shape)
        if ev:
            ev[0].record(stream)
        rp, ci = do_select(p)
        if ev:
            ev[1].record(stream)
        if args.ring:
            lcsa.attend_ring(p, q, k_ring, v_ring, ring, rp, ci, out=out, workspace=att_ws)
        elif args.rope:
            lcsa.attend(p, q_rot, k_rot, v, rp, ci, out=out, workspace=att_ws)
        else:
            lcsa.attend(p, q, k, v, rp, ci, out=out, workspace=att_ws)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps

    sel_ms = [e[0].elapsed_time(e[1]) for e in evs]
    att_ms = [e[1].elapsed_time(e[2]) for e in evs]
    both_ms = [e[0].elapsed_time(e[2]) for e in evs]
    gpu_ms = t_start.elapsed_time(t_end) / args.steps

    # Cold caches: before each of these steps a fill kernel writes 512 MiB,
    # which evicts every XCD's L2 and the memory-side cache; the flush is
    # outside the timed event pairs.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(i & 0xFF)
            step(cevs[i])
        torch.cuda.synchronize()
        del flush
        cold = {
            "steps": args.cold_steps,
            "flush_bytes": 512 << 20,
            "select_ms_median": float(np.median([e[0].elapsed_time(e[1]) for e in cevs])),
            "attend_ms_median": float(np.median([e[1].elapsed_time(e[2]) for e in cevs])),
            "select_attend_ms_median": float(np.median([e[0].elapsed_time(e[2]) for e in cevs])),
        }
    # The same select + attend captured once in a HIP graph and replayed:
    # the step a serving loop would launch, without per-kernel launch calls.
    graph = None
    if args.graph_steps > 0:
        gplan = lcsa.Plan.from_desc(desc)

        def graph_body():
            rp, ci = do_select(gplan)
            if args.ring:
                lcsa.attend_ring(gplan, q, k_ring, v_ring, ring, rp, ci, out=out, workspace=att_ws)
            elif args.rope:
                lcsa.attend(gplan, q_rot, k_rot, v, rp, ci, out=out, workspace=att_ws)
            else:
                lcsa.attend(gplan, q, k, v, rp, ci, out=out, workspace=att_ws)
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
        for _ in range(10):      # the first replays of a new graph run slower
            g.replay()
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
            "traffic": _traffic(name),
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
    if not args.no_cpu_baseline and not args.reuse:
        res["cpu_baseline"] = cpu_baseline(name, desc, inp, flops, tabs if args.rope else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
