#!/usr/bin/env python3
"""Throughput of the partition-attention hot path on one MI355X.

A step is one pass of the whole hot path on the selective-reuse workload (long
video DiT, B=1 H=24 D=128, 122880 keys in 32 partitions of 3840, a 3840-token
query shard): at the anchor step, partition attention over all 32 partitions,
their partition weights and the 28-way composition of the far partitions into a
cached state; at the next step, partition attention over the 4 nearest
partitions with the step's new inputs, the 5-way composition with the cached
state and the 5-way weights. ``--config 2|3|4`` benches a single workload
instead (all partitions, the P-way composition and the weights).

Inputs are synthetic (seeded, see sequence_dit_amd/inputs.py) and resident in
HBM before the timed region. Per-kernel times come from HIP events recorded on
the launch stream inside the timed region. One JSON line is printed on stdout.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "partition-attn TFLOP/s (% bf16 MFMA peak) + as_merge GB/s (% HBM peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
# S = K Q^T (half the FLOPs) at the fp8 peak, PV (the other half) at the bf16 peak
PEAK_FP8_TFLOPS = 5000.0
PEAK_MIXED_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partition_attn_traffic.txt")
ATTN_SOURCES = [os.path.join(ROOT, "sequence_dit_amd", "csrc", f)
                for f in ("attn_kernel.h", "partition_attn.hip", "partition_attn_grouped.hip")]
# the anchor composes the far partitions in runs of this many inside the attention launch
FAR_GROUP = 4
# The next step's near partitions, two per grouped launch: the cached state is folded into
# the first group's result and the two group states are composed by a 2-way merge (measured
# faster than one launch per near partition plus a 5-way merge, and than one group of four)
NEAR_GROUP = 2


def reuse_step(runner, anchor_in, step_in, anchor_scales=None, step_scales=None):
    """One selective-reuse step as bench.py times it: the grouped anchor, then the next step's
    near partitions in groups of NEAR_GROUP."""
    runner.anchor_grouped(*anchor_in, FAR_GROUP, anchor_scales)
    return runner.step_grouped(*step_in, NEAR_GROUP, step_scales)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(paths=ATTN_SOURCES):
    """sha256 over the attention kernel's sources (the template and its bf16 launcher)."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed counter summary (``key: value`` lines),
    or None when that summary was taken on a different kernel source."""
    t = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.lstrip().startswith("#"):
                    k, v = line.split(":", 1)
                    t[k.strip()] = v.strip()
    except OSError:
        return None
    if t.get("source_sha256") != source_digest():
        return None
    try:
        return float(t["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------- #
# CPU baseline: the oracle on a bounded sample of the same workload
# --------------------------------------------------------------------------- #

def cpu_baseline(w, target_s, reuse):
    """The oracle on whole heads of the workload (every query row, every partition of the step).

    One head is timed first; then as many further heads as fit in about ``target_s``
    seconds are timed together, and that run is reported. Whole heads keep the
    oracle's fixed per-head cost (upcasting the head's keys and values) in the
    same proportion as in a full run.
    """
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))

    def run(heads):
        nh = len(heads)
        t0 = time.perf_counter()
        o, l = oracle.partition_states(w.q[:, heads], w.k[:, heads], w.v[:, heads], w.ranges, w.scale, workers=cores)
        oracle.contribution(l.reshape(w.P, -1), w.Sq)
        flops = 4 * nh * w.Sq * w.D * sum(e - s for s, e in w.ranges)
        if reuse:
            near_ranges = [w.ranges[i] for i in w.near]
            o1, l1 = oracle.partition_states(w.q1[:, heads], w.k1[:, heads], w.v1[:, heads], near_ranges,
                                             w.scale, workers=cores)
            full_o1 = np.zeros_like(o)
            full_l1 = np.full_like(l, -np.inf)
            full_o1[w.near], full_l1[w.near] = o1, l1
            _, _, _, c_l = oracle.selective_reuse(o, l, full_o1, full_l1, w.near)
            oracle.contribution(np.concatenate([l1, c_l[None]]).reshape(len(w.near) + 1, -1), w.Sq)
            flops += 4 * nh * w.Sq * w.D * sum(e - s for s, e in near_ranges)
        else:
            oracle.merge(o, l)
        return flops, time.perf_counter() - t0

    flops, dt = run([0])
    heads = [0]
    more = min(w.H - 1, int((target_s - dt) / max(dt, 1e-3)))
    if more >= 1:
        heads = list(range(1, 1 + more))
        flops, dt = run(heads)
        # several heads share the cores better than one: rescale once from this run
        if dt < 0.6 * target_s and len(heads) < w.H - 1:
            nh = min(w.H - 1, max(len(heads) + 1, int(len(heads) * target_s / max(dt, 1e-3))))
            heads = list(range(1, 1 + nh))
            flops, dt = run(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(heads)} of {w.H} heads, all {w.Sq} query rows, every partition of the step "
                      f"(fp64 numpy oracle, {dt:.1f} s)"}


# --------------------------------------------------------------------------- #
# GPU bench
# --------------------------------------------------------------------------- #

def _timed_launches(torch, launch, mode, scratch, reps):
    """Launch time (ms) of `launch` in one of three modes. warm: inputs in the caches where
    they fit; `reps` back-to-back launches between one event pair, averaged (events around
    every launch would add their own gaps to a ~50 us kernel), median of 5 such batches.
    cold: a read of a 512 MB scratch buffer before every launch, outside its events, so that
    L2 and the 256 MB MALL hold none of the inputs; median of `reps` launches. cold_wflush:
    the same with a 512 MB write instead, which also leaves up to 256 MB of dirty lines to
    be written back while the launch runs."""
    for _ in range(3):
        launch()
    if mode == "warm":
        # no host synchronisation between batches: an idle GPU would start them at a lower clock
        ev = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                launch()
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) / reps for a, b in ev)
        return ms[len(ms) // 2]
    ev = []
    sink = torch.zeros((), dtype=torch.float32, device=scratch.device)
    for _ in range(reps):
        if mode == "cold":
            sink += scratch.sum()
        else:
            scratch.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2]


def shape_sweep(N, inputs, torch, dev, reps=10):
    """a1 alone on the image DiT and video DiT workloads, warm, cold and cold with a write flush
    (`_timed_launches`). The fraction is max(t_MFMA, t_HBM) / t with the algorithmic FLOP and
    bytes of the launch."""
    res = {}
    scratch = torch.ones(512 << 18, dtype=torch.float32, device=dev)
    for cfg, name in ((2, "image"), (3, "video")):
        w = inputs.make(cfg)
        q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
        out = torch.empty((w.P, w.B, w.H, w.Sq, w.D), dtype=torch.float32, device=dev)
        lse = torch.empty((w.P, w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
        keys = sum(e - s for s, e in w.ranges)
        flops = 4 * w.B * w.H * w.Sq * keys * w.D
        nbytes = 2 * w.B * w.H * (w.Sq * w.D + 2 * keys * w.D) + w.P * w.B * w.H * w.Sq * (4 * w.D + 4)
        t_floor = max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9)) * 1e3

        # arguments checked and marshalled once: Python's per-call checks would outlast the
        # ~50 us image launch and leave the GPU idle between back-to-back launches
        launch, _, _ = N.prepare_partition_attn(q, k, v, w.ranges, w.scale, out=out, lse=lse)

        for mode in ("warm", "cold", "cold_wflush"):
            t = _timed_launches(torch, launch, mode, scratch, reps if mode != "warm" else (40 if cfg == 2 else 10))
            res[f"attn_{name}_{mode}"] = {"ms": round(t, 4), "TFLOP/s": round(flops / t / 1e9, 1),
                                          "frac_mfma": round(flops / t / 1e9 / PEAK_BF16_TFLOPS, 4),
                                          "frac_roofline": round(t_floor / t, 4)}
        del q, k, v, out, lse
    del scratch
    return res


def merge_sweep(N, torch, dev, state_out, state_lse, far, near_plus_cached, reps=10):
    """as_merge alone, warm, cold and cold with a write flush (`_timed_launches`): the 32-way
    composition of all partition states (the long-video workload's P-way merge), the 28-way
    composition of the far ones, and the 5-way merge of a reuse step. Bytes = (k + 1) * rows *
    (4D + 4)."""
    res = {}
    scratch = torch.ones(512 << 18, dtype=torch.float32, device=dev)
    rows = state_lse[0].numel()
    D = state_out.shape[-1]
    out = torch.empty(state_out.shape[1:], dtype=torch.float32, device=dev)
    lse = torch.empty(state_lse.shape[1:], dtype=torch.float32, device=dev)
    cases = (("merge_all_32", list(range(state_out.shape[0])), state_out, state_lse),
             ("merge_cached_28", far, state_out, state_lse),
             ("merge_step_5", list(range(near_plus_cached[0].shape[0])), near_plus_cached[0], near_plus_cached[1]))
    for name, idx, so, sl in cases:
        outs, lses = [so[i] for i in idx], [sl[i] for i in idx]
        by = (len(idx) + 1) * rows * (4 * D + 4)

        launch, _, _ = N.prepare_merge(outs, lses, out=out, lse=lse)

        for mode in ("warm", "cold", "cold_wflush"):
            t = _timed_launches(torch, launch, mode, scratch, reps)
            res[f"{name}_{mode}"] = {"k": len(idx), "ms": round(t, 4), "GB/s": round(by / t / 1e6, 1),
                                     "frac_hbm": round(by / t / 1e6 / PEAK_HBM_GBPS, 4)}
    del scratch, out, lse
    return res


def variant_sweep(runner, torch, q, k, v, q1, k1, v1, steps, ms_step, step_flops, attn_flops):
    """The reuse step in other arrangements of the same work, each timed as a whole step like the
    main one and per call: every launch ungrouped (the anchor writes all 32 partition states, then
    the 28-way composition of the far ones; one launch for the near partitions and a 5-way merge
    at the next step), the grouped anchor with that ungrouped next step, and the grouped anchor
    with all near partitions in one group (the cached state folded in, no merge)."""
    res = {}
    anchor_flops = attn_flops["attn_anchor_grouped"]
    variants = (("ungrouped", lambda: (runner.anchor(q, k, v), runner.step(q1, k1, v1))),
                ("grouped_anchor_only", lambda: (runner.anchor_grouped(q, k, v, FAR_GROUP), runner.step(q1, k1, v1))),
                ("grouped_near_in_one", lambda: (runner.anchor_grouped(q, k, v, FAR_GROUP),
                                                 runner.step_grouped(q1, k1, v1, None))))
    for tag, fn in variants:
        runner.timer = None
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / steps
        res[f"step_{tag}"] = {"ms": round(t, 4), "TFLOP/s": round(step_flops / t / 1e9, 1),
                              "main_step_speedup_over_it": round(t / ms_step, 3)}
        runner.timer = []
        for _ in range(max(1, steps // 2)):
            fn()
        torch.cuda.synchronize()
        times = {}
        for name, a, b in runner.timer:
            times.setdefault(name, []).append(a.elapsed_time(b))
        for name, ts in times.items():
            ms = sum(ts) / len(ts)
            entry = {"ms": round(ms, 4)}
            fl = {"attn_anchor": anchor_flops, "attn_anchor_grouped": anchor_flops,
                  "attn_fresh": attn_flops["attn_fresh_grouped"], "attn_fresh_grouped": attn_flops["attn_fresh_grouped"]}.get(name)
            if fl:
                entry["TFLOP/s"] = round(fl / ms / 1e9, 1)
                entry["frac_mfma"] = round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
            res[f"{tag}:{name}"] = entry
    runner.timer = None
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=22.0)
    ap.add_argument("--main-only", action="store_true",
                    help="time the step only: skip the other kernels, arrangements and shapes reported under "
                         "`kernels` (for short profiler runs)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy (y = x * 1, fp32) reading and writing this many MiB, "
                         "outside the timed region, to calibrate HBM byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this library "
              "models one device's share of sequence-parallel attention and has no multi-GPU path.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    from sequence_dit_amd import _native as N
    from sequence_dit_amd import inputs
    from sequence_dit_amd.reuse import SelectiveReuse

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    N.lib()
    dev = "cuda:0"
    log(f"generating workload {args.config}")
    w = inputs.make(args.config)
    reuse = args.config == 5
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    if reuse:
        q1, k1, v1 = w.q1.to(dev), w.k1.to(dev), w.v1.to(dev)
        near = w.near
    else:
        near = list(range(w.P))  # unused
    runner = SelectiveReuse(w.B, w.H, w.Sq, w.D, w.ranges, near, dev, w.scale)
    all_idx = list(range(w.P))
    merge_out = torch.empty((w.B, w.H, w.Sq, w.D), dtype=torch.float32, device=dev)
    merge_lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)

    def step():
        if reuse:
            reuse_step(runner, (q, k, v), (q1, k1, v1))
        else:
            runner._timed("attn_anchor", N.partition_attn, q, k, v, w.ranges, w.scale,
                          out=runner.state_out, lse=runner.state_lse)
            runner._timed("contrib_anchor", runner._contribution, runner.state_lse, runner.anchor_weights,
                          runner.anchor_scores)
            runner._timed("merge_all", N.merge, [runner.state_out[i] for i in all_idx],
                          [runner.state_lse[i] for i in all_idx], out=merge_out, lse=merge_lse)

    if args.copy_mib:
        x = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the dominant kernel: the anchor's attention launch (grouped for the reuse workload); inside
    # the timed region only its launches are bracketed by events (every event pair on the
    # stream costs the step a few microseconds)
    dom = "attn_anchor_grouped" if reuse else "attn_anchor"
    runner.timer, runner.timer_only = [], {dom}
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_step = start.elapsed_time(end) / args.steps
    log(f"timed region: {ms_step:.3f} ms/step (wall {wall_ms / args.steps:.3f} ms/step)")
    dom_times = [s.elapsed_time(e) for name, s, e in runner.timer]

    # every launch of the step timed on its own, in further steps after the timed region
    runner.timer, runner.timer_only = [], None
    for _ in range(max(2, args.steps // 2)):
        step()
    torch.cuda.synchronize()
    times = {}
    for name, s, e in runner.timer:
        times.setdefault(name, []).append(s.elapsed_time(e))
    runner.timer = None
    rows = w.B * w.H * w.Sq
    state_bytes = rows * (4 * w.D + 4)
    per_key = 4 * w.B * w.H * w.Sq * w.D
    all_keys = sum(e - s for s, e in w.ranges)
    anchor_flops = per_key * all_keys
    attn_flops = {"attn_anchor": anchor_flops}
    attn_bytes = {"attn_anchor": 2 * w.B * w.H * (w.Sq * w.D + 2 * all_keys * w.D) + w.P * state_bytes}
    merges = {}
    contribs = {"contrib_anchor": w.P}
    if reuse:
        # the anchor on grouped launches: composed states of the far groups and of each near
        # partition, plus every partition's LSE
        _, starts = runner.grouped_layout(FAR_GROUP)
        n_groups = len(starts) - 1
        n_far_groups = n_groups - len(near)
        attn_flops.pop("attn_anchor")
        attn_bytes.pop("attn_anchor")
        attn_flops["attn_anchor_grouped"] = anchor_flops
        attn_bytes["attn_anchor_grouped"] = (2 * w.B * w.H * (w.Sq * w.D + 2 * all_keys * w.D) + n_groups * state_bytes
                                             + w.P * rows * 4)
        fresh_keys = sum(w.ranges[i][1] - w.ranges[i][0] for i in near)
        n_near_groups = (len(near) + NEAR_GROUP - 1) // NEAR_GROUP
        attn_flops["attn_fresh_grouped"] = per_key * fresh_keys
        # Q and the near partitions' K/V, the cached state folded in, the group states and
        # every near partition's LSE
        attn_bytes["attn_fresh_grouped"] = (2 * w.B * w.H * (w.Sq * w.D + 2 * fresh_keys * w.D)
                                            + (1 + n_near_groups) * state_bytes + len(near) * rows * 4)
        merges = {"merge_cached_grouped": n_far_groups, "merge_step_grouped": n_near_groups}
        contribs["contrib_step"] = len(near) + 1
    else:
        merges = {"merge_all": w.P}

    step_flops = sum(attn_flops.values())
    attn_ms = sum(dom_times)
    attn_launches = len(dom_times)
    attn_total_flops = attn_flops[dom] * attn_launches
    achieved = attn_total_flops / (attn_ms * 1e-3) / 1e12
    kernels = {}
    for n in attn_flops:
        ms = sum(times[n]) / len(times[n])
        kernels[n] = {"ms": round(ms, 4), "TFLOP/s": round(attn_flops[n] / ms / 1e9, 1),
                      "frac_mfma": round(attn_flops[n] / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                      "GB/s_algorithmic": round(attn_bytes[n] / ms / 1e6, 1)}
    merge_bytes_total, merge_ms_total = 0, 0.0
    for n, kway in merges.items():
        ms = sum(times[n]) / len(times[n])
        by = (kway + 1) * state_bytes
        merge_bytes_total += by * len(times[n])
        merge_ms_total += sum(times[n])
        kernels[n] = {"k": kway, "ms": round(ms, 4), "GB/s": round(by / ms / 1e6, 1),
                      "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBPS, 4)}
    for n, P in contribs.items():
        ms = sum(times[n]) / len(times[n])
        by = 2 * P * rows * 4
        kernels[n] = {"P": P, "ms": round(ms, 4), "GB/s": round(by / ms / 1e6, 1)}
    merge_gbps = merge_bytes_total / (merge_ms_total * 1e-3) / 1e9

    reuse_quality = None
    if reuse and not args.main_only:
        # quality of the reuse step (outside the timed region): the step's result against full
        # attention at t+1 (all 32 partitions, composed), and the time that full attention takes
        runner.timer = None
        runner.anchor(q, k, v)
        r_out, r_lse = runner.step(q1, k1, v1)
        full_out = torch.empty_like(runner.state_out)
        full_lse = torch.empty_like(runner.state_lse)
        f_out = torch.empty_like(merge_out)
        f_lse = torch.empty_like(merge_lse)
        torch.cuda.synchronize()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        N.partition_attn(q1, k1, v1, w.ranges, w.scale, out=full_out, lse=full_lse)
        e1.record()
        N.merge(list(full_out), list(full_lse), out=f_out, lse=f_lse)
        e2.record()
        torch.cuda.synchronize()
        near_mass = runner.anchor_scores[:, near].sum(dim=1).mean().item()
        fresh_ms = kernels["attn_fresh_grouped"]["ms"] + kernels["merge_step_grouped"]["ms"]
        reuse_quality = {
            "mse_vs_full": float(torch.mean((r_out - f_out) ** 2).item()),
            "lse_max_abs_vs_full": float((r_lse - f_lse).abs().max().item()),
            "near_weight_mass": round(near_mass, 4),
            "full_attention_ms": round(e0.elapsed_time(e1) + e1.elapsed_time(e2), 4),
            "reuse_attention_ms": round(fresh_ms, 4),
            "attention_time_ratio": round((e0.elapsed_time(e1) + e1.elapsed_time(e2)) / fresh_ms, 2)}
        del full_out, full_lse, f_out, f_lse

        # planner statistics (timed on their own, outside the step): anchor norms of every
        # partition's OUT, global weights, the local drift and the decision
        eps = torch.tensor([1e-4], dtype=torch.float32, device=dev)
        runner.timer = None
        runner.plan_anchor()
        runner.plan_step(w.local, 4, eps, 0.5)
        torch.cuda.synchronize()
        runner.timer = []
        for _ in range(args.steps):
            runner.plan_anchor()
            runner.plan_step(w.local, 4, eps, 0.5)
        torch.cuda.synchronize()
        ptimes = {}
        for name, s, e in runner.timer:
            ptimes.setdefault(name, []).append(s.elapsed_time(e))
        n_state = rows * w.D
        for name, by in (("plan_norms_anchor", w.P * n_state * 4), ("plan_drift", 2 * n_state * 4),
                         ("plan_weights", w.P * rows * 4), ("plan_decide", None)):
            ms = sum(ptimes[name]) / len(ptimes[name])
            kernels[name] = {"ms": round(ms, 4)}
            if by:
                kernels[name].update({"GB/s": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBPS, 4)})

        # compact (bf16 OUT) states, timed on their own: the anchor writing bf16 states, the
        # 28-way composition of the far ones, and group-wise composition of all 32 (g = 4)
        st16 = torch.empty(runner.state_out.shape, dtype=torch.bfloat16, device=dev)
        c16 = torch.empty(runner.state_out.shape[1:], dtype=torch.bfloat16, device=dev)
        c16_lse = torch.empty(runner.state_lse.shape[1:], dtype=torch.float32, device=dev)
        G = (w.P + 3) // 4
        g16 = torch.empty((G,) + tuple(runner.state_out.shape[1:]), dtype=torch.bfloat16, device=dev)
        g16_lse = torch.empty((G,) + tuple(runner.state_lse.shape[1:]), dtype=torch.float32, device=dev)
        far = runner.far
        # fp8 state payloads (E4M3 codes + one factor per row), the same three calls
        sshape = tuple(runner.state_out.shape[1:])
        st8 = N.Fp8States.empty(w.P, sshape, dev)
        c8 = N.Fp8States.empty(1, sshape, dev)
        g8 = N.Fp8States.empty(G, sshape, dev)

        def compact_calls():
            runner._timed("attn_anchor_bf16_states", N.partition_attn_states, q, k, v, w.ranges, w.scale,
                          torch.bfloat16, out=st16, lse=runner.state_lse)
            runner._timed("merge_cached_bf16", N.merge_states, [st16[i] for i in far],
                          [runner.state_lse[i] for i in far], torch.bfloat16, out=c16, lse=c16_lse)
            runner._timed("compose_groups_g4_bf16", N.compose_groups, st16, runner.state_lse, 4, torch.bfloat16,
                          out=g16, lse=g16_lse)
            runner._timed("attn_anchor_fp8_states", N.partition_attn_states, q, k, v, w.ranges, w.scale,
                          N.FP8, out=st8, lse=runner.state_lse)
            runner._timed("merge_cached_fp8", N.merge_states, [st8[i] for i in far],
                          [runner.state_lse[i] for i in far], N.FP8, out=c8, lse=c16_lse)
            runner._timed("compose_groups_g4_fp8", N.compose_groups, st8, runner.state_lse, 4, N.FP8,
                          out=g8, lse=g16_lse)

        runner.timer = None
        compact_calls()
        torch.cuda.synchronize()
        runner.timer = []
        for _ in range(max(1, args.steps // 2)):
            compact_calls()
        torch.cuda.synchronize()
        ctimes = {}
        for name, s, e in runner.timer:
            ctimes.setdefault(name, []).append(s.elapsed_time(e))
        st16_bytes = rows * (2 * w.D + 4)
        st8_bytes = N.state_bytes(N.FP8, rows, w.D) + rows * 4
        for name in ("attn_anchor_bf16_states", "attn_anchor_fp8_states"):
            ms = sum(ctimes[name]) / len(ctimes[name])
            kernels[name] = {"ms": round(ms, 4), "TFLOP/s": round(anchor_flops / ms / 1e9, 1)}
        for name, by in (("merge_cached_bf16", (len(far) + 1) * st16_bytes),
                         ("compose_groups_g4_bf16", (w.P + G) * st16_bytes),
                         ("merge_cached_fp8", (len(far) + 1) * st8_bytes),
                         ("compose_groups_g4_fp8", (w.P + G) * st8_bytes)):
            ms = sum(ctimes[name]) / len(ctimes[name])
            kernels[name] = {"ms": round(ms, 4), "GB/s": round(by / ms / 1e6, 1),
                             "frac_hbm": round(by / ms / 1e6 / PEAK_HBM_GBPS, 4)}
        kernels["state_bytes_per_row"] = {"fp32": 4 * w.D + 4, "bf16": 2 * w.D + 4, "fp8": w.D + 8,
                                          "kv_bytes_per_key_bf16": 4 * w.D, "kv_bytes_per_key_fp8": 2 * w.D}
        del st16, c16, g16, st8, c8, g8

        # fp8 E4M3 queries and keys (per-(b, h) factors; the quantisation is the caller's input
        # preparation and is not timed): the anchor over all partitions and the fresh partitions
        # of the next step, against the peak of their mix (S on the fp8 MFMA, PV on the bf16 MFMA)
        q8, qs8 = inputs.quantize_fp8(q)
        k8, ks8 = inputs.quantize_fp8(k)
        q18, qs18 = inputs.quantize_fp8(q1)
        k18, ks18 = inputs.quantize_fp8(k1)
        v8, vs8 = inputs.quantize_fp8(v)
        v18, vs18 = inputs.quantize_fp8(v1)
        near_ranges = [w.ranges[i] for i in near]
        f_out = torch.empty((len(near),) + tuple(runner.state_out.shape[1:]), dtype=torch.float32, device=dev)
        f_lse = torch.empty((len(near),) + tuple(runner.state_lse.shape[1:]), dtype=torch.float32, device=dev)

        def fp8_calls():
            # the same single-partition launches on bf16 and fp8 q/k, back to back
            runner._timed("attn_anchor_bf16", N.partition_attn, q, k, v, w.ranges, w.scale,
                          out=runner.state_out, lse=runner.state_lse)
            runner._timed("attn_anchor_fp8", N.partition_attn_fp8, q8, k8, v, qs8, ks8, w.ranges, w.scale,
                          out=runner.state_out, lse=runner.state_lse)
            runner._timed("attn_fresh_bf16", N.partition_attn, q1, k1, v1, near_ranges, w.scale,
                          out=f_out, lse=f_lse)
            runner._timed("attn_fresh_fp8", N.partition_attn_fp8, q18, k18, v1, qs18, ks18, near_ranges, w.scale,
                          out=f_out, lse=f_lse)
            runner._timed("attn_anchor_fp8qkv", N.partition_attn_fp8_qkv, q8, k8, v8, qs8, ks8, vs8, w.ranges,
                          w.scale, out=runner.state_out, lse=runner.state_lse)
            runner._timed("attn_fresh_fp8qkv", N.partition_attn_fp8_qkv, q18, k18, v18, qs18, ks18, vs18,
                          near_ranges, w.scale, out=f_out, lse=f_lse)

        # the whole step (anchor + next step, with their compositions and weights) on fp8 q/k
        runner.timer = None
        reuse_step(runner, (q8, k8, v), (q18, k18, v1), (qs8, ks8), (qs18, ks18))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            reuse_step(runner, (q8, k8, v), (q18, k18, v1), (qs8, ks8), (qs18, ks18))
        e1.record()
        torch.cuda.synchronize()
        fp8_step_ms = e0.elapsed_time(e1) / args.steps
        kernels["step_fp8"] = {"ms": round(fp8_step_ms, 4), "TFLOP/s": round(step_flops / fp8_step_ms / 1e9, 1),
                               "speedup_vs_bf16": round(ms_step / fp8_step_ms, 3)}
        # and on fp8 q/k/v
        reuse_step(runner, (q8, k8, v8), (q18, k18, v18), (qs8, ks8, vs8), (qs18, ks18, vs18))
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            reuse_step(runner, (q8, k8, v8), (q18, k18, v18), (qs8, ks8, vs8), (qs18, ks18, vs18))
        e1.record()
        torch.cuda.synchronize()
        ms8 = e0.elapsed_time(e1) / args.steps
        kernels["step_fp8qkv"] = {"ms": round(ms8, 4), "TFLOP/s": round(step_flops / ms8 / 1e9, 1),
                                  "speedup_vs_bf16": round(ms_step / ms8, 3)}

        runner.timer = None
        fp8_calls()
        torch.cuda.synchronize()
        runner.timer = []
        for _ in range(max(1, args.steps // 2)):
            fp8_calls()
        torch.cuda.synchronize()
        ftimes = {}
        for name, s, e in runner.timer:
            ftimes.setdefault(name, []).append(s.elapsed_time(e))
        for name, base, fl in (("attn_anchor_fp8", "attn_anchor_bf16", anchor_flops),
                               ("attn_fresh_fp8", "attn_fresh_bf16", attn_flops["attn_fresh_grouped"]),
                               ("attn_anchor_fp8qkv", "attn_anchor_bf16", anchor_flops),
                               ("attn_fresh_fp8qkv", "attn_fresh_bf16", attn_flops["attn_fresh_grouped"])):
            ms = sum(ftimes[name]) / len(ftimes[name])
            ms16 = sum(ftimes[base]) / len(ftimes[base])
            tf = fl / ms / 1e9
            kernels[name] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_mixed_peak": round(tf / PEAK_MIXED_TFLOPS, 4),
                             "speedup_vs_bf16": round(ms16 / ms, 3)}
            kernels[base] = {"ms": round(ms16, 4), "TFLOP/s": round(fl / ms16 / 1e9, 1),
                             "frac_mfma": round(fl / ms16 / 1e9 / PEAK_BF16_TFLOPS, 4)}
        del q8, k8, v8, q18, k18, v18, f_out, f_lse

    traffic = measured_traffic()
    roofline = {"kernel": ("attn_bf16_kernel<128, 0, false, true, false> (grouped anchor: 7 groups of 4 far "
                           "partitions, 4 near ones alone)") if reuse else f"attn_bf16_kernel<{w.D}, 0, false, false, false>",
                "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "algorithmic_flops_per_launch": attn_total_flops / attn_launches,
                "avg_launch_ms": round(attn_ms / attn_launches, 4)}

    if reuse and not args.main_only:
        log("other arrangements of the step")
        kernels.update(variant_sweep(runner, torch, q, k, v, q1, k1, v1, args.steps, ms_step, step_flops,
                                     attn_flops))
        log("merges warm and cold (32-way, 28-way, 5-way)")
        runner.timer = None
        runner.anchor(q, k, v)
        runner.step(q1, k1, v1)
        torch.cuda.synchronize()
        kernels.update(merge_sweep(N, torch, dev, runner.state_out, runner.state_lse, runner.far,
                                   (runner.step_out, runner.step_lse)))
        log("image and video DiT shapes, warm and cold")
        kernels.update(shape_sweep(N, inputs, torch, dev))

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, args.cpu_seconds, reuse)
        log(f"cpu baseline {cpu['value']:.4f} TFLOP/s on {cpu['cores']} cores")

    config = {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "Sq": w.Sq, "Skv": w.Skv, "P": w.P}
    if reuse:
        config.update({"fresh_partitions": near, "cached_partitions": w.P - len(near), "denoising_steps": 2})
    line = {
        "metric": METRIC,
        "value": round(step_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
        "merge_GBps": round(merge_gbps, 1),
        "merge_frac_hbm": round(merge_gbps / PEAK_HBM_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "reuse_quality": reuse_quality,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
