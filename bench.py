"""Benchmark: zigzag varlen ring attention, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

One step is one pass of the attention core over one batch of synthetic input
already resident in HBM in the zigzag layout: every forward ring step (all
simulated CP ranks of a step in one launch; step 0 writes the partial, later
steps merge in the kernel epilogue); finalize (bf16 O); the backward
pre-pass; every backward ring step (dK/dV kernel and dQ kernel); finalize of
dQ, dK, dV.  The zigzag permute of Q, K, V, dO and the un-permute of O are
timed separately and reported in GB/s ("permute").

Headline value: useful attention TFLOP/s of the whole step, with useful
forward FLOPs 4*d*Hq*P (P = visible query/key pairs, masked work excluded)
and useful backward FLOPs 2.5x that (five matrix products per pair).

Also printed, on the same JSON line:
 * roofline of the dominant kernel: algorithmic FLOPs per launch over its
   mean duration (HIP events around every launch in the timed steps), against
   the bf16 dense MFMA peak of MI355X (2.5 PFLOP/s);
 * per-rank balance: useful pairs per simulated rank from the plan, and the
   measured time of each rank's forward (and backward) run in isolation,
   median of four passes (max/mean);
 * cpu_baseline: the CPU oracle (fp64, OpenMP) timed on a bounded sample of
   the same workload's rows, in useful TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timers:
    """Event pairs around kernel launches on the current (torch) stream."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn):
        import torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def summary(self):
        out = {}
        for k, v in self.pairs.items():
            ms = [a.elapsed_time(b) for a, b in v]
            out[k] = {"launches": len(ms), "mean_ms": sum(ms) / len(ms), "total_ms": sum(ms)}
        return out


def cpu_baseline(w, q, k, v, budget_s: float):
    """Time the oracle on sampled query rows of head 0 (one sequence or
    packed): exact rows, scaled to useful TFLOP/s."""
    import numpy as np
    import torch

    import oracle
    import synthetic
    cu = synthetic.cu_seqlens_for(w)
    g = 0
    qh = q[:, 0:1, :].float().cpu().contiguous()
    kh = k[:, g:g + 1, :].float().cpu().contiguous()
    vh = v[:, g:g + 1, :].float().cpu().contiguous()
    rng = np.random.default_rng(12345)
    seg = np.searchsorted(cu, np.arange(w.total), side="right") - 1
    pos_in_seq = np.arange(w.total) - cu[seg]

    def run(n):
        rows = np.sort(rng.choice(w.total, size=n, replace=False))
        heads = np.zeros(n, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.attn_fwd_rows(qh, kh, vh, cu, w.scale, rows, heads)
        dt = time.perf_counter() - t0
        flops = float(4 * w.d * (pos_in_seq[rows] + 1).sum())
        return n, dt, flops

    n0, dt0, f0 = run(16)
    rate = f0 / max(dt0, 1e-6)
    mean_row = f0 / n0
    n = int(max(16, min(w.total, budget_s * rate / mean_row)))
    n, dt, flops = run(n)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "forward of %d uniformly sampled query rows of head 0 (all their visible keys), "
                  "%.1f GFLOP in %.1f s; full-workload forward extrapolates to %.0f s"
                  % (n, flops / 1e9, dt, 4.0 * w.d * w.hq * pairs_of(cu) / (flops / dt)),
    }


def pairs_of(cu):
    tot = 0
    for i in range(len(cu) - 1):
        L = int(cu[i + 1] - cu[i])
        tot += L * (L + 1) // 2
    return tot


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c5", help="c1..c5 (c5: 131072-token causal, fwd+bwd)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-balance", action="store_true")
    ap.add_argument("--with-backward", action="store_true",
                    help="also time the backward on a forward-only workload (synthetic dO)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured in a HIP graph (one eager step gives the kernel "
                         "times); replays are checked bit for bit against the eager step first")
    ap.add_argument("--gathered", action="store_true",
                    help="the all-gather form: forward and backward as one launch (per kernel) against "
                         "all shards, no step partials, merges or accumulation")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: every simulated CP rank executes on the same device, "
              "so --gpus must be 1 (got %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic
    import zigzag_ring_attention_amd as zz

    w = synthetic.WORKLOADS[args.workload]
    backward = w.backward or args.with_backward
    cu = synthetic.cu_seqlens_for(w)
    T, hq, hkv, d, cp = w.total, w.hq, w.hkv, w.d, w.cp
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log("bench: workload %s T=%d hq=%d hkv=%d d=%d cp=%d dtype=%s backward=%s" %
        (w.name, T, hq, hkv, d, cp, w.dtype, backward))
    plan = zz.Plan(cu, cp, hq, hkv, d, w.dtype, device=dev)
    useful_pairs, issued_pairs = plan.pair_counts()
    fwd_flops = 4.0 * d * hq * useful_pairs
    bwd_flops = 2.5 * fwd_flops if backward else 0.0

    q, k, v, *rest = synthetic.randn_qkv_device(w.seed, T, hq, hkv, d, w.dtype, dev, with_do=backward)
    do = rest[0] if backward else None
    tdt = plan.torch_dtype
    f32 = torch.float32
    q_zz, k_zz, v_zz = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    do_zz = torch.empty_like(do) if backward else None
    o_acc = torch.empty((T, hq, d), dtype=f32, device=dev)
    lse = torch.empty((hq, T), dtype=f32, device=dev)
    o_zz = torch.empty((T, hq, d), dtype=tdt, device=dev)
    o = torch.empty_like(o_zz)
    if backward:
        delta = torch.empty((hq, T), dtype=f32, device=dev)
        dq_acc = torch.empty((T, hq, d), dtype=f32, device=dev)
        dk_acc = torch.empty((T, hkv, d), dtype=f32, device=dev)
        dv_acc = torch.empty((T, hkv, d), dtype=f32, device=dev)
        grads = (torch.empty((T, hq, d), dtype=tdt, device=dev), torch.empty((T, hkv, d), dtype=tdt, device=dev),
                 torch.empty((T, hkv, d), dtype=tdt, device=dev))

    def step(tm: Timers | None):
        def launch(name, fn):
            if tm is None:
                fn()
            else:
                tm.run(name, fn)
        if args.gathered:
            launch("fwd_gathered", lambda: zz.varlen_gathered_fwd(plan, zz.ALL_RANKS, q_zz, k_zz, v_zz, o_acc, lse))
        else:
            for s in range(cp):
                launch("fwd_step", lambda s=s: zz.varlen_ring_step_fwd(plan, zz.ALL_RANKS, s, q_zz, k_zz, v_zz,
                                                                       o_acc, lse, merge=s > 0))
        zz.finalize_fwd(plan, o_acc, unpermute=False, out=o_zz)
        if not backward:
            return
        zz.bwd_preprocess(plan, o_zz, do_zz, delta)
        if args.gathered:
            launch("bwd_gathered", lambda: zz.varlen_gathered_bwd(plan, zz.ALL_RANKS, q_zz, k_zz, v_zz, do_zz, lse,
                                                                  delta, dq_acc, dk_acc, dv_acc))
            zz.finalize_bwd(plan, dq_acc, dk_acc, dv_acc, unpermute=False, out=grads)
            return
        for s in range(cp):
            launch("bwd_dkv", lambda s=s: zz.varlen_ring_step_bwd_dkv(
                plan, zz.ALL_RANKS, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dk_acc, dv_acc, accumulate=s > 0))
            launch("bwd_dq", lambda s=s: zz.varlen_ring_step_bwd_dq(
                plan, zz.ALL_RANKS, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dq_acc, accumulate=s > 0))
        zz.finalize_bwd(plan, dq_acc, dk_acc, dv_acc, unpermute=False, out=grads)

    def permutes():
        zz.zigzag_permute(plan, q, q_zz)
        zz.zigzag_permute(plan, k, k_zz)
        zz.zigzag_permute(plan, v, v_zz)
        if backward:
            zz.zigzag_permute(plan, do, do_zz)

    # inputs to zigzag layout (outside the timed core), then the permute
    # bandwidth on its own: Q, K, V (and dO) in, O back out
    permutes()
    torch.cuda.synchronize()
    pa, pb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pa.record()
    for _ in range(3):
        permutes()
        zz.zigzag_unpermute(plan, o_zz, o)
    pb.record()
    pb.synchronize()
    perm_ms = pa.elapsed_time(pb) / 3
    esz = 2 if w.dtype == "bf16" else 4
    perm_bytes = 2 * esz * d * T * (hq + 2 * hkv + (hq if backward else 0) + hq)   # read + write
    permute = {"ms": round(perm_ms, 4), "gbps": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1),
               "tensors": "Q, K, V%s in, O out" % (", dO" if backward else "")}

    for i in range(args.warmup):
        step(None)
        torch.cuda.synchronize()
        log("bench: warmup step %d done" % i)

    tm = Timers()
    graph = None
    if args.graph:
        # kernel times from one eager step, then the step captured once and
        # replayed; the library's calls launch on torch's current stream, which
        # is the capture stream inside the graph context
        step(tm)
        torch.cuda.synchronize()
        outs = [o_zz] + (list(grads) if backward else [])
        want = [x.clone() for x in outs]
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(None)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step(None)
        for rep in range(2):
            for x in outs:
                x.zero_()
            graph.replay()
            torch.cuda.synchronize()
            for x, y in zip(outs, want):
                if not torch.equal(x, y):
                    raise SystemExit("graph replay %d differs from the eager step" % rep)
        log("bench: graph captured, replays match the eager step")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(tm)
        if i + 1 < args.steps:
            torch.cuda.synchronize()
            log("bench: timed step %d done" % i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    log("bench: %.1f ms/step" % ms_per_step)
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12

    ks = tm.summary()
    per_launch = {
        "fwd_step": 4.0 * d * hq * useful_pairs / cp,
        "fwd_gathered": 4.0 * d * hq * useful_pairs,
        "bwd_gathered": 14.0 * d * hq * useful_pairs,
        "bwd_dkv": 8.0 * d * hq * useful_pairs / cp,
        "bwd_dq": 6.0 * d * hq * useful_pairs / cp,
    }
    dom = max(ks, key=lambda n: ks[n]["total_ms"])
    achieved = per_launch[dom] / (ks[dom]["mean_ms"] * 1e-3) / 1e12
    # HBM bytes per launch of the dominant kernel from the committed counter
    # summary of this workload (None once the kernel sources have changed).
    # Clock and matrix-unit busy fraction of the three kernels under this
    # load, from the committed counter summary (None once sources changed).
    traffic = None
    util = None
    if w.name == "c5":
        from zigzag_ring_attention_amd import profiling
        traffic = profiling.read_traffic(os.path.join(ROOT, "profiles", "c5_hbm_traffic.txt"), dom + "_kernel")
        u = profiling.read_util(os.path.join(ROOT, "profiles", "c5_mfma_utilization.md"))
        if u:
            util = {"source": "profiles/c5_mfma_utilization.md (rocprofv3 --pmc)"}
            for name, (ghz, busy) in u.items():
                util[name] = {"clock_ghz": ghz, "mfma_busy": busy}
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    timed_steps = 1 if args.graph else args.steps   # steps the kernel timers saw
    fwd_ms = ks["fwd_gathered" if args.gathered else "fwd_step"]["total_ms"] / timed_steps
    if not backward:
        bwd_ms = 0.0
    elif args.gathered:
        bwd_ms = ks["bwd_gathered"]["total_ms"] / timed_steps
    else:
        bwd_ms = (ks["bwd_dkv"]["total_ms"] + ks["bwd_dq"]["total_ms"]) / timed_steps

    balance = None
    if not args.no_balance and not args.gathered:
        # Each rank's work runs alone, as it would on a GPU of its own: its
        # forward steps, and (with the backward) its dK/dV and dQ launches of
        # every step.  One untimed pass over all ranks first; then four timed
        # passes in ascending, descending, ascending, descending rank order,
        # and each rank's median, so clock or cache drift over the measurement
        # does not masquerade as imbalance.
        def rank_fwd(r):
            for s in range(cp):
                zz.varlen_ring_step_fwd(plan, r, s, q_zz, k_zz, v_zz, o_acc, lse, merge=s > 0)

        def rank_bwd(r):
            for s in range(cp):
                zz.varlen_ring_step_bwd_dkv(plan, r, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dk_acc, dv_acc,
                                            accumulate=s > 0)
                zz.varlen_ring_step_bwd_dq(plan, r, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dq_acc,
                                           accumulate=s > 0)

        def per_rank(fn):
            for r in range(cp):
                fn(r)
            torch.cuda.synchronize()
            times = [[] for _ in range(cp)]
            for order in (list(range(cp)), list(reversed(range(cp)))) * 2:
                for r in order:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record()
                    fn(r)
                    b.record()
                    b.synchronize()
                    times[r].append(a.elapsed_time(b))
            return [sorted(t)[len(t) // 2 - 1: len(t) // 2 + 1] for t in times]

        def med(pair):
            return 0.5 * (pair[0] + pair[1])

        pairs = [int(x) for x in plan.rank_useful_pairs()]
        fwd_rank = [med(t) for t in per_rank(rank_fwd)]
        balance = {
            "useful_pairs_max_over_mean": max(pairs) / (sum(pairs) / cp),
            "fwd_ms_per_rank_isolated": [round(x, 3) for x in fwd_rank],
            "measured_max_over_mean": max(fwd_rank) / (sum(fwd_rank) / cp),
        }
        if backward:
            bwd_rank = [med(t) for t in per_rank(rank_bwd)]
            balance["bwd_ms_per_rank_isolated"] = [round(x, 3) for x in bwd_rank]
            balance["bwd_measured_max_over_mean"] = max(bwd_rank) / (sum(bwd_rank) / cp)
        log("bench: balance %s" % json.dumps(balance))

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (~%.0f s)" % args.cpu_budget)
        cpu = cpu_baseline(w, q, k, v, args.cpu_budget)

    out = {
        "metric": "useful attention TFLOP/s (%s) and %% of bf16 MFMA peak, 1 MI355X" % ("fwd+bwd" if backward else "fwd"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": "%s: %s, %d tokens, lengths %s, GQA %d/%d, head_dim %d, simulated CP=%d zigzag, %s"
                        % (w.name, w.dtype, T, ("%d sequences" % (len(cu) - 1)) if len(cu) > 2 else "one causal sequence",
                           hq, hkv, d, cp, ("forward + backward" if backward else "forward")
                           + (", all-gather K/V form" if args.gathered else "")
                           + (", step replayed from a HIP graph" if args.graph else "")),
            "tokens": T, "heads_q": hq, "heads_kv": hkv, "head_dim": d, "cp": cp,
            "parallelism": "cp%d simulated on 1 GPU" % cp,
        },
        "pct_of_peak": round(100.0 * value / peak, 2),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2) if backward else None,
        "useful_fwd_tflop": round(fwd_flops / 1e12, 3),
        "tile_efficiency": round(useful_pairs / issued_pairs, 4),
        "kernels_ms": {n: round(v["mean_ms"], 4) for n, v in ks.items()},
        # algorithmic TFLOP/s of every MFMA kernel (executed products, the
        # recomputed ones in dQ included) and its fraction of the peak
        "kernels_tflops": {n: {"tflops": round(per_launch[n] / (v["mean_ms"] * 1e-3) / 1e12, 2),
                               "frac": round(per_launch[n] / (v["mean_ms"] * 1e-3) / 1e12 / peak, 4)}
                           for n, v in ks.items() if n in per_launch},
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "mfma_util": util,
        "permute": permute,
        "balance": balance,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
