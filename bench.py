#!/usr/bin/env python3
"""Benchmark of one data-parallel rank's local ZeRO/FSDP step on one MI355X.

A step is one pass of the whole path over the rank's shard: pack the bf16
gradient slice, its sum of squares, clip + AdamW + bf16 cast, unpack. The
default workload is the 7.5B GPT-style model at N_d = 64 (rank 1, a
119,408,512-element shard, warm-started moments at step 1000).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line: the step throughput (shard parameters per second),
per-kernel times and achieved HBM bandwidth, the roofline of the dominant
kernel (AdamW, measured with HIP events on the stream it runs on) and the
oracle's throughput on the host cores as a baseline.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, AMD's published peak
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt-7.5b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


# --------------------------------------------------------------- oracle leg

def cpu_baseline(wl, seconds):
    """The oracle's step (pack, sum of squares, clip, AdamW, unpack) on chunks
    of 2^22 shard elements spread over the rank's shard, on one host core,
    until about ``seconds`` of oracle time has been spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from fsdp_sharded_mixed_zero_amd import synth
    from oracle import step as O
    from oracle.layout import Layout, Segment, build_layout

    lay = build_layout(wl.sizes, wl.n_d, wl.rank, wl.align)
    chunk = 1 << 22
    n_chunks = max(1, lay.shard // chunk)
    hp = O.AdamWHParams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                        weight_decay=wl.weight_decay, max_norm=wl.max_norm)
    others = sum(max(0, min(lay.shard, lay.psi - r * lay.shard)) for r in range(wl.n_d)
                 if r != wl.rank) * wl.grad_sq_mean()
    done = 0
    spent = 0.0
    k = 0
    with threadpool_limits(limits=1):
        while spent < seconds and k < n_chunks:
            b = (k * 7919 % n_chunks) * chunk
            c = min(chunk, lay.shard - b)
            # the chunk as its own small layout over windows of the tensors
            segs, wins = [], []
            for s in lay.segments:
                lo, hi = max(s.dst_off, b), min(s.dst_off + s.length, b + c)
                if lo < hi:
                    segs.append(Segment(len(wins), 0, lo - b, hi - lo))
                    wins.append(hi - lo)
            sub = Layout(tuple(wins), 1, 0, 1, (), lay.psi, c, c, 0, tuple(segs), c, c)
            grads = [synth.to_bf16_bits(synth.host_grad_f32(n, wl, wl.step, 1000 + i))
                     for i, n in enumerate(wins)]
            params = [np.zeros(n, np.uint16) for n in wins]
            master, m, v = synth.host_shard_state(wl, b, c, c, piece=k)
            t0 = time.perf_counter()
            g = O.pack(sub, grads)
            G = O.global_sqnorm([O.sqnorm(g), others])
            coef = O.clip_coef(G, hp.max_norm, hp.clip_eps)
            _, _, _, bits = O.adamw_step(g, master, m, v, wl.step, hp, coef)
            O.unpack(sub, bits, params)
            spent += time.perf_counter() - t0
            done += c
            k += 1
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": (f"{k} chunks of {chunk} elements of the {wl.name} rank-{wl.rank} shard "
                       f"({done} elements, {spent:.1f} s), numpy float64 oracle, one thread")}


# ------------------------------------------------------------------ GPU leg

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's shard on one GPU; runs on more than one GPU are "
              "not part of this build (the collectives around the step are not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from fsdp_sharded_mixed_zero_amd import synth, zero
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    zero.library()                       # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    rs = RankShard(wl)
    torch.cuda.synchronize()

    t = wl.step
    for _ in range(args.warmup):
        rs.step(t)
        t += 1
    torch.cuda.synchronize()
    timing = {}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rs.step(t, timing=timing)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    S = rs.shard
    algo = rs.bytes_per_step()
    kernels = {}
    for phase, evs in timing.items():
        per_step_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
        launches = len(evs) / args.steps
        gbps = algo[phase] / (per_step_ms * 1e-3) / 1e9
        kernels[phase] = {"us_per_step": round(per_step_ms * 1e3, 2), "launches_per_step": launches,
                          "algorithmic_bytes": algo[phase], "GBps": round(gbps, 1),
                          "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    adamw_launch_ms = sum(e0.elapsed_time(e1) for e0, e1 in timing["adamw"]) / len(timing["adamw"])
    launch_elems = S / (len(timing["adamw"]) / args.steps)
    achieved = 28 * launch_elems / (adamw_launch_ms * 1e-3) / 1e9
    step_bytes = sum(algo.values())

    out = {
        "metric": "fused sharded AdamW params/sec/GPU + achieved HBM GB/s (% of MI355X peak)",
        "value": S / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} rank {rs.rank} of N_d={wl.n_d}: one rank's shard, "
                               f"pack -> sum of squares -> clip+AdamW+bf16 cast -> unpack",
                   "shard_params": S, "n_d": wl.n_d, "rank": rs.rank, "tensors": len(wl.sizes),
                   "segments_in_shard": len(rs.segments), "adamw_step": wl.step,
                   "bucket": rs.bucket},
        "adamw_params_per_s": launch_elems / (adamw_launch_ms * 1e-3),
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    del rs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
