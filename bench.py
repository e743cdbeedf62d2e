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
BREAKDOWN_MIN_STEPS = 100     # steps with events around every phase, before the timed region
BREAKDOWN_MIN_SECONDS = 1.0   # ... and at least this much wall time
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
KERNEL_SOURCE = os.path.join(ROOT, "fsdp_sharded_mixed_zero_amd", "csrc", "kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt-7.5b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the plain-copy ceiling (it launches the unpack kernel, so profiled runs "
                         "leave it out to keep that kernel's statistics to the step's own launches)")
    ap.add_argument("--separate-norm", action="store_true",
                    help="run pack and the sum of squares as two calls instead of the fused one")
    ap.add_argument("--accum", type=int, default=1, metavar="K",
                    help="fp32 gradient accumulation over K micro-batches per step (K > 1)")
    ap.add_argument("--separate-unpack", action="store_true",
                    help="run AdamW and the unpack as two calls instead of the fused one")
    ap.add_argument("--state-arrays", action="store_true",
                    help="fp32 master, m and v as three separate arrays (zero_adamw_step_arrays), the unpack "
                         "as its own pass")
    ap.add_argument("--flat", action="store_true",
                    help="ZeRO-1 flat buffers: gradients and parameters are views into flat buffers, the "
                         "shard is the rank's slice (no pack, no unpack)")
    ap.add_argument("--offload", action="store_true",
                    help="ZeRO-Offload: fp32 state in host memory, AdamW on the host cores")
    ap.add_argument("--offload-bucket", type=int, default=1 << 24, metavar="N",
                    help="elements per PCIe staging bucket in the offload step (workloads with their "
                         "own bucket size keep it)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "benchmark into HBM bytes per launch and exit")
    ap.add_argument("--update-sweep", action="store_true",
                    help="time the fused update over the first n elements of the workload's shard for several n "
                         "(20 launches each, events around each) and fit time = fixed + bytes / rate; print "
                         "markdown and exit")
    ap.add_argument("--stats-summary", metavar="STATS_DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run of this benchmark "
                         "(kernel durations, achieved GB/s) as markdown and exit")
    return ap.parse_args()


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


# ---------------------------------------------------------------- HBM traffic

def kernel_name(raw):
    """Short kernel name from a profiler's demangled name, template arguments
    kept (copy_pieces_kernel<true> is pack + sum of squares)."""
    name = raw.replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0].split("::")[-1]


def update_kernel(accum=1, separate_unpack=False, flat=False, state_arrays=False):
    """The update kernel of a mode (the roofline's dominant kernel)."""
    grad = "float" if accum > 1 else "unsigned short"
    if state_arrays:
        return f"adamw_arrays_vec_kernel<{grad}>"
    fused = not separate_unpack and not flat
    return f"adamw_unpack_vec_kernel<{grad}>" if fused else f"adamw_vec_kernel<{grad}>"


def ceiling_elems(launch_bytes):
    """bf16 elements of the copy ceiling's buffers for an update launch of
    ``launch_bytes`` (the copy moves 4 bytes per element)."""
    return max(8, min(int(launch_bytes), 8 << 30) // 4 // 8 * 8)


def algorithmic_bytes(wl, accum=1, separate_norm=False, flat=False, separate_unpack=False, state_arrays=False):
    """Algorithmic HBM bytes per step of each kernel over the whole shard, for
    the benchmark's mode (fused norm and fused unpack by default, separate
    norm, separate unpack, fp32 accumulation over ``accum`` micro-batches,
    flat buffers, or three state arrays with the unpack separate)."""
    from fsdp_sharded_mixed_zero_amd import zero
    info = zero.zero_layout(wl.sizes, wl.n_d, wl.rank, wl.align).info
    S = info["shard"]
    real = S - (info["pad_end"] - info["pad_begin"])
    pack = 4 * real + 2 * (S - real)
    if flat:
        return S, real, {"sqnorm_partial_kernel": 2 * S, "adamw_vec_kernel<unsigned short>": 28 * S}
    separate_unpack = separate_unpack or state_arrays
    update = update_kernel(accum, separate_unpack, state_arrays=state_arrays)
    out = {}
    if separate_unpack:
        out["copy_pieces_kernel<false>"] = 4 * real          # unpack
    if accum > 1:
        out["copy_pieces_kernel<false>"] = out.get("copy_pieces_kernel<false>", 0) + accum * pack   # packs
        out.update({"accumulate_kernel": (6 + 10 * (accum - 1)) * S, "sqnorm_f32_partial_kernel": 4 * S,
                    update: 30 * S})
    else:
        if separate_norm:
            out["copy_pieces_kernel<false>"] = out.get("copy_pieces_kernel<false>", 0) + pack
            out["sqnorm_partial_kernel"] = 2 * S
        else:
            out["copy_pieces_kernel<true>"] = pack
        out[update] = 28 * S
    if not separate_unpack:
        out[update] += 2 * real                                # the tensor writes of the fused unpack
    return S, real, out


def steps_traced(counts, wl, S, combine=False):
    """Steps a trace covers (warm-up included): the sum-of-squares final
    kernel runs once per bucket in the modes without the combine, and once
    per step (the combine) in a bucketed default step, whose buckets' own
    final stages run as one row-sum launch; an update over more than 64 tensor
    pieces takes several launches."""
    pieces = -(-S // wl.bucket) if wl.bucket > 0 else 1
    return counts["sqnorm_final_kernel"] / (1 if combine else pieces)


def setup_sqnorm_launches(wl):
    """Launches of each sum-of-squares kernel the benchmark makes before its
    first step: RankShard.fill_other_ranks runs one zero_shard_sqnorm (a
    partial and a final kernel) per part of a tensor in another rank's shard.
    They come first in a trace, and the summaries leave them out."""
    from fsdp_sharded_mixed_zero_amd import zero
    from fsdp_sharded_mixed_zero_amd.rank import other_rank_slices
    S = zero.zero_layout(wl.sizes, wl.n_d, wl.rank, wl.align).info["shard"]
    return sum(len(parts) for _, parts in other_rank_slices(wl.sizes, S, wl.rank))


SETUP_KERNELS = ("sqnorm_partial_kernel", "sqnorm_final_kernel")


def code_text(text):
    """C++ source with its comments removed and blank space collapsed (string
    and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash():
    """sha256 of the kernels' code (comments and blank space aside): the
    counters of a profile stay valid across comment edits, not code edits."""
    import hashlib
    with open(KERNEL_SOURCE, encoding="utf-8") as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()


def traffic_file(workload):
    return os.path.join(PROFILES, f"hbm_traffic_{workload}.json")


def pmc_summary(fetch_dir, write_dir, wl, steps=20, warmup=2, separate_unpack=False):
    """HBM bytes per launch of each kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain copy of known size: by default the copy ceiling's copy (the
    library's plain copy kernel over the ceiling's buffers, run in the same
    benchmark), with --separate-unpack the unpack (2 bytes read and written
    per real shard element)."""
    import csv
    import glob

    n_setup = setup_sqnorm_launches(wl)

    def load(d, counter):
        """Per kernel, the mean counter value per dispatch (the set-up
        launches left out) and the dispatch count; the copy kernel's mean is
        over its largest-grid dispatches only (the copy ceiling's full-size
        copy)."""
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        per = {}
        for i, row in enumerate(csv.DictReader(open(path))):
            if row["Counter_Name"] != counter:
                continue
            per.setdefault(kernel_name(row["Kernel_Name"]), []).append(
                ((int(row.get("Dispatch_Id") or 0), i), int(row.get("Grid_Size") or 0), float(row["Counter_Value"])))
        mean, count = {}, {}
        for k, rows in per.items():
            rows.sort()                                    # dispatch order
            if k in SETUP_KERNELS:
                rows = rows[n_setup:]
            if k == "copy_pieces_kernel<false>" and not separate_unpack and rows:
                big = max(g for _, g, _ in rows)
                rows = [r for r in rows if r[1] == big]
            if rows:
                mean[k] = sum(v for _, _, v in rows) / len(rows)
                count[k] = len(rows)
        return mean, count

    fetch, n_f = load(fetch_dir, "FETCH_SIZE")
    write, n_w = load(write_dir, "WRITE_SIZE")
    mode = f"--steps {steps} --warmup {warmup}" + (" --separate-unpack --no-copy-ceiling" if separate_unpack else "")
    S, real, algo = algorithmic_bytes(wl, separate_unpack=separate_unpack)
    steps = steps_traced(n_f, wl, S, combine=True)
    update = update_kernel(separate_unpack=separate_unpack)
    per_dispatch = {k: algo[k] / (n_f[k] / steps) for k in algo if k in n_f and k != "copy_pieces_kernel<false>"}
    if separate_unpack:
        per_dispatch["copy_pieces_kernel<false>"] = algo["copy_pieces_kernel<false>"] / (
            n_f["copy_pieces_kernel<false>"] / steps)
    copy = "copy_pieces_kernel<false>"
    if separate_unpack:
        known = per_dispatch[copy] / 2               # unpack: as many bytes read as written
        source = "the unpack (2 bytes read and written per real shard element)"
    else:
        known = 2 * ceiling_elems(per_dispatch[update])  # the copy ceiling's copy: 2 bytes each way per element
        per_dispatch[copy] = 2 * known
        source = "the copy ceiling's plain copy of the same benchmark run"
    known_kib = known / 1024.0
    f_fetch = known_kib / fetch[copy]
    f_write = known_kib / write[copy]
    kernels = {}
    for k in fetch:
        if k not in per_dispatch and not k.startswith(("sqnorm_final", "sum_rows")):
            continue
        bytes_ = (fetch[k] * f_fetch + write.get(k, 0.0) * f_write) * 1024.0
        kernels[k] = {"fetch_kib_raw": round(fetch[k], 1), "write_kib_raw": round(write.get(k, 0.0), 1),
                      "dispatches": n_f[k], "traffic_bytes": int(bytes_),
                      "algorithmic_bytes": int(per_dispatch[k]) if k in per_dispatch else None,
                      "traffic_over_algorithmic": round(bytes_ / per_dispatch[k], 4) if k in per_dispatch else None}
    return {"workload": wl.name, "rank": wl.rank, "shard": S,
            "commands": [
                "cd /tmp && export TMPDIR=/tmp   # R: the repository root",
                f"timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $R/{fetch_dir} -o bench -- "
                f"python3 $R/bench.py --workload {wl.name} {mode} --no-cpu-baseline",
                f"timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $R/{write_dir} -o bench -- "
                f"python3 $R/bench.py --workload {wl.name} {mode} --no-cpu-baseline",
                f"cd $R && python bench.py --workload {wl.name} {mode} --pmc-summary {fetch_dir} {write_dir}"],
            "counter_units": "KiB per dispatch, averaged over dispatches",
            "kernel_code_sha256": source_hash(),
            "calibration": {"kernel": copy, "source": source, "known_read_kib": known_kib,
                            "known_write_kib": known_kib, "fetch_factor": round(f_fetch, 5),
                            "write_factor": round(f_write, 5)},
            "kernels": kernels}


def stats_summary(stats_dir, wl, steps, warmup, accum=1, separate_norm=False, flat=False, separate_unpack=False,
                  state_arrays=False):
    """Markdown table of the launches in a rocprofv3 kernel trace of this
    benchmark, with achieved bandwidth from each kernel's algorithmic bytes
    per launch (the step's bytes spread over that kernel's launches per
    step)."""
    import csv
    import glob

    S, real, algo = algorithmic_bytes(wl, accum, separate_norm, flat, separate_unpack, state_arrays)
    # every launch from the trace, in time order; the set-up launches of the
    # sum-of-squares kernels (the other ranks' partial sums) left out
    spans = {}
    for tpath in glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(tpath)):
            spans.setdefault(kernel_name(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    n_setup = setup_sqnorm_launches(wl)
    for k in spans:
        spans[k].sort()
        if k in SETUP_KERNELS:
            spans[k] = spans[k][n_setup:]
    rows = {k: {"Calls": len(iv), "AverageNs": sum(b - a for a, b in iv) / len(iv),
                "MinNs": min(b - a for a, b in iv), "MaxNs": max(b - a for a, b in iv)}
            for k, iv in spans.items() if iv}
    # busy time of each kernel: the union of its launches' intervals (launches
    # on two streams overlap, and each one's duration then includes time the
    # other stream shares)
    busy_ns = {}
    for k, iv in spans.items():
        total, end = 0, None
        for a, b in sorted(iv):
            if end is None or a > end:
                total += b - a
                end = b
            elif b > end:
                total += b - end
                end = b
        busy_ns[k] = total
    steps_run = steps_traced({k: int(r["Calls"]) for k, r in rows.items()}, wl, S,
                             combine=accum == 1 and not separate_norm and not flat)
    mode = ((f" --accum {accum}" if accum > 1 else "") + (" --separate-norm" if separate_norm else "") +
            (" --flat" if flat else "") + (" --separate-unpack" if separate_unpack else "") +
            (" --state-arrays" if state_arrays else ""))
    lines = [f"# Kernel durations: {wl.name}, rank {wl.rank} of N_d={wl.n_d} "
             f"(shard {S} elements{f', buckets of {wl.bucket}' if wl.bucket else ''})", "",
             "Commands (one MI355X; R is the repository root):", "",
             "    cd /tmp && export TMPDIR=/tmp",
             f"    timeout -k 10 600 rocprofv3 --kernel-trace --stats --output-format csv -d $R/{stats_dir} -o bench -- "
             f"python3 $R/bench.py --workload {wl.name} --steps {steps} --warmup {warmup}{mode} "
             f"--no-cpu-baseline --no-copy-ceiling",
             f"    cd $R && python bench.py --workload {wl.name} --steps {steps} --warmup {warmup}{mode} "
             f"--stats-summary {stats_dir}", "",
             f"kernels.hip code sha256 (comments and blank space aside): `{source_hash()}`", "",
             f"{steps_run:.0f} steps traced; bytes per launch = the step's algorithmic bytes for that "
             f"kernel divided by its launches per step. The {n_setup} launches of each sum-of-squares "
             f"kernel that set up the other ranks' partial sums come first and are left out.", "",
             "Busy us/step is the union of the kernel's launch intervals per step (the same as launches x avg "
             "when launches do not overlap); GB/s (busy) divides the step's bytes for the kernel by it.", "",
             "| kernel | calls | launches/step | avg us | min us | max us | algorithmic bytes/launch | "
             "GB/s at avg | % of 8 TB/s | busy us/step | GB/s (busy) | % (busy) |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for short, row in rows.items():
        if short not in algo and not short.startswith(("sqnorm_final", "sum_rows")):
            continue
        calls = int(row["Calls"])
        per_step = calls / steps_run
        avg = float(row["AverageNs"]) / 1e3
        b = algo[short] / per_step if short in algo else None
        gbps = f"{b / (avg * 1e-6) / 1e9:.1f}" if b else "-"
        pct = f"{100 * b / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS:.1f}" if b else "-"
        busy = busy_ns.get(short, 0) / 1e3 / steps_run if busy_ns else None
        step_b = algo.get(short)
        bgbps = f"{step_b / (busy * 1e-6) / 1e9:.1f}" if busy and step_b else "-"
        bpct = f"{100 * step_b / (busy * 1e-6) / 1e9 / HBM_PEAK_GBPS:.1f}" if busy and step_b else "-"
        lines.append(f"| {short} | {calls} | {per_step:.2f} | {avg:.1f} | {float(row['MinNs']) / 1e3:.1f} | "
                     f"{float(row['MaxNs']) / 1e3:.1f} | {int(b) if b else '-'} | {gbps} | {pct} | "
                     f"{f'{busy:.1f}' if busy else '-'} | {bgbps} | {bpct} |")
    return "\n".join(lines) + "\n"


def update_sweep(wl, reps=20):
    """The fused update (zero_adamw_step_unpack) over shard elements [0, n)
    for n from 1/16 of the shard to all of it, each timed over ``reps``
    launches with HIP events around each (median), after the breakdown-style
    warm-up; then a least-squares fit time = fixed + bytes / rate. The fixed
    part is what a launch costs beyond its bytes: the ramp while the first
    waves form the clip coefficient and issue their first loads, and the
    drain while the last waves finish."""
    import torch

    from fsdp_sharded_mixed_zero_amd import zero
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    rs = RankShard(wl)
    hp = rs.hparams(wl.step)
    S = rs.shard
    sizes = sorted({max(zero.ZERO_STATE_TILE, (S * k // 16) // zero.ZERO_STATE_TILE * zero.ZERO_STATE_TILE)
                    for k in (1, 2, 3, 4, 6, 8, 12, 16)})
    sizes[-1] = S

    def launch(n):
        zero.zero_adamw_step_unpack(rs.grad_shard, rs.state, rs.param_shard, S, 0, n, hp, rs.rank_sq, wl.n_d,
                                    rs.layout, rs.param_ptrs)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < BREAKDOWN_MIN_SECONDS:     # steady clocks
        for _ in range(10):
            launch(S)
        torch.cuda.synchronize()
    rows = []
    for n in sizes:
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in pairs:
            e0.record()
            launch(n)
            e1.record()
        torch.cuda.synchronize()
        us = median([e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs])
        nbytes = 28 * n + 2 * min(n, rs.real)
        rows.append((n, nbytes, us))
    xs = [b for _, b, _ in rows]
    ys = [t for _, _, t in rows]
    mx, my = sum(xs) / len(xs), sum(ys) / len(ys)
    slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    fixed = my - slope * mx
    lines = [f"# The fused update against its size: {wl.name}, rank {wl.rank} of N_d={wl.n_d}", "",
             "Command (one MI355X; R is the repository root):", "",
             f"    cd $R && python3 bench.py --workload {wl.name} --update-sweep", "",
             f"kernels.hip code sha256 (comments and blank space aside): `{source_hash()}`", "",
             f"zero_adamw_step_unpack over shard elements [0, n), {reps} launches each, HIP events around each "
             f"launch, median. Fit: time = {fixed:.1f} us + bytes / {1e-3 / slope:.1f} GB/s "
             f"({100 * 1e-3 / slope / HBM_PEAK_GBPS:.1f} % of 8 TB/s).", "",
             "| elements | algorithmic bytes | us | GB/s | % of 8 TB/s | fit us |", "|---|---|---|---|---|---|"]
    for n, b, us in rows:
        gbps = b / (us * 1e-6) / 1e9
        lines.append(f"| {n} | {b} | {us:.1f} | {gbps:.1f} | {100 * gbps / HBM_PEAK_GBPS:.1f} | "
                     f"{fixed + slope * b:.1f} |")
    return "\n".join(lines) + "\n"


def single_launch_calls(rs, fused):
    """Whether every update call of the step is one kernel launch: its range
    is at most ZERO_ADAMW_LAUNCH_ELEMS elements and, for the update with the
    unpack fused, touches at most ZERO_PIECES_PER_LAUNCH tensor pieces."""
    from fsdp_sharded_mixed_zero_amd import zero
    for b, n in rs.pieces():
        if n > zero.ZERO_ADAMW_LAUNCH_ELEMS:
            return False
        touched = sum(1 for _, _, dst, length in rs.segments if dst < b + n and dst + length > b)
        if fused and touched > zero.ZERO_PIECES_PER_LAUNCH:
            return False
    return True


def measured_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from the committed summary, or None
    when there is none or the kernels changed since it was taken."""
    import json as _json
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    data = _json.load(open(path))
    if data.get("kernel_code_sha256") != source_hash():
        return None
    return data["kernels"].get(kernel, {}).get("traffic_bytes")


# --------------------------------------------------------------- oracle leg

ORACLE_CHUNK = 1 << 22


def _oracle_setup(wl):
    """The rank's layout, hyperparameters, the other ranks' expected sum of
    squares, and the number of 2^22-element chunks of the shard."""
    from oracle import step as O
    from oracle.layout import build_layout

    lay = build_layout(wl.sizes, wl.n_d, wl.rank, wl.align)
    hp = O.AdamWHParams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                        weight_decay=wl.weight_decay, max_norm=wl.max_norm)
    others = sum(max(0, min(lay.shard, lay.psi - r * lay.shard)) for r in range(wl.n_d)
                 if r != wl.rank) * wl.grad_sq_mean()
    return lay, hp, others, max(1, lay.shard // ORACLE_CHUNK)


def _oracle_sample(wl, lay, k, n_chunks):
    """Chunk k of the shard (spread across it) as its own small layout over
    windows of the tensors it covers, with its gradients and state."""
    from fsdp_sharded_mixed_zero_amd import synth
    from oracle.layout import Layout, Segment

    b = (k * 7919 % n_chunks) * ORACLE_CHUNK
    c = min(ORACLE_CHUNK, lay.shard - b)
    segs, wins = [], []
    for s in lay.segments:
        lo, hi = max(s.dst_off, b), min(s.dst_off + s.length, b + c)
        if lo < hi:
            segs.append(Segment(len(wins), 0, lo - b, hi - lo))
            wins.append(hi - lo)
    sub = Layout(tuple(wins), 1, 0, 1, (), lay.psi, c, c, 0, tuple(segs), c, c)
    grads = [synth.to_bf16_bits(synth.host_grad_f32(n, wl, wl.step, 1000 + i)) for i, n in enumerate(wins)]
    real = max(0, min(c, lay.real_elems - b))
    return b, c, sub, grads, synth.host_shard_state(wl, b, c, real, piece=k)


def _oracle_run(wl, hp, others, sample):
    """One oracle step over a sample; returns the seconds it took."""
    import numpy as np

    from oracle import step as O

    _, _, sub, grads, (master, m, v) = sample
    params = [np.zeros(n, np.uint16) for n in sub.sizes]
    t0 = time.perf_counter()
    g = O.pack(sub, grads)
    G = O.global_sqnorm([O.sqnorm(g), others])
    coef = O.clip_coef(G, hp.max_norm, hp.clip_eps)
    _, _, _, bits = O.adamw_step(g, master, m, v, wl.step, hp, coef)
    O.unpack(sub, bits, params)
    return time.perf_counter() - t0


def cpu_baseline(wl, seconds):
    """The oracle's step (pack, sum of squares, clip, AdamW, unpack) on chunks
    of 2^22 shard elements taken from across the rank's shard, on one host
    thread, repeated over up to 8 distinct chunks until about ``seconds`` of
    oracle time has been spent (input generation is not timed)."""
    from threadpoolctl import threadpool_limits

    lay, hp, others, n_chunks = _oracle_setup(wl)
    samples = [_oracle_sample(wl, lay, k, n_chunks) for k in range(min(8, n_chunks))]
    done = 0
    spent = 0.0
    runs = 0
    with threadpool_limits(limits=1):
        _oracle_run(wl, hp, others, samples[0])    # untimed: the first call pays start-up costs
        while spent < seconds:
            sample = samples[runs % len(samples)]
            spent += _oracle_run(wl, hp, others, sample)
            done += sample[1]
            runs += 1
    return {"value": done / spent, "unit": "params/s", "cores": 1, "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": (f"{runs} runs over {len(samples)} distinct chunks of {ORACLE_CHUNK} elements of the "
                       f"{wl.name} rank-{wl.rank} shard ({done} elements, {spent:.1f} s of oracle time), "
                       f"numpy float64 oracle on one host thread")}


def _oracle_worker(name, k, seconds, barrier, results):
    """One process of the parallel baseline: its own chunk, one thread, timed
    from a barrier that all workers pass together."""
    from threadpoolctl import threadpool_limits

    from fsdp_sharded_mixed_zero_amd import synth

    wl = synth.WORKLOADS[name]
    lay, hp, others, n_chunks = _oracle_setup(wl)
    sample = _oracle_sample(wl, lay, k % n_chunks, n_chunks)
    done, spent = 0, 0.0
    with threadpool_limits(limits=1):
        _oracle_run(wl, hp, others, sample)
        barrier.wait()
        while spent < seconds:
            spent += _oracle_run(wl, hp, others, sample)
            done += sample[1]
    results.put((done, spent))


def cpu_baseline_parallel(wl, seconds, workers):
    """The same oracle step in ``workers`` single-threaded processes at once,
    each on its own chunk (the bucket-parallel form: chunks are independent
    once the clip coefficient is known). Throughput = the sum of the workers'
    rates over the common timed window."""
    import multiprocessing as mp

    ctx = mp.get_context("spawn")          # fresh interpreters: nothing inherited from the GPU process
    barrier = ctx.Barrier(workers)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(wl.name, k, seconds, barrier, results))
             for k in range(workers)]
    for pr in procs:
        pr.start()
    out = [results.get(timeout=600) for _ in procs]
    for pr in procs:
        pr.join()
    rate = sum(d / s for d, s in out)
    return {"value": rate, "unit": "params/s", "cores": workers, "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": (f"{workers} processes, one host thread each, each on its own chunk of {ORACLE_CHUNK} "
                       f"elements of the {wl.name} rank-{wl.rank} shard for about {seconds:.0f} s "
                       f"({sum(d for d, _ in out)} elements in all)")}


def copy_ceiling(torch, n, reps=20):
    """The streaming ceiling the kernels are compared with: a plain copy of
    ``n`` bf16 elements per launch (4n bytes, half read, half written), timed
    with HIP events around each launch like the kernels. The copy is the library's
    unpack over a one-tensor layout (one piece: the plain copy kernel);
    torch's device-to-device ``copy_`` of the same bytes is listed beside it."""
    from fsdp_sharded_mixed_zero_amd import zero

    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")   # the copy moves 4 bytes per element
    dst = torch.empty_like(src)
    lay = zero.zero_layout([n], 1, 0, 1)
    ptrs = zero.pointer_array([dst])
    stream = torch.cuda.current_stream().cuda_stream

    def per_launch(fn):
        for _ in range(3):
            fn()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(reps)]
        for e0, e1 in pairs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in pairs) * 1e-3 / reps

    sec = per_launch(lambda: zero.zero_unpack_params(lay, src, ptrs, 0, n, stream))
    ok = torch.equal(dst.view(torch.int16), src.view(torch.int16))
    sec_torch = per_launch(lambda: dst.copy_(src))
    gbps, gbps_torch = 4 * n / sec / 1e9, 4 * n / sec_torch / 1e9
    del src, dst, lay
    torch.cuda.empty_cache()
    return {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_copy": 4 * n,
            "copied_correctly": ok,
            "how": f"zero_unpack_params over a one-tensor layout of {n} bf16 elements, mean of {reps} "
                   f"launches with events around each",
            "torch_copy_GBps": round(gbps_torch, 1)}


# ------------------------------------------------------------------ GPU leg

def host_copy_ceiling(nbytes, threads, reps=5):
    """Host memory streaming ceiling for the offloaded update: ``threads``
    threads copying disjoint slices of one buffer into another (numpy
    releases the interpreter lock while it copies), ``nbytes`` moved per
    pass (half read, half written)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    n = max(1, nbytes // 2)
    src = np.ones(n, np.uint8)
    dst = np.zeros(n, np.uint8)
    cuts = [n * i // threads for i in range(threads + 1)]

    def part(i):
        np.copyto(dst[cuts[i]:cuts[i + 1]], src[cuts[i]:cuts[i + 1]])

    with ThreadPoolExecutor(threads) as pool:
        list(pool.map(part, range(threads)))          # first touch of the pages
        best = float("inf")
        for _ in range(reps):
            t0 = time.perf_counter()
            list(pool.map(part, range(threads)))
            best = min(best, time.perf_counter() - t0)
    return {"GBps": round(2 * n / best / 1e9, 1), "threads": threads, "bytes_per_pass": 2 * n,
            "how": f"{threads} threads copying disjoint slices of a {n}-byte buffer, best of {reps}"}


def offload_main(args, wl):
    """The ZeRO-Offload step: GPU pack + norm, PCIe copies, AdamW on the host
    cores, GPU unpack. Reports the step, the host update and the PCIe rate."""
    import torch

    from fsdp_sharded_mixed_zero_amd.rank import OffloadRank

    rs = OffloadRank(wl, bucket=args.offload_bucket)
    torch.cuda.synchronize()
    t = wl.step
    for _ in range(args.warmup):
        rs.step(t)
        t += 1
    torch.cuda.synchronize()
    rs.host_seconds = 0.0
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rs.step(t)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    S = rs.shard
    host_s = rs.host_seconds / args.steps
    out = {
        "metric": "ZeRO-Offload step: shard params/sec with AdamW on the host cores",
        "value": S / (ms * 1e-3), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name} rank {rs.rank} of N_d={wl.n_d}, optimizer state offloaded to "
                               f"host memory", "shard_params": S, "buckets": len(rs.transfer_pieces()),
                   "staging_slots": len(rs.stage_g), "host_threads": rs.threads or len(os.sched_getaffinity(0))},
        "host_adamw_ms_per_step": host_s * 1e3,
        "host_adamw_params_per_s": S / host_s,
        "host_adamw_GBps": 28 * S / host_s / 1e9,
        "pcie_GBps_over_step": rs.pcie_bytes_per_step() / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "host", "achieved": round(28 * S / host_s / 1e9, 1), "peak": None,
                     "unit": "GB/s", "frac": None, "traffic": None},
    }
    threads = rs.threads or len(os.sched_getaffinity(0))
    del rs
    host = host_copy_ceiling(min(28 * S, 8 << 30), threads)
    out["host_copy_ceiling"] = host
    out["roofline"].update(peak=host["GBps"], frac=round(out["roofline"]["achieved"] / host["GBps"], 4),
                           peak_note="the host copy ceiling measured here, not a published figure")
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.pmc_summary:
        from fsdp_sharded_mixed_zero_amd import synth
        if args.accum > 1 or args.separate_norm or args.flat:
            sys.exit("counters are summarised for the default mode or --separate-unpack")
        print(json.dumps(pmc_summary(*args.pmc_summary, synth.WORKLOADS[args.workload], args.steps,
                                     args.warmup, args.separate_unpack), indent=1))
        return
    if args.stats_summary:
        from fsdp_sharded_mixed_zero_amd import synth
        print(stats_summary(args.stats_summary, synth.WORKLOADS[args.workload], args.steps, args.warmup,
                            args.accum, args.separate_norm, args.flat, args.separate_unpack, args.state_arrays),
              end="")
        return
    if args.update_sweep:
        from fsdp_sharded_mixed_zero_amd import synth
        import torch
        torch.cuda.set_device(0)
        print(update_sweep(synth.WORKLOADS[args.workload]), end="")
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's shard on one GPU; it does not run on more than one GPU "
              "(the collectives around the step are not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    from fsdp_sharded_mixed_zero_amd import synth, zero
    from fsdp_sharded_mixed_zero_amd.rank import RankShard

    zero.library()                       # fail loudly if the HIP library is missing
    wl = synth.WORKLOADS[args.workload]
    # the oracle legs run first, before this process touches the GPU, so the
    # parallel leg starts its worker processes from a process with no GPU state
    baselines = {}
    if not args.no_cpu_baseline and not args.offload:
        baselines["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        workers = min(16, len(os.sched_getaffinity(0)))
        if workers > 1:
            baselines["cpu_baseline_parallel"] = cpu_baseline_parallel(wl, args.cpu_seconds / 3, workers)
    torch.cuda.set_device(0)
    if args.offload:
        return offload_main(args, wl)
    rs = RankShard(wl, fused_norm=not args.separate_norm, accum_steps=args.accum, flat=args.flat,
                   fused_unpack=not args.separate_unpack, state_arrays=args.state_arrays)
    torch.cuda.synchronize()

    # Per-phase breakdown first, outside the timed region: events around every
    # phase of each step, for at least BREAKDOWN_MIN_STEPS steps and
    # BREAKDOWN_MIN_SECONDS of wall time. Besides the per-kernel table and the
    # roofline (the median update launch), this keeps the GPU busy long
    # enough to reach its steady clocks before the timed steps: an idle GPU
    # starts a short run ~10% slower.
    t = wl.step
    n_p = len(rs.pieces())
    per_step = 2 * (n_p * (2 if args.separate_norm else 1) + 2 * n_p + (3 * args.accum + 1) * n_p)
    phase_timing = {}
    breakdown_steps = 0
    t0 = time.perf_counter()
    while breakdown_steps < BREAKDOWN_MIN_STEPS or time.perf_counter() - t0 < BREAKDOWN_MIN_SECONDS:
        batch = 10
        events = iter([torch.cuda.Event(enable_timing=True) for _ in range(per_step * batch)])
        for _ in range(batch):
            rs.step(t, timing=phase_timing, events=events)
            t += 1
        breakdown_steps += batch
        torch.cuda.synchronize()

    # the timed region: W warm-up steps, then exactly K steps, nothing else
    for _ in range(args.warmup):
        rs.step(t)
        t += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        rs.step(t)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_per_step = wall * 1e3 / args.steps
    S = rs.shard
    algo = rs.bytes_per_step()
    kernels = {}
    for phase, evs in phase_timing.items():
        launches = len(evs) // breakdown_steps
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        per_step_ms = median([sum(ms[k * launches:(k + 1) * launches]) for k in range(breakdown_steps)])
        gbps = algo[phase] / (per_step_ms * 1e-3) / 1e9
        kernels[phase] = {"us_per_step": round(per_step_ms * 1e3, 2), "launches_per_step": launches,
                          "algorithmic_bytes": algo[phase], "GBps": round(gbps, 1),
                          "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    # each event pair spans one update call: one kernel launch unless the
    # call's range needs several (then the pair spans them all, back to back)
    call_times = sorted(e0.elapsed_time(e1) for e0, e1 in phase_timing["adamw"])
    call_ms = median(call_times)
    calls = len(call_times) / breakdown_steps
    call_elems = S / calls
    call_bytes = algo["adamw"] / calls
    achieved = call_bytes / (call_ms * 1e-3) / 1e9
    single = single_launch_calls(rs, rs.fused_unpack)
    bucketed, n_streams = rs.bucketed, rs.n_streams
    step_bytes = sum(algo.values())
    default_kernel = rs.bucket <= 0 and args.accum == 1 and not args.flat
    traffic = (measured_traffic(wl.name, update_kernel(args.accum, args.separate_unpack, args.flat,
                                                       args.state_arrays))
               if default_kernel else None)

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
        "config": {"workload": f"{wl.name} rank {rs.rank} of N_d={wl.n_d}: one rank's shard, " + (
                               "ZeRO-1 flat buffers: sum of squares -> clip+AdamW+bf16 cast on the rank's slice"
                               if args.flat else
                               "pack + sum of squares -> clip+AdamW+bf16 cast over three state arrays (master, "
                               "m, v) -> unpack" if args.state_arrays else
                               "pack -> sum of squares -> clip+AdamW+bf16 cast -> unpack" if args.separate_unpack
                               else "pack + sum of squares -> clip+AdamW+bf16 cast with the unpack fused"),
                   "shard_params": S, "n_d": wl.n_d, "rank": rs.rank, "tensors": len(wl.sizes),
                   "segments_in_shard": len(rs.segments), "adamw_step": wl.step,
                   "bucket": rs.bucket, "streams": rs.n_streams,
                   "norm": "separate" if args.separate_norm or args.flat else "fused into pack",
                   "unpack": ("none (flat buffers)" if args.flat else
                              "separate" if args.separate_unpack or args.state_arrays else "fused into AdamW"),
                   "state": "three arrays" if args.state_arrays else "tiled (master|m|v in 8192-element tiles)",
                   "fp32_grad_accumulation_micro_batches": args.accum if args.accum > 1 else None},
        "adamw_params_per_s": call_elems / (call_ms * 1e-3),
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "kernels_note": f"median per-step time of each phase over {breakdown_steps} steps with events around "
                        f"every phase, run before the warm-up (outside the timed region)",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
    }
    unit, units = ("phase", "phases") if bucketed else ("launch", "launches") if single else ("call", "calls")
    out["roofline"].update({
        f"algorithmic_bytes_per_{unit}": int(call_bytes), f"timed_{units}": len(call_times),
        "statistic": f"median {unit} duration",
        f"us_per_{unit}": {"median": round(call_ms * 1e3, 2),
                           "p10": round(call_times[len(call_times) // 10] * 1e3, 2),
                           "p90": round(call_times[(9 * len(call_times)) // 10] * 1e3, 2)},
        "events": f"a HIP event pair on the update's stream around each AdamW {unit} of the "
                  f"{breakdown_steps} breakdown steps"})
    if bucketed:
        out["roofline"]["note"] = (f"the update phase: one launch per bucket, the buckets dealt out to {n_streams} "
                                   f"streams; achieved is the phase's bytes over its time")
    elif not single:
        out["roofline"]["note"] = ("each update call runs as several kernel launches back to back (a range longer "
                                   "than ZERO_ADAMW_LAUNCH_ELEMS elements or touching more than "
                                   "ZERO_PIECES_PER_LAUNCH tensor pieces): achieved is per call")
    del rs
    torch.cuda.empty_cache()
    if not args.no_copy_ceiling:
        out["copy_ceiling"] = copy_ceiling(torch, ceiling_elems(call_bytes))
        if "pack_sqnorm" in algo and not bucketed:
            # the same copy over the pack's bytes: the ceiling of pack + sum of squares
            out["copy_ceiling_pack_size"] = copy_ceiling(torch, ceiling_elems(algo["pack_sqnorm"]))
    out.update(baselines)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
